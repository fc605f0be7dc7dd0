"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.

* The decode step of the benchmark: one grouped launch of the Q4_0 SwiGLU FFN
  GEMVs (gate and up 4864x896, down 896x4864, batch 1), each quantising its
  own activation inside the kernel; every output against the oracle (all
  rows), the written Q8_0 blocks bit-exact.
* Every GEMV of the per-matrix suite (B <= 16, activations staged by
  quantize_act_q8_0): all outputs of matrices up to 8192 rows, and a seeded
  sample of rows (plus the first and last rows and rows on 16-row tile
  edges) of larger ones, against the oracle computed on exactly those rows.
* Every GEMM of the suite (M = 512 or 2048): a sample of tokens x rows
  against the oracle, and each sampled token's full output row bit-identical
  to the batch-1 GEMV of that token (a property that holds at any size).

Outputs are checked bitwise against the oracle's replay of the documented f32
order and within 1e-4 * sum|w^ x^| of its f64 result.
"""
import numpy as np
import pytest

import oracle
import synth
from checks import assert_bitwise, assert_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gguf_quantized_matvec_amd as g
    g.lib()  # raises if the library is missing: no fallback
    return g


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample_rows(N, seed, n=384):
    """Rows checked at full size: all of them up to 8192, else the first and
    last rows, both sides of a few 16- and 128-row tile edges, and a seeded
    uniform sample."""
    if N <= 8192:
        return np.arange(N)
    rng = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 15, 16, 127, 128, N // 2, N - 17, N - 16, N - 2, N - 1]
    return np.unique(np.concatenate([edges, rng.choice(N, n, replace=False)]))


def rows_of(fmt, blob, N, K, rows):
    R = synth.row_bytes(fmt, K)
    return np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)


def check_against_oracle(fmt, blob, N, K, xq_pub, B, y, rows, what):
    """y: GPU output [B, N] (host); rows: the weight rows to check."""
    sub = rows_of(fmt, blob, N, K, rows)
    yc = oracle.matmul_canon_f32(fmt, sub, len(rows), K, xq_pub, B)
    y64, A = oracle.matmul_f64(fmt, sub, len(rows), K, xq_pub, B)
    got = np.ascontiguousarray(y[:, rows])
    assert_tol(got, y64, A, what=f"{what} vs f64")
    assert_bitwise(got, yc, f"{what} vs f32 order")


_BLOBS = {}


def workload_matrix(wl, mi):
    """The suite's seeded weight blob of matrix mi of workload wl (cached)."""
    key = (wl, mi)
    if key not in _BLOBS:
        _BLOBS.clear()
        ci = list(synth.WORKLOADS).index(wl)
        fmt, N, K, ds = synth.WORKLOADS[wl]["mats"][mi]
        blob, _ = synth.weights(fmt, N, K, synth.seed_for(ci, mi), dscale=ds)
        _BLOBS[key] = blob
    return _BLOBS[key]


def _cases(small):
    out = []
    for wl, spec in synth.WORKLOADS.items():
        for mi, (fmt, N, K, _) in enumerate(spec["mats"]):
            for B in spec["batches"]:
                if (B <= 16) == small:
                    tag = f"B{B}" if small else f"M{B}"
                    out.append(pytest.param(wl, mi, B, id=f"{wl}-{synth.NAMES[fmt]}-{N}x{K}-{tag}"))
    return out


def test_headline_ffn_step(g):
    """The benchmark's step: gate, up and down as one grouped launch with the
    quantisation fused; gate and down also write their Q8_0 blocks."""
    fmt = synth.Q4_0
    shapes = [("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864)]
    blobs = {n: synth.weights(fmt, N, K, synth.seed_for(1, i), dscale=0.02)[0]
             for i, (n, N, K) in enumerate(shapes)}
    x1 = synth.activations(1, 896, synth.act_seed_for(1, 1))
    x2 = synth.activations(1, 4864, synth.act_seed_for(1, 1) + 1)
    w = {n: dev(b) for n, b in blobs.items()}
    X1, X2 = dev(x1), dev(x2)
    q1, q2 = g.act_buffer(1, 896), g.act_buffer(1, 4864)
    ys = g.matvec_group(fmt, [dict(w=w["gate"], N=4864, K=896, x=X1, xq=q1),
                              dict(w=w["up"], N=4864, K=896, x=X1),
                              dict(w=w["down"], N=896, K=4864, x=X2, xq=q2)])
    xq1, xq2 = oracle.quantize_act(x1), oracle.quantize_act(x2)
    assert_bitwise(host(q1)[:xq1.size], xq1, "gate Q8_0 blocks")
    assert_bitwise(host(q2)[:xq2.size], xq2, "down Q8_0 blocks")
    for (n, N, K), y in zip(shapes, ys):
        xq = xq1 if K == 896 else xq2
        check_against_oracle(fmt, blobs[n], N, K, xq, 1, host(y), np.arange(N), n)


@pytest.mark.parametrize("wl,mi,B", _cases(small=True))
def test_suite_gemv_full_size(g, wl, mi, B):
    fmt, N, K, _ = synth.WORKLOADS[wl]["mats"][mi]
    ci = list(synth.WORKLOADS).index(wl)
    blob = workload_matrix(wl, mi)
    x = synth.activations(B, K, synth.act_seed_for(ci, B))
    xq = g.quantize(dev(x))
    y = host(g.matvec(fmt, dev(blob), N, K, xq=xq, B=B))
    xq_pub = oracle.quantize_act(x)
    assert_bitwise(host(xq)[:xq_pub.size], xq_pub, "Q8_0 blocks")
    rows = sample_rows(N, 7 + 13 * ci + mi)
    check_against_oracle(fmt, blob, N, K, xq_pub, B, y, rows, f"{wl} B={B}")


@pytest.mark.parametrize("wl,mi,M", _cases(small=False))
def test_suite_gemm_full_size(g, wl, mi, M):
    fmt, N, K, _ = synth.WORKLOADS[wl]["mats"][mi]
    ci = list(synth.WORKLOADS).index(wl)
    blob = workload_matrix(wl, mi)
    x = synth.activations(M, K, synth.act_seed_for(ci, M))
    w = dev(blob)
    xq = g.quantize(dev(x))
    y = host(g.matmul(fmt, w, N, K, xq=xq, M=M))
    rng = np.random.Generator(np.random.PCG64(31 + ci))
    toks = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 12, replace=False)]))
    rows = sample_rows(N, 11 + 13 * ci + mi, n=256)
    xq_pub = oracle.quantize_act(x[toks])
    check_against_oracle(fmt, blob, N, K, xq_pub, len(toks), y[toks], rows, f"{wl} M={M}")
    for t in toks[:6]:
        y1 = host(g.matvec(fmt, w, N, K, x=dev(x[t:t + 1])))
        assert_bitwise(y[t:t + 1], y1, f"{wl} M={M} token {t} vs batch-1 GEMV")
