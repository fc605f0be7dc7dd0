"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.

* The benchmark's headline step (one 8B-class decoder layer at batch 1 and
  16: q/k/v grouped, o, gate/up with the SwiGLU, down on h) and the pages'
  Qwen2.5-0.5B FFN step, in the launch configuration the benchmark times;
  outputs against the oracle chain, h and the Q8_0 blocks bit-exact.
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


# The benchmark's headline step: one 8B-class decoder layer's projections.
LAYER = [("q", synth.Q4_K, 4096, 4096), ("k", synth.Q4_K, 1024, 4096),
         ("v", synth.Q4_K, 1024, 4096), ("o", synth.Q4_K, 4096, 4096),
         ("gate", synth.Q4_K, 14336, 4096), ("up", synth.Q4_K, 14336, 4096),
         ("down", synth.Q6_K, 4096, 14336)]


@pytest.mark.parametrize("B", [1, 16])
def test_headline_layer_step(g, B):
    """The benchmark's step, in its launch configuration: q/k/v as one grouped
    launch (x fused at B <= 4, quantised once otherwise), o, gate/up with the
    SwiGLU, down on h; every stage's outputs on sampled rows against the
    oracle chain (canonical-f32 gate and up -> SwiGLU -> Q8_0 of h -> down),
    h and the down GEMV's Q8_0 blocks bit-exact."""
    blobs = {n: synth.weights(f, N, K, synth.seed_for(4, 10 + i), dscale=0.02)[0]
             for i, (n, f, N, K) in enumerate(LAYER)}
    w = {n: dev(b) for n, b in blobs.items()}
    xs = [synth.activations(B, 4096, synth.act_seed_for(4, B) + j) for j in range(3)]
    xa, xo, xc = (dev(x) for x in xs)
    print(f"layer step B={B}", flush=True)
    qa = g.act_buffer(B, 4096)
    if B <= 4:
        items = [dict(w=w["q"], N=4096, K=4096, x=xa, xq=qa), dict(w=w["k"], N=1024, K=4096, x=xa),
                 dict(w=w["v"], N=1024, K=4096, x=xa)]
    else:
        g.quantize(xa, xq=qa)
        items = [dict(w=w[n], N=N, K=4096, xq=qa, B=B) for n, N in (("q", 4096), ("k", 1024),
                                                                      ("v", 1024))]
    yq, yk, yv = g.matvec_group(synth.Q4_K, items)
    yo = g.matvec(synth.Q4_K, w["o"], 4096, 4096, x=xo)
    h = g.gateup_swiglu(synth.Q4_K, w["gate"], w["up"], 14336, 4096, x=xc)
    qd = g.act_buffer(B, 14336)
    yd = g.matvec(synth.Q6_K, w["down"], 4096, 14336, x=h, xq=qd)
    xq = [oracle.quantize_act(x) for x in xs]
    for n, y, xqi in (("q", yq, xq[0]), ("k", yk, xq[0]), ("v", yv, xq[0]), ("o", yo, xq[1])):
        f, N, K = next((f, N, K) for m, f, N, K in LAYER if m == n)
        check_against_oracle(f, blobs[n], N, K, xqi, B, host(y), sample_rows(N, 50 + N), n)
    # h on sampled rows: oracle SwiGLU of the oracle's gate and up rows
    rows = sample_rows(14336, 61)
    gt = oracle.matmul_canon_f32(synth.Q4_K, rows_of(synth.Q4_K, blobs["gate"], 14336, 4096, rows),
                                 len(rows), 4096, xq[2], B)
    up = oracle.matmul_canon_f32(synth.Q4_K, rows_of(synth.Q4_K, blobs["up"], 14336, 4096, rows),
                                 len(rows), 4096, xq[2], B)
    hh = host(h)
    assert_bitwise(np.ascontiguousarray(hh[:, rows]), oracle.swiglu(gt, up), "h")
    # down: its Q8_0 blocks of the GPU's h bit-exact, outputs against the oracle
    xq_h = oracle.quantize_act(hh)
    assert_bitwise(host(qd)[: xq_h.size], xq_h, "Q8_0 of h")
    check_against_oracle(synth.Q6_K, blobs["down"], 4096, 14336, xq_h, B, host(yd),
                         sample_rows(4096, 62), "down")


def test_qwen_ffn_step(g):
    """The pages' Qwen2.5-0.5B FFN at batch 1 as the benchmark runs it:
    gate/up (Q4_0 4864x896) with the SwiGLU, then down (896x4864) on h."""
    fmt = synth.Q4_0
    shapes = [("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864)]
    blobs = {n: synth.weights(fmt, N, K, synth.seed_for(1, i), dscale=0.02)[0]
             for i, (n, N, K) in enumerate(shapes)}
    x1 = synth.activations(1, 896, synth.act_seed_for(1, 1))
    w = {n: dev(b) for n, b in blobs.items()}
    h = g.gateup_swiglu(fmt, w["gate"], w["up"], 4864, 896, x=dev(x1))
    q2 = g.act_buffer(1, 4864)
    y = g.matvec(fmt, w["down"], 896, 4864, x=h, xq=q2)
    xq1 = oracle.quantize_act(x1)
    h_o = oracle.swiglu(oracle.matmul_canon_f32(fmt, blobs["gate"], 4864, 896, xq1, 1),
                        oracle.matmul_canon_f32(fmt, blobs["up"], 4864, 896, xq1, 1))
    assert_bitwise(host(h), h_o, "h")
    xq2 = oracle.quantize_act(h_o)
    assert_bitwise(host(q2)[: xq2.size], xq2, "Q8_0 of h")
    check_against_oracle(fmt, blobs["down"], 896, 4864, xq2, 1, host(y), np.arange(896), "down")


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
