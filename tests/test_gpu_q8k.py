"""GPU parity of the K-quant x Q8_K path (Q4_K / Q6_K weights, activations
quantised per 256 elements with an f32 scale) against the CPU oracle:

* the Q8_K blocks of the quantiser: bit-exact (zero, tiny and normal blocks,
  16- and 4-byte aligned x);
* the superblock partials of every kernel path (the lane-per-chunk GEMV for
  B <= 4, the batched int8-MFMA kernel for B = 5..16, the int8-MFMA GEMM
  with 32- and 64-row tiles for more rows): bit-exact, including superblock
  partials above 2^24;
* y: bit-identical to the oracle's replay of the Q8_K f32 order and within
  1e-4 * sum|w^ x^| of its f64 result; GEMM rows bit-identical to the
  batch-1 GEMV; at the 8B-class sizes (M = 2048) on sampled tokens and rows.
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
    g.lib()
    return g


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def pubk(xq, rows, K):
    return host(xq)[: rows * (K // 256) * 292]


@pytest.mark.parametrize("rows,K", [(1, 256), (3, 1024), (16, 4096), (40, 512), (7, 14336)])
def test_quantize_q8k_bit_exact(g, rows, K):
    x = synth.activations(rows, K, 2000 + K) * np.float32(3.0)
    x[0, :256] = 0.0                        # an all-zero block
    if K >= 768:
        x[-1, 256:512] *= np.float32(1e-40)  # 1/d not finite: zero codes
        x[-1, 512:768] *= np.float32(1e-30)  # tiny but quantised normally
    want = oracle.quantize_act_q8k(x)
    print(f"quantize q8k rows={rows} K={K}", flush=True)
    assert_bitwise(pubk(g.quantize_q8k(dev(x)), rows, K), want, "Q8_K blocks")
    # only 4-byte aligned x
    buf = torch.zeros(rows * K + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev(x).reshape(-1)
    assert_bitwise(pubk(g.quantize_q8k(buf[1:].view(rows, K)), rows, K), want, "Q8_K, x unaligned")


FMTS = [synth.Q4_K, synth.Q6_K]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(37, 256), (130, 1024), (300, 4096 + 256)])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 16, 33, 70])
def test_partials_q8k_every_path(g, fmt, N, K, M):
    blob, _ = synth.weights(fmt, N, K, 2100 + N + M, s_range=(-128, 127))
    x = synth.activations(M, K, 2101 + K)
    print(f"partials q8k fmt={fmt} N={N} K={K} M={M}", flush=True)
    xq = g.quantize_q8k(dev(x))
    P = host(g.partials_q8k(fmt, dev(blob), N, K, xq, M))
    assert_bitwise(P, oracle.partials_q8k(fmt, blob, N, K, oracle.quantize_act_q8k(x), M),
                   "q8k partials")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 3, 9, 40])
def test_partials_q8k_above_2_24(g, fmt, M):
    """Large scales, codes and activations: superblock partials beyond 2^24
    (Q4_K's P up to 8*63*15*32*127), where (float)P rounds."""
    N, K = 64, 1024
    f = synth.draw_fields(fmt, N, K, 2200, s_range=(-128, 127))
    if fmt == synth.Q4_K:
        f["sc"] = np.maximum(f["sc"], 56)
        f["q"] = np.maximum(f["q"], 12)
    else:
        f["s"] = np.where(np.abs(f["s"]) < 100, np.int8(-128), f["s"]).astype(np.int8)
        f["q"] = np.minimum(f["q"], 3)
    blob = synth.encode(f)
    x = (np.abs(synth.activations(M, K, 2201)) * 0.2 + 4).astype(np.float32)
    xq_o = oracle.quantize_act_q8k(x)
    P_o = oracle.partials_q8k(fmt, blob, N, K, xq_o, M)
    assert np.abs(P_o[..., 0] if fmt == synth.Q4_K else P_o).max() > 2 ** 24
    print(f"q8k large partials fmt={fmt} M={M}", flush=True)
    xd = dev(x)
    P = host(g.partials_q8k(fmt, dev(blob), N, K, g.quantize_q8k(xd), M))
    assert_bitwise(P, P_o, "q8k partials > 2^24")
    y = host(g.matmul_q8k(fmt, dev(blob), N, K, x=xd))
    assert_bitwise(y, oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq_o, M), "y, (float)P rounding")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(45, 1024, 1), (96, 4352, 3), (33, 768, 4), (129, 1024, 7),
                                   (250, 2048, 16), (130, 512, 65), (70, 4096, 200)])
def test_q8k_against_oracle(g, fmt, N, K, M):
    blob, _ = synth.weights(fmt, N, K, 2300 + N, s_range=(-128, 127))
    x = synth.activations(M, K, 2301 + M)
    print(f"q8k y fmt={fmt} N={N} K={K} M={M}", flush=True)
    y = host(g.matmul_q8k(fmt, dev(blob), N, K, x=dev(x)))
    xq = oracle.quantize_act_q8k(x)
    y64, A = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, M)
    assert_tol(y, y64, A, what="q8k vs f64")
    assert_bitwise(y, oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq, M), "q8k f32 order")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [5, 16, 64, 130])
def test_q8k_rows_equal_batch1(g, fmt, M):
    N, K = 200, 2048
    blob, _ = synth.weights(fmt, N, K, 2400, s_range=(-128, 127))
    x = synth.activations(M, K, 2401)
    w = dev(blob)
    y = host(g.matmul_q8k(fmt, w, N, K, x=dev(x)))
    for t in sorted({0, 1, M // 2, M - 1}):
        y1 = host(g.matmul_q8k(fmt, w, N, K, x=dev(x[t:t + 1])))
        assert_bitwise(y[t:t + 1], y1, f"row {t} of M={M} vs batch 1")


@pytest.mark.parametrize("fmt,N,K", [(synth.Q4_K, 14336, 4096), (synth.Q6_K, 4096, 14336),
                                     (synth.Q4_K, 1024, 4096)])
def test_q8k_gemm_8b_class_full_size(g, fmt, N, K):
    """The 8B-class shapes at 2048 tokens, in the benchmark's launch
    configuration: sampled tokens x rows against the oracle, sampled tokens'
    full rows against the batch-1 GEMV."""
    M = 2048
    blob, _ = synth.weights(fmt, N, K, synth.seed_for(4, {4096: 0, 1024: 1, 14336: 2}[N]
                                                      if fmt == synth.Q4_K else 3), dscale=0.02)
    x = synth.activations(M, K, synth.act_seed_for(4, M))
    w, xd = dev(blob), dev(x)
    print(f"q8k full size fmt={fmt} N={N} K={K}", flush=True)
    y = host(g.matmul_q8k(fmt, w, N, K, x=xd))
    rng = np.random.Generator(np.random.PCG64(2500 + N))
    toks = np.unique(np.concatenate([[0, 63, 64, M - 1], rng.choice(M, 8, replace=False)]))
    rows = np.unique(np.concatenate([[0, 127, 128, N - 1], rng.choice(N, 200, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xq = oracle.quantize_act_q8k(x[toks])
    got = np.ascontiguousarray(y[toks][:, rows])
    y64, A = oracle.matmul_q8k_f64(fmt, sub, len(rows), K, xq, len(toks))
    assert_tol(got, y64, A, what="q8k full size")
    assert_bitwise(got, oracle.matmul_q8k_canon_f32(fmt, sub, len(rows), K, xq, len(toks)),
                   "q8k full size f32 order")
    for t in toks[:4]:
        y1 = host(g.matmul_q8k(fmt, w, N, K, x=dev(x[t:t + 1])))
        assert_bitwise(y[t:t + 1], y1, f"token {t} vs batch-1 GEMV")


@pytest.mark.parametrize("fmt", FMTS)
def test_q8k_gemm_wide_grid_ragged(g, fmt):
    """A grid of more than 512 tiles of 128 x 128 with ragged M and N (130 tokens,
    32805 rows): the launch shape with 128 activation rows per workgroup, on
    sampled rows against the oracle and on sampled tokens against batch 1."""
    N, K, M = 32805, 512, 130
    blob, _ = synth.weights(fmt, N, K, 2600 + fmt, s_range=(-128, 127))
    x = synth.activations(M, K, 2601)
    w, xd = dev(blob), dev(x)
    print(f"q8k wide ragged fmt={fmt}", flush=True)
    y = host(g.matmul_q8k(fmt, w, N, K, x=xd))
    rng = np.random.Generator(np.random.PCG64(2602))
    rows = np.unique(np.concatenate([[0, 127, 128, N - 38, N - 1], rng.choice(N, 300, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xq = oracle.quantize_act_q8k(x)
    assert_bitwise(np.ascontiguousarray(y[:, rows]),
                   oracle.matmul_q8k_canon_f32(fmt, sub, len(rows), K, xq, M), "wide grid f32 order")
    for t in (0, 127, 128, 129):
        y1 = host(g.matmul_q8k(fmt, w, N, K, x=dev(x[t:t + 1])))
        assert_bitwise(y[t:t + 1], y1, f"token {t} vs batch 1")
    P = host(g.partials_q8k(fmt, w, N, K, g.quantize_q8k(xd), M))
    assert_bitwise(np.ascontiguousarray(P[:, rows]),
                   oracle.partials_q8k(fmt, sub, len(rows), K, xq, M), "wide grid partials")


@pytest.mark.parametrize("fmt,N,K,M", [(synth.Q6_K, 151936, 1024, 16), (synth.Q6_K, 151936, 1024, 5),
                                       (synth.Q4_K, 14336, 4096, 16), (synth.Q6_K, 4096, 14336, 16),
                                       (synth.Q4_K, 1024, 4096, 11)])
def test_q8k_batched_decode_full_size(g, fmt, N, K, M):
    """Batched decode (5..16 rows) at the LM-head and 8B-class shapes: sampled
    weight rows of every token against the oracle, bitwise in the Q8_K f32
    order and within tolerance of f64; a few tokens' full rows against the
    batch-1 GEMV; the partials on the sampled rows."""
    blob, _ = synth.weights(fmt, N, K, 2700 + N % 97, dscale=0.02)
    x = synth.activations(M, K, 2701 + M)
    w, xd = dev(blob), dev(x)
    print(f"q8k batched full size fmt={fmt} N={N} K={K} M={M}", flush=True)
    y = host(g.matmul_q8k(fmt, w, N, K, x=xd))
    rng = np.random.Generator(np.random.PCG64(2702 + N))
    rows = np.unique(np.concatenate([[0, 15, 16, N - 1], rng.choice(N, 200, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xq = oracle.quantize_act_q8k(x)
    got = np.ascontiguousarray(y[:, rows])
    y64, A = oracle.matmul_q8k_f64(fmt, sub, len(rows), K, xq, M)
    assert_tol(got, y64, A, what="batched q8k full size")
    assert_bitwise(got, oracle.matmul_q8k_canon_f32(fmt, sub, len(rows), K, xq, M),
                   "batched q8k f32 order")
    for t in sorted({0, M // 2, M - 1}):
        y1 = host(g.matmul_q8k(fmt, w, N, K, x=dev(x[t:t + 1])))
        assert_bitwise(y[t:t + 1], y1, f"token {t} vs batch-1 GEMV")
    P = host(g.partials_q8k(fmt, w, N, K, g.quantize_q8k(xd), M))
    assert_bitwise(np.ascontiguousarray(P[:, rows]),
                   oracle.partials_q8k(fmt, sub, len(rows), K, xq, M), "batched partials")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [2, 8])
def test_q8k_batched_long_rows(g, fmt, M):
    """Rows of 65536 elements (256 superblocks, 32 rounds of the workgroup's
    waves; too long for the lane-per-chunk kernel's LDS staging, so at 2
    tokens too the batched kernel runs) with a ragged last tile (N = 37)."""
    N, K = 37, 65536
    blob, _ = synth.weights(fmt, N, K, 2800 + fmt, s_range=(-128, 127))
    x = synth.activations(M, K, 2801)
    xd = dev(x)
    print(f"q8k batched long rows fmt={fmt} M={M}", flush=True)
    y = host(g.matmul_q8k(fmt, dev(blob), N, K, x=xd))
    xq = oracle.quantize_act_q8k(x)
    y64, A = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, M)
    assert_tol(y, y64, A, what="long rows vs f64")
    assert_bitwise(y, oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq, M), "long rows f32 order")
    P = host(g.partials_q8k(fmt, dev(blob), N, K, g.quantize_q8k(xd), M))
    assert_bitwise(P, oracle.partials_q8k(fmt, blob, N, K, xq, M), "long rows partials")


@pytest.mark.parametrize("fmt,N,K,B", [(synth.Q4_K, 14336, 4096, 16), (synth.Q4_K, 333, 1024, 5),
                                       (synth.Q6_K, 90, 1024, 1), (synth.Q6_K, 77, 4352, 11),
                                       (synth.Q4_K, 40, 65536, 8), (synth.Q6_K, 16, 256, 16)])
def test_gateup_swiglu_q8k(g, fmt, N, K, B):
    """qmv_launch_gateup_swiglu_q8k: h bit-identical to the oracle's SwiGLU of
    the oracle's gate and up products in the Q8_K f32 order (sampled rows at
    the 8B-class shape), with x quantised by the launch and staged."""
    wg, _ = synth.weights(fmt, N, K, 2900 + N, dscale=0.02)
    wu, _ = synth.weights(fmt, N, K, 2901 + N, dscale=0.02)
    x = synth.activations(B, K, 2902 + B)
    xd = dev(x)
    print(f"gate/up swiglu q8k fmt={fmt} N={N} K={K} B={B}", flush=True)
    h = host(g.gateup_swiglu_q8k(fmt, dev(wg), dev(wu), N, K, x=xd))
    xq = g.quantize_q8k(xd)
    h2 = host(g.gateup_swiglu_q8k(fmt, dev(wg), dev(wu), N, K, xq=xq, B=B))
    assert_bitwise(h2, h, "staged x")
    rows = np.arange(N)
    if N > 400:
        rng = np.random.Generator(np.random.PCG64(2903))
        rows = np.unique(np.concatenate([[0, 15, 16, N - 1], rng.choice(N, 200, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = lambda blob: np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xo = oracle.quantize_act_q8k(x)
    gate = oracle.matmul_q8k_canon_f32(fmt, sub(wg), len(rows), K, xo, B)
    up = oracle.matmul_q8k_canon_f32(fmt, sub(wu), len(rows), K, xo, B)
    assert_bitwise(np.ascontiguousarray(h[:, rows]), oracle.swiglu(gate, up), "h = silu(g) u")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("B,Ks", [(16, (1024, 1024, 1024)), (5, (512, 512)), (3, (1024, 1024, 1024)),
                                  (16, (1024, 2048))])
def test_group_q8k_equals_single(g, fmt, B, Ks):
    """qmv_launch_group_q8k: every entry bit-identical to qmv_launch_q8k on
    its own (one launch of the batched kernel for B = 5..16 and one K, ragged
    N; the sequential path for B <= 4 or mixed K), with x quantised by the
    launch and staged in one shared xq; one entry also against the oracle."""
    Ns = (520, 130, 37)[:len(Ks)]
    blobs = [synth.weights(fmt, N, K, 3000 + i, s_range=(-128, 127))[0] for i, (N, K) in enumerate(zip(Ns, Ks))]
    xs = [synth.activations(B, K, 3010 + i) for i, K in enumerate(Ks)]
    ws = [dev(b) for b in blobs]
    print(f"group q8k fmt={fmt} B={B} Ks={Ks}", flush=True)
    want = [host(g.matmul_q8k(fmt, w, N, K, x=dev(x))) for w, N, K, x in zip(ws, Ns, Ks, xs)]
    # x given: each entry quantises its own x
    xds = [dev(x) for x in xs]
    xqs = [torch.empty(g.qmv_act_bytes_q8k(B, K), dtype=torch.uint8, device="cuda") for K in Ks]
    ys = [torch.full((B, N), float("nan"), device="cuda") for N in Ns]
    g.qmv_launch_group_q8k(fmt, B, [(w.data_ptr(), N, K, xd.data_ptr(), xq.data_ptr(), y.data_ptr())
                                    for w, N, K, xd, xq, y in zip(ws, Ns, Ks, xds, xqs, ys)])
    for i in range(len(Ns)):
        assert_bitwise(host(ys[i]), want[i], f"entry {i}, x given")
    # staged: one x for the entries of the first K, one shared xq
    if len(set(Ks)) == 1:
        xq = g.quantize_q8k(xds[0])
        ys2 = [torch.full((B, N), float("nan"), device="cuda") for N in Ns]
        g.qmv_launch_group_q8k(fmt, B, [(w.data_ptr(), N, Ks[0], None, xq.data_ptr(), y.data_ptr())
                                        for w, N, y in zip(ws, Ns, ys2)])
        for i, (w, N) in enumerate(zip(ws, Ns)):
            assert_bitwise(host(ys2[i]), host(g.matmul_q8k(fmt, w, N, Ks[0], x=xds[0])),
                           f"entry {i}, staged")
    xo = oracle.quantize_act_q8k(xs[1])
    assert_bitwise(host(ys[1]), oracle.matmul_q8k_canon_f32(fmt, blobs[1], Ns[1], Ks[1], xo, B),
                   "entry 1 vs oracle")
