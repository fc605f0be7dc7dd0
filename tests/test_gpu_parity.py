"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

* Q8_0 activation blocks and int32 block partials: bit-exact.
* f32 outputs: within 1e-4 * sum|w^ x^| of the oracle's f64 result, and
  bit-identical to the oracle's emulation of the documented f32 order.
* Every row of a batched (B <= 16) or prefill call is bit-identical to the
  batch-1 call on that row.
Shapes span several 16-row tiles, ragged row tiles, ragged last chunks, every
weight-row alignment the layouts allow, and the blob's unaligned end.
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


def pub(xq, rows, K):
    return host(xq)[: rows * (K // 32) * 34]


# (fmt, N, K): K=896 ragged chunk; K=416 13 blocks; K=32 single block;
# Q6_K K=768 -> 630-byte rows (2-byte aligned spans), odd N -> unaligned end;
# Q5_0 K=4192 -> 2882-byte rows (2-byte aligned).
SMALL = [
    (synth.Q8_0, 100, 896), (synth.Q8_0, 16, 32), (synth.Q8_0, 33, 4096 + 96),
    (synth.Q4_0, 37, 416), (synth.Q4_0, 50, 4864), (synth.Q4_0, 17, 32),
    (synth.Q4_K, 45, 1024), (synth.Q4_K, 16, 256), (synth.Q4_K, 7, 4864),
    (synth.Q6_K, 33, 768), (synth.Q6_K, 16, 256), (synth.Q6_K, 19, 1024),
    (synth.Q5_0, 45, 896), (synth.Q5_0, 16, 32), (synth.Q5_0, 33, 4096 + 96),
    (synth.Q4_1, 45, 896), (synth.Q4_1, 17, 32), (synth.Q5_1, 33, 4096 + 96),
    (synth.Q5_1, 16, 416), (synth.Q8_1, 40, 896), (synth.Q8_1, 19, 64),
    # whole 256-element chunks (the branch-free weight loads) with rows past
    # the last full unit of a wave: 64 / C rows per wave for C chunks a row
    (synth.Q8_0, 37, 512), (synth.Q4_0, 129, 256), (synth.Q5_0, 29, 1024),
    (synth.Q4_1, 21, 768), (synth.Q5_1, 13, 2048), (synth.Q8_1, 11, 4096),
]


def _inputs(fmt, N, K, B, seed):
    blob, _ = synth.weights(fmt, N, K, seed, s_range=(-128, 127))
    x = synth.activations(B, K, seed + 7)
    return blob, x


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 896), (16, 4096), (21, 1024), (40, 4864)])
def test_quantize_bit_exact(g, rows, K):
    x = synth.activations(rows, K, 5) * np.float32(4.0)
    x[0, :32] = 0.0                        # an all-zero block
    x[-1, 32:64] = np.float32(1e-3)        # a tiny block (subnormal fp16 scale)
    want = oracle.quantize_act(x)
    xq = g.quantize(dev(x))
    assert_bitwise(pub(xq, rows, K), want, "Q8_0 blocks")


@pytest.mark.parametrize("fmt,N,K", SMALL)
@pytest.mark.parametrize("B", [1, 3, 16])
def test_partials_bit_exact(g, fmt, N, K, B):
    blob, x = _inputs(fmt, N, K, B, 100 + N)
    xq = g.quantize(dev(x))
    P = g.partials(fmt, dev(blob), N, K, xq, B)
    want = oracle.partials(fmt, blob, N, K, oracle.quantize_act(x), B)
    assert_bitwise(host(P), want, "partials")


@pytest.mark.parametrize("fmt,N,K", SMALL)
@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 16])
def test_qmv_against_oracle(g, fmt, N, K, B):
    blob, x = _inputs(fmt, N, K, B, 200 + N)
    y = host(g.matvec(fmt, dev(blob), N, K, x=dev(x)))
    xq = oracle.quantize_act(x)
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    assert_tol(y, y64, A, what="qmv vs f64")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, B), "qmv vs f32 order")


@pytest.mark.parametrize("fmt,N,K", SMALL)
def test_batch_rows_equal_batch1(g, fmt, N, K):
    blob, x = _inputs(fmt, N, K, 16, 300 + N)
    w = dev(blob)
    y16 = host(g.matvec(fmt, w, N, K, x=dev(x)))
    for B in (2, 7, 16):
        yB = host(g.matvec(fmt, w, N, K, x=dev(x[:B])))
        assert_bitwise(yB, y16[:B], f"B={B} vs B=16")
    for m in (0, 5, 15):
        y1 = host(g.matvec(fmt, w, N, K, x=dev(x[m:m + 1])))
        assert_bitwise(y1[0], y16[m], f"row {m} vs batch-1")
    # permuting the batch permutes the rows
    perm = np.random.default_rng(1).permutation(16)
    yp = host(g.matvec(fmt, w, N, K, x=dev(x[perm])))
    assert_bitwise(yp, y16[perm], "permuted batch")


@pytest.mark.parametrize("fmt,N,K", [SMALL[0], SMALL[4], SMALL[6], SMALL[9], SMALL[12],
                                     SMALL[15], SMALL[17], SMALL[19]])
@pytest.mark.parametrize("M", [17, 40])
def test_qmm_rows_equal_qmv(g, fmt, N, K, M):
    blob, x = _inputs(fmt, N, K, M, 400 + N)
    w = dev(blob)
    y = host(g.matmul(fmt, w, N, K, x=dev(x)))
    xq = oracle.quantize_act(x)
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, M), "qmm vs f32 order")
    for m in (0, 16, M - 1):
        y1 = host(g.matvec(fmt, w, N, K, x=dev(x[m:m + 1])))
        assert_bitwise(y[m], y1[0], f"qmm row {m} vs qmv")


# Prefill GEMM over several workgroup tiles with ragged edges in M
# and N, and a ragged last K step (K = 416: 13 blocks).  Q6_K also with the
# sub-scale range of the workloads ([-32, 31], folded into f16 codes) and with
# a few rows whose odd sub-scales beyond +-64 force the unfolded path in
# their steps only.
GEMM = [
    (synth.Q8_0, 129, 416, 129, None), (synth.Q4_0, 300, 896, 130, None),
    (synth.Q4_K, 200, 1024, 150, None), (synth.Q6_K, 140, 768, 131, (-128, 127)),
    (synth.Q6_K, 140, 768, 131, (-32, 31)), (synth.Q6_K, 260, 1024, 257, "mixed"),
    (synth.Q5_0, 150, 896, 140, None), (synth.Q5_0, 129, 4192, 129, None),
    (synth.Q4_1, 150, 896, 140, None), (synth.Q5_1, 129, 4192, 129, None),
    (synth.Q8_1, 131, 416, 150, None),
]


@pytest.mark.parametrize("fmt,N,K,M,srange", GEMM)
def test_gemm_tiles_against_oracle(g, fmt, N, K, M, srange):
    seed = 900 + N + M
    if srange == "mixed":
        f = synth.draw_fields(fmt, N, K, seed, s_range=(-32, 31))
        f["s"][7, 0, 5] = 101     # odd, beyond +-64: row 7, superblock 0, block 2
        f["s"][200, 1, 14] = -77  # row 200, superblock 1, block 15
        blob = synth.encode(f)
    else:
        blob, _ = synth.weights(fmt, N, K, seed, s_range=srange or (-32, 31))
    x = synth.activations(M, K, seed + 7)
    w = dev(blob)
    y = host(g.matmul(fmt, w, N, K, x=dev(x)))
    xq = oracle.quantize_act(x)
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, M)
    assert_tol(y, y64, A, what="gemm vs f64")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, M), "gemm vs f32 order")
    for m in (0, 127, 128, M - 1):
        y1 = host(g.matvec(fmt, w, N, K, x=dev(x[m:m + 1])))
        assert_bitwise(y[m], y1[0], f"gemm row {m} vs qmv")


# The shapes above launch at most 128 tiles of 128 x 128 and run the 64 x 64
# workgroup tile; this grid (17 x 16 tiles of 128, ragged in M, N and K) runs
# the 128 x 128 one, for every format and for Q6_K steps staged unfolded.  Sampled tokens are checked against the oracle on every row.
@pytest.mark.parametrize("fmt,srange", [(synth.Q8_0, None), (synth.Q4_0, None), (synth.Q5_0, None),
                                        (synth.Q4_1, None), (synth.Q5_1, None), (synth.Q8_1, None),
                                        (synth.Q4_K, None), (synth.Q6_K, None), (synth.Q6_K, "mixed")])
def test_gemm_large_tile_grid(g, fmt, srange):
    M, N = 2067, 1921
    K = 768 if fmt in (synth.Q4_K, synth.Q6_K) else 416
    seed = 1700 + fmt
    if srange == "mixed":
        f = synth.draw_fields(fmt, N, K, seed, s_range=(-32, 31))
        f["s"][7, 0, 5] = 101      # odd, beyond +-64
        f["s"][1900, 2, 14] = -77
        blob = synth.encode(f)
    else:
        blob, _ = synth.weights(fmt, N, K, seed)
    x = synth.activations(M, K, seed + 7)
    w = dev(blob)
    y = host(g.matmul(fmt, w, N, K, x=dev(x)))
    toks = np.array([0, 1, 63, 64, 127, 128, 1000, 2047, 2048, M - 1])
    xq = oracle.quantize_act(x[toks])
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, len(toks))
    assert_tol(y[toks], y64, A, what="gemm vs f64")
    assert_bitwise(y[toks], oracle.matmul_canon_f32(fmt, blob, N, K, xq, len(toks)),
                   "gemm vs f32 order")
    for m in (0, 128, M - 1):
        y1 = host(g.matvec(fmt, w, N, K, x=dev(x[m:m + 1])))
        assert_bitwise(y[m], y1[0], f"gemm row {m} vs qmv")


@pytest.mark.parametrize("fmt,N,K", [SMALL[1], SMALL[5], SMALL[7], SMALL[10], SMALL[13],
                                     SMALL[16], SMALL[18], SMALL[20]])
def test_staged_xq_paths(g, fmt, N, K):
    """x = NULL uses xq as staged; quantize with x = NULL re-stages Q8_0 blocks
    written by someone else (here the oracle) over a scribbled staging area."""
    B = 4
    blob, x = _inputs(fmt, N, K, B, 500)
    w = dev(blob)
    y_ref = host(g.matvec(fmt, w, N, K, x=dev(x)))
    xq = g.quantize(dev(x))
    assert_bitwise(host(g.matvec(fmt, w, N, K, xq=xq, B=B)), y_ref, "staged xq")
    xq2 = g.act_buffer(B, K)
    xq2.fill_(0xAB)
    xq2[: B * (K // 32) * 34] = dev(oracle.quantize_act(x))
    g.quantize(None, xq2, rows=B, K=K)
    pub_end = B * (K // 32) * 34
    assert_bitwise(host(xq2)[:pub_end], host(xq)[:pub_end], "re-staged xq: Q8_0 blocks")
    # both staging copies: the MFMA one (partials hook) and the row-major one (B <= 4 GEMV)
    assert_bitwise(host(g.partials(fmt, w, N, K, xq2, B)), host(g.partials(fmt, w, N, K, xq, B)),
                   "re-staged xq: MFMA staging")
    assert_bitwise(host(g.matvec(fmt, w, N, K, xq=xq2, B=B)), y_ref, "x=NULL vs x")
    assert_bitwise(host(g.matmul(fmt, w, N, K, xq=xq2, M=B)), y_ref, "qmm x=NULL vs qmv")


@pytest.mark.parametrize("fmt,N,K", [SMALL[0], SMALL[4], SMALL[8], SMALL[11], SMALL[14],
                                     SMALL[15], SMALL[17], SMALL[19]])
@pytest.mark.parametrize("B", [1, 3, 4, 5])
def test_fused_quantisation_leaves_xq_as_quantize(g, fmt, N, K, B):
    """qmv with x quantises inside the GEMV for B <= 4: xq must then hold the
    same Q8_0 blocks as quantize_act_q8_0 and serve a later x = NULL call."""
    blob, x = _inputs(fmt, N, K, B, 700 + B)
    w = dev(blob)
    xq = g.act_buffer(B, K)
    xq.fill_(0x5A)
    y = host(g.matvec(fmt, w, N, K, x=dev(x), xq=xq))
    pub_end = B * (K // 32) * 34
    assert_bitwise(host(xq)[:pub_end], oracle.quantize_act(x).reshape(-1), "fused xq blocks")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, oracle.quantize_act(x), B),
                   "fused vs f32 order")
    y2 = torch.empty(B, N, dtype=torch.float32, device="cuda")
    assert_bitwise(host(g.matvec(fmt, w, N, K, xq=xq, B=B, y=y2)), y, "reuse of fused xq")
    xq3 = g.quantize(dev(x))
    assert_bitwise(host(g.matvec(fmt, w, N, K, xq=xq3, B=B)), y, "quantize + x=NULL vs fused")


def test_repeat_runs_are_identical(g):
    fmt, N, K = synth.Q4_K, 300, 4096
    blob, x = _inputs(fmt, N, K, 5, 600)
    w, xd = dev(blob), dev(x)
    ys = [host(g.matvec(fmt, w, N, K, x=xd)) for _ in range(3)]
    assert_bitwise(ys[0], ys[1], "run 1 vs 2")
    assert_bitwise(ys[0], ys[2], "run 1 vs 3")


def test_scaling_and_negation(g):
    fmt, N, K = synth.Q6_K, 40, 1024
    blob, x = _inputs(fmt, N, K, 3, 700)
    w = dev(blob)
    y = host(g.matvec(fmt, w, N, K, x=dev(x)))
    yn = host(g.matvec(fmt, w, N, K, x=dev(-x)))
    assert_bitwise(yn, -y, "negated x")
    y4 = host(g.matvec(fmt, w, N, K, x=dev(x * np.float32(4.0))))
    assert_bitwise(y4, y * np.float32(4.0), "x * 4")


def test_zero_activations_give_zero(g):
    fmt, N, K = synth.Q4_K, 20, 512
    blob, _ = _inputs(fmt, N, K, 1, 800)
    y = host(g.matvec(fmt, dev(blob), N, K, x=dev(np.zeros((2, K), np.float32))))
    assert np.all(y == 0) and not np.any(np.signbit(y))


def test_largest_k(g):
    fmt, N, K, B = synth.Q4_0, 3, 1 << 20, 2
    blob, x = _inputs(fmt, N, K, B, 900)
    y = host(g.matvec(fmt, dev(blob), N, K, x=dev(x)))
    xq = oracle.quantize_act(x)
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    assert_tol(y, y64, A, what="K=2^20")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, B), "K=2^20 f32 order")


def test_byte_coverage(g):
    """Changing any single weight byte of a small blob changes some output."""
    fmt, N, K = synth.Q4_K, 2, 256
    f = synth.draw_fields(fmt, N, K, 950)
    f["sc"] = np.maximum(f["sc"], 1)                # every code and min matters
    f["m"] = np.maximum(f["m"], 1)
    f["d"] = np.maximum(f["d"], np.float16(1e-2))
    f["dmin"] = np.maximum(f["dmin"], np.float16(1e-2))
    blob = synth.encode(f)
    x = np.abs(synth.activations(1, K, 951)) + np.float32(0.5)   # codes all >= 1
    xd = dev(x)
    base = host(g.matvec(fmt, dev(blob), N, K, x=xd))
    unchanged = []
    for i in range(blob.size):
        b2 = blob.copy()
        b2[i] ^= 0x11
        if np.array_equal(host(g.matvec(fmt, dev(b2), N, K, x=xd)), base):
            unchanged.append(i)
    assert not unchanged, f"bytes with no effect: {unchanged[:10]}"


@pytest.mark.parametrize("fmt", [synth.Q5_0, synth.Q4_1, synth.Q5_1])
@pytest.mark.parametrize("B", [1, 5])
def test_byte_coverage_32(g, fmt, B):
    """Flipping bit 0 or bit 4 of any byte (scale, minimum, fifth-bit word or
    nibbles; each flip moves exactly one field) changes the output, through
    the lane-per-chunk path (B = 1) and the MFMA path (B = 5)."""
    N, K = 2, 64
    f = synth.draw_fields(fmt, N, K, 960)
    f["d"] = np.maximum(f["d"], np.float16(1e-2))
    if "m" in f:
        f["m"] = np.minimum(f["m"], np.float16(-1e-2))
    blob = synth.encode(f)
    x = np.abs(synth.activations(B, K, 961)) + np.float32(0.5)   # codes all >= 1
    xd = dev(x)
    base = host(g.matvec(fmt, dev(blob), N, K, x=xd))
    unchanged = []
    for i in range(blob.size):
        for mask in (0x01, 0x10):
            b2 = blob.copy()
            b2[i] ^= mask
            if np.array_equal(host(g.matvec(fmt, dev(b2), N, K, x=xd)), base):
                unchanged.append((i, mask))
    assert not unchanged, f"bytes with no effect: {unchanged[:10]}"


@pytest.mark.parametrize("fmt,shapes", [
    (synth.Q4_0, [(4864, 896), (4864, 896), (896, 4864)]),
    (synth.Q4_K, [(300, 1024), (45, 4864), (7, 256)]),
    (synth.Q6_K, [(33, 768), (19, 1024)]),
    (synth.Q8_0, [(100, 896), (16, 32), (33, 4192), (17, 64), (5, 32), (70, 416), (9, 96), (40, 4096)]),
    (synth.Q5_0, [(4864, 896), (896, 896), (128, 896)]),
    (synth.Q4_1, [(300, 896), (45, 4864)]),
    (synth.Q5_1, [(300, 896), (45, 4864)]),
    (synth.Q8_1, [(100, 896), (33, 4192)]),
    # every entry of whole chunks (the branch-free loads), rows past the
    # last full unit of a wave in each
    (synth.Q8_0, [(37, 512), (129, 256), (5, 4096)]),
    (synth.Q5_0, [(29, 1024), (3, 4864)]),
    # one large GEMV between two tiny ones: most workgroup rows of the grid
    # belong to no work and exit
    (synth.Q4_0, [(8, 32), (20000, 896), (3, 4864)]),
])
@pytest.mark.parametrize("B", [1, 3, 5])
def test_group_equals_single_launches(g, fmt, shapes, B):
    """qmv_launch_group: every entry bit-identical to its own qmv_launch, with
    quantisation in the launch (xq written for the first entry only) and with
    staged xq."""
    items, ref, xs, blobs = [], [], [], []
    for k, (N, K) in enumerate(shapes):
        blob, x = _inputs(fmt, N, K, B, 800 + 10 * k + B)
        w = dev(blob)
        blobs.append(w)
        xs.append(x)
        ref.append(host(g.matvec(fmt, w, N, K, x=dev(x))))
        # xq may be left out only when the group runs as one launch (B <= 4)
        items.append({"w": w, "N": N, "K": K, "x": dev(x),
                      "xq": g.act_buffer(B, K) if k == 0 or B > 4 else None})
    ys = g.matvec_group(fmt, items)
    for k, (N, K) in enumerate(shapes):
        assert_bitwise(host(ys[k]), ref[k], f"group entry {k} ({N}x{K})")
    pub_end = B * (shapes[0][1] // 32) * 34
    assert_bitwise(host(items[0]["xq"])[:pub_end], oracle.quantize_act(xs[0]).reshape(-1),
                   "group xq")
    staged = [{"w": blobs[k], "N": N, "K": K, "B": B, "xq": g.quantize(dev(xs[k]))}
              for k, (N, K) in enumerate(shapes)]
    ys2 = g.matvec_group(fmt, staged)
    for k in range(len(shapes)):
        assert_bitwise(host(ys2[k]), ref[k], f"staged group entry {k}")


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0, synth.Q4_K, synth.Q6_K, synth.Q5_0,
                                 synth.Q4_1, synth.Q5_1, synth.Q8_1])
@pytest.mark.parametrize("fused", [False, True])
def test_large_gemv_many_workgroups(g, fmt, fused):
    """Batch 1 over 24613 rows: more workgroups than the chip holds at once,
    a ragged last unit, with the quantisation fused and staged, against the
    documented f32 order."""
    N, K = 24613, 4096
    blob, x = _inputs(fmt, N, K, 1, 950 + fmt)
    w = dev(blob)
    xq = oracle.quantize_act(x)
    if fused:
        y = host(g.matvec(fmt, w, N, K, x=dev(x)))
    else:
        y = host(g.matvec(fmt, w, N, K, xq=g.quantize(dev(x)), B=1))
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, 1), "large gemv vs f32 order")
