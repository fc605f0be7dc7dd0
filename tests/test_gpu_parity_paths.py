"""GPU parity of every kernel path, at the level of its exact integers:

* the int32 block partials straight from the kernel that qmv_launch /
  qmm_launch runs at that many rows (lane-per-chunk for B <= 4, MFMA for
  B = 5..16, the prefill GEMM for M > 16), compared bit for bit with the
  oracle's partials, including blocks whose fp16 weight scale is subnormal
  (where the f32 replay could not see a wrong partial);
* byte coverage: flipping bit 0 or bit 4 of any weight byte changes the
  output, on each path and for every format (Q8_1's stored s, which the
  multiply does not read, excepted);
* activation blocks whose fp16 scale underflows to 0 while their codes are
  not 0 (amax < 127 * 2^-25);
* rows longer than 64 chunks (K > 16384), which the lane-per-chunk kernel
  walks in several passes, fused and staged.
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


ALL = [synth.Q8_0, synth.Q4_0, synth.Q5_0, synth.Q4_1, synth.Q5_1, synth.Q8_1, synth.Q4_K,
       synth.Q6_K]


def _with_subnormal_scales(fmt, N, K, seed):
    """Weights whose fp16 block scales are subnormal in about a quarter of the blocks."""
    f = synth.draw_fields(fmt, N, K, seed, s_range=(-128, 127))
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    d = f["d"]
    tiny = rng.random(d.shape) < 0.25
    d[tiny] = (rng.integers(1, 1023, size=int(tiny.sum())) * 2.0 ** -24).astype(np.float16)
    return synth.encode(f)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K", [(37, 896), (16, 256), (70, 4096 + 256)])
@pytest.mark.parametrize("B", [1, 2, 4, 5, 9])
def test_partials_of_the_gemv_path(g, fmt, N, K, B):
    if K % synth.BLOCK[fmt][0]:
        pytest.skip("K not a whole number of blocks")
    blob = _with_subnormal_scales(fmt, N, K, 700 + N + B)
    x = synth.activations(B, K, 701 + K)
    print(f"partials gemv fmt={fmt} N={N} K={K} B={B}", flush=True)
    xq = g.quantize(dev(x))
    P = host(g.partials(fmt, dev(blob), N, K, xq, B))
    assert_bitwise(P, oracle.partials(fmt, blob, N, K, oracle.quantize_act(x), B), "partials")


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("N,K,M", [(40, 896, 17), (40, 512, 17), (130, 1024, 70), (300, 256, 129)])
def test_partials_of_the_gemm_path(g, fmt, N, K, M):
    if K % synth.BLOCK[fmt][0]:
        pytest.skip("K not a whole number of blocks")
    blob = _with_subnormal_scales(fmt, N, K, 800 + N)
    x = synth.activations(M, K, 801 + M)
    print(f"partials gemm fmt={fmt} N={N} K={K} M={M}", flush=True)
    xq = g.quantize(dev(x))
    P = host(g.partials(fmt, dev(blob), N, K, xq, M, gemm=True))
    assert_bitwise(P, oracle.partials(fmt, blob, N, K, oracle.quantize_act(x), M), "gemm partials")


def _coverage_fields(fmt, N, K, seed):
    f = synth.draw_fields(fmt, N, K, seed)
    f["d"] = np.maximum(f["d"], np.float16(1e-2))
    if "m" in f and fmt in (synth.Q4_1, synth.Q5_1):
        f["m"] = np.minimum(f["m"], np.float16(-1e-2))
    if fmt == synth.Q4_K:
        f["sc"] = np.maximum(f["sc"], 1)
        f["m"] = np.maximum(f["m"], 1)
        f["dmin"] = np.maximum(f["dmin"], np.float16(1e-2))
    if fmt == synth.Q6_K:
        f["s"] = np.where(f["s"] == 0, np.int8(3), f["s"]).astype(np.int8)
    return f


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("path", ["gemv_b1", "gemv_b5", "gemm_m17"])
def test_byte_coverage_every_path(g, fmt, path):
    """Flipping bit 0 or bit 4 of any weight byte (each flip moves exactly one
    field: a scale, a minimum, a code, a fifth or high bit) changes y."""
    N = 2
    K = 256 if fmt in (synth.Q4_K, synth.Q6_K) else 64
    rows = {"gemv_b1": 1, "gemv_b5": 5, "gemm_m17": 17}[path]
    blob = synth.encode(_coverage_fields(fmt, N, K, 960 + fmt))
    x = np.abs(synth.activations(rows, K, 961)) + np.float32(0.5)   # codes all >= 1
    xd = dev(x)
    fn = g.matmul if path == "gemm_m17" else g.matvec
    print(f"coverage fmt={fmt} path={path}", flush=True)
    base = host(fn(fmt, dev(blob), N, K, x=xd))
    unchanged = set()
    for i in range(blob.size):
        for mask in (0x01, 0x10):
            b2 = blob.copy()
            b2[i] ^= mask
            if np.array_equal(host(fn(fmt, dev(b2), N, K, x=xd)), base):
                unchanged.add(i)
    expected = set()
    if fmt == synth.Q8_1:   # the stored s = d * sum(q) is not part of the multiply
        bb = synth.BLOCK[fmt][1]
        expected = {blk * bb + o for blk in range(blob.size // bb) for o in (2, 3)}
    assert unchanged == expected, f"bytes with no effect: {sorted(unchanged - expected)[:10]}"


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q4_1])
@pytest.mark.parametrize("rows", [1, 3, 6, 40])
def test_underflowing_activation_scales(g, fmt, rows):
    """Blocks whose amax < 127 * 2^-25: d rounds to fp16 0 while the codes
    (taken from the f32 d) are not 0; the block then adds nothing."""
    K, N = 1024, 96
    blob, _ = synth.weights(fmt, N, K, 990)
    x = synth.activations(rows, K, 991)
    x[:, 64:96] *= np.float32(1e-7)     # amax ~ 3e-7 -> d ~ 2.4e-9 < 2^-25
    x[:, 256:288] *= np.float32(2e-6)   # d near the smallest fp16 subnormal
    xq_o = oracle.quantize_act(x)
    blk = xq_o.reshape(rows, K // 32, 34)
    assert np.all(blk[:, 2, :2] == 0) and np.any(blk[:, 2, 2:] != 0)
    xd = dev(x)
    print(f"underflow fmt={fmt} rows={rows}", flush=True)
    xq = g.quantize(xd)
    assert_bitwise(host(xq)[: xq_o.size], xq_o, "Q8_0 blocks")
    fn = g.matmul if rows > 16 else g.matvec
    y = host(fn(fmt, dev(blob), N, K, x=xd))
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq_o, rows)
    assert_tol(y, y64, A, what="underflow")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq_o, rows), "underflow f32 order")
    P = host(g.partials(fmt, dev(blob), N, K, g.quantize(xd), rows, gemm=rows > 16))
    assert_bitwise(P, oracle.partials(fmt, blob, N, K, xq_o, rows), "underflow partials")


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0, synth.Q6_K, synth.Q4_K])
@pytest.mark.parametrize("K", [28672, 32768])
@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_multipass_rows(g, fmt, K, B, fused):
    """Rows of more than 64 chunks: one row per wave, walked in passes."""
    N = 40
    blob, _ = synth.weights(fmt, N, K, 1100 + K)
    x = synth.activations(B, K, 1101)
    xd = dev(x)
    print(f"multipass fmt={fmt} K={K} B={B} fused={fused}", flush=True)
    if fused:
        y = host(g.matvec(fmt, dev(blob), N, K, x=xd))
    else:
        y = host(g.matvec(fmt, dev(blob), N, K, xq=g.quantize(xd), B=B))
    xq_o = oracle.quantize_act(x)
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq_o, B)
    assert_tol(y, y64, A, what="multipass")
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq_o, B), "multipass f32 order")


@pytest.mark.parametrize("rows,K", [(1, 1024), (3, 896), (16, 4096), (40, 512)])
def test_blocks_too_small_for_a_finite_reciprocal_scale(g, rows, K):
    """Subnormal-amax blocks (1/d overflows f32) quantise to all-zero codes on
    every quantiser: the standalone launch, the GEMV-fused one and the
    gate/up pair's; the multiply then adds nothing for them."""
    x = synth.activations(rows, K, 1200 + K)
    x[:, 32:64] *= np.float32(1e-40)     # subnormal amax
    x[:, 64:96] *= np.float32(5e-38)     # d ~ 1.6e-39: 1/d = inf
    x[:, 128:160] *= np.float32(3e-36)   # 1/d finite, fp16(d) = 0
    xq_o = oracle.quantize_act(x)
    blk = xq_o.reshape(rows, K // 32, 34)
    assert np.all(blk[:, 1:3] == 0) and np.any(blk[:, 4, 2:] != 0)
    xd = dev(x)
    print(f"tiny scales rows={rows} K={K}", flush=True)
    assert_bitwise(host(g.quantize(xd))[: xq_o.size], xq_o, "standalone quantiser")
    fmt, N = synth.Q4_0, 48
    blob, _ = synth.weights(fmt, N, K, 1201)
    xq = g.act_buffer(rows, K) if rows <= 16 else None
    if rows <= 16:
        y = host(g.matvec(fmt, dev(blob), N, K, x=xd, xq=xq))
        assert_bitwise(host(xq)[: xq_o.size], xq_o, "GEMV quantiser")
    else:
        y = host(g.matmul(fmt, dev(blob), N, K, x=xd))
    assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq_o, rows), "y")
    if rows <= 16:
        wu, _ = synth.weights(fmt, N, K, 1202)
        h = host(g.gateup_swiglu(fmt, dev(blob), dev(wu), N, K, x=xd))
        want = oracle.swiglu(oracle.matmul_canon_f32(fmt, blob, N, K, xq_o, rows),
                             oracle.matmul_canon_f32(fmt, wu, N, K, xq_o, rows))
        assert_bitwise(h, want, "h")
