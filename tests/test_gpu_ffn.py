"""GPU parity of the fused decode FFN: qmv_launch_gateup_swiglu (gate and up
GEMVs with the SwiGLU h = silu(g) * u in their epilogue) and the down GEMV
fed with h, against the CPU oracle chain: canonical-f32 gate and up ->
oracle SwiGLU -> Q8_0 of h -> down.

* h: bit-identical to oracle.swiglu of the oracle's canonical-f32 gate and up
  (every product bit-identical to qmv_launch; the SwiGLU evaluated in f64 on
  both sides and rounded once);
* the quantisation of h (xq of the down GEMV): bit-exact;
* y: within 1e-4 * sum|w^ x^| of the f64 result and bit-identical to the
  canonical f32 order.
Covers the one-launch path (B <= 4, K <= 8192; shapes with an odd number of
rows per wave and a ragged last unit), the fallback (B > 4; K > 8192),
staged and 4-byte-aligned activations."""
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


def _pair(fmt, N, K, seed):
    wg, _ = synth.weights(fmt, N, K, seed, dscale=0.02)
    wu, _ = synth.weights(fmt, N, K, seed + 1, dscale=0.02)
    return wg, wu


def _oracle_h(fmt, wg, wu, N, K, x):
    xq = oracle.quantize_act(x)
    gate = oracle.matmul_canon_f32(fmt, wg, N, K, xq, x.shape[0])
    up = oracle.matmul_canon_f32(fmt, wu, N, K, xq, x.shape[0])
    return oracle.swiglu(gate, up)


# (fmt, N, K, B): K = 896 -> 4 chunks, 8 pairs per wave; K = 4864 -> 19 chunks,
# 3 rows per wave -> 1 pair (one lane row idle); K = 4096 -> 2 pairs;
# K = 32 single block; N not a multiple of the pairs per wave.
ONE_LAUNCH = [
    (synth.Q4_0, 4864, 896, 1), (synth.Q4_0, 333, 896, 3), (synth.Q4_K, 1000, 4096, 1),
    (synth.Q4_K, 77, 4096, 4), (synth.Q6_K, 90, 1024, 2), (synth.Q8_0, 129, 4864, 1),
    (synth.Q5_0, 40, 896, 4), (synth.Q4_1, 31, 32, 1), (synth.Q5_1, 45, 416, 2),
    (synth.Q8_1, 64, 896, 3),
]
FALLBACK = [
    (synth.Q4_0, 200, 896, 5), (synth.Q4_K, 130, 4096, 16), (synth.Q6_K, 50, 9216, 1),
    (synth.Q8_0, 70, 8192 + 32, 2),
]


@pytest.mark.parametrize("fmt,N,K,B", ONE_LAUNCH + FALLBACK)
def test_gateup_swiglu_h_bit_exact(g, fmt, N, K, B):
    wg, wu = _pair(fmt, N, K, 300 + N)
    x = synth.activations(B, K, 301 + K)
    print(f"gateup fmt={fmt} N={N} K={K} B={B}", flush=True)
    h = g.gateup_swiglu(fmt, dev(wg), dev(wu), N, K, x=dev(x))
    torch.cuda.synchronize()
    assert_bitwise(h.cpu().numpy(), _oracle_h(fmt, wg, wu, N, K, x), "h")


@pytest.mark.parametrize("fmt,N,K,B", [ONE_LAUNCH[2], FALLBACK[1]])
def test_gateup_swiglu_staged_and_unaligned_x(g, fmt, N, K, B):
    wg, wu = _pair(fmt, N, K, 400 + N)
    x = synth.activations(B, K, 401)
    want = _oracle_h(fmt, wg, wu, N, K, x)
    wgd, wud = dev(wg), dev(wu)
    # staged: quantise first, then x NULL
    xq = torch.zeros(g.qmv_gateup_act_bytes(B, N, K), dtype=torch.uint8, device="cuda")
    g.quantize(dev(x), xq=xq)
    h = g.gateup_swiglu(fmt, wgd, wud, N, K, xq=xq, B=B)
    torch.cuda.synchronize()
    assert_bitwise(h.cpu().numpy(), want, "h from staged xq")
    # x 4-byte aligned only (one float into a buffer)
    buf = torch.zeros(B * K + 1, dtype=torch.float32, device="cuda")
    buf[1:] = dev(x).reshape(-1)
    xv = buf[1:].view(B, K)
    assert xv.data_ptr() % 16 == 4
    h2 = g.gateup_swiglu(fmt, wgd, wud, N, K, x=xv)
    torch.cuda.synchronize()
    assert_bitwise(h2.cpu().numpy(), want, "h from 4-byte aligned x")


@pytest.mark.parametrize("fmt,N,K,B", [
    (synth.Q4_0, 4864, 896, 1),    # the pages' Qwen2.5-0.5B FFN (down 896 x 4864)
    (synth.Q4_K, 1536, 4096, 2),   # 8B-class gate/up rows (a slice), down Q6_K
    (synth.Q4_K, 512, 4096, 8),
])
def test_ffn_chain(g, fmt, N, K, B):
    """gate/up + SwiGLU, then down on h: y against the oracle chain."""
    fdown = synth.Q6_K if fmt == synth.Q4_K else fmt
    wg, wu = _pair(fmt, N, K, 500 + N)
    wd, _ = synth.weights(fdown, K, N, 502 + N, dscale=0.02)
    x = synth.activations(B, K, 503)
    h = g.gateup_swiglu(fmt, dev(wg), dev(wu), N, K, x=dev(x))
    xq_d = g.act_buffer(B, N)
    y = g.matvec(fdown, dev(wd), K, N, x=h, xq=xq_d)
    torch.cuda.synchronize()
    h_o = _oracle_h(fmt, wg, wu, N, K, x)
    assert_bitwise(h.cpu().numpy(), h_o, "h")
    xq_o = oracle.quantize_act(h_o)
    assert_bitwise(xq_d.cpu().numpy()[: xq_o.size], xq_o, "Q8_0 of h")
    y64, A = oracle.matmul_f64(fdown, wd, K, N, xq_o, B)
    assert_tol(y.cpu().numpy(), y64, A, what="ffn down")
    assert_bitwise(y.cpu().numpy(), oracle.matmul_canon_f32(fdown, wd, K, N, xq_o, B), "ffn f32")


# (fmt, N, K, B): the paired launch quantises h itself for K = 2048 (8-wave
# workgroups), 896 and 1024 (4 waves), B <= 4; it falls back to a
# quantisation launch for K = 4096 (2 pairs per wave would need 16 waves),
# Q4_1 (format), K = 8192 (1 pair per wave), K = 4864 (3 rows per wave) and
# B > 4.
Q8_CASES = [
    (synth.Q4_K, 14336, 4096, 1), (synth.Q4_K, 96, 4096, 4), (synth.Q6_K, 64, 2048, 2),
    (synth.Q4_K, 4864, 2048, 1), (synth.Q4_K, 256, 512, 4),
    (synth.Q4_0, 4864, 896, 1), (synth.Q8_0, 160, 1024, 3), (synth.Q5_0, 32, 896, 4),
    (synth.Q4_1, 64, 896, 1), (synth.Q4_K, 64, 8192, 1), (synth.Q8_0, 96, 4864, 2),
    (synth.Q4_0, 128, 896, 5), (synth.Q4_K, 256, 4096, 16),
]


@pytest.mark.parametrize("fmt,N,K,B", Q8_CASES)
def test_gateup_swiglu_q8_leaves_h_quantised(g, fmt, N, K, B):
    """h bit-identical to qmv_launch_gateup_swiglu; hq holds exactly what
    quantize_act_q8_0(h) writes (the public blocks against the oracle, the
    staging through the down GEMV: y from hq equals y from h)."""
    wg, wu = _pair(fmt, N, K, 600 + N + K)
    fdown = synth.Q6_K if N % 256 == 0 else synth.Q4_0   # down: K outputs of N inputs
    wd, _ = synth.weights(fdown, K, N, 602, dscale=0.02)
    x = synth.activations(B, K, 603 + B)
    xd, wgd, wud = dev(x), dev(wg), dev(wu)
    print(f"gateup q8 fmt={fmt} N={N} K={K} B={B}", flush=True)
    h, hq = g.gateup_swiglu_q8(fmt, wgd, wud, N, K, x=xd)
    h1 = g.gateup_swiglu(fmt, wgd, wud, N, K, x=xd)
    torch.cuda.synchronize()
    h_o = _oracle_h(fmt, wg, wu, N, K, x)
    assert_bitwise(h.cpu().numpy(), h_o, "h")
    assert_bitwise(h1.cpu().numpy(), h_o, "h without hq")
    xq_o = oracle.quantize_act(h_o)
    assert_bitwise(hq.cpu().numpy()[: xq_o.size], xq_o, "Q8_0 blocks of h")
    wdd = dev(wd)
    y_q = g.matvec(fdown, wdd, K, N, xq=hq, B=B)
    y_h = g.matvec(fdown, wdd, K, N, x=h)
    torch.cuda.synchronize()
    assert_bitwise(y_q.cpu().numpy(), y_h.cpu().numpy(), "down from hq vs from h")
    assert_bitwise(y_q.cpu().numpy(), oracle.matmul_canon_f32(fdown, wd, K, N, xq_o, B),
                   "down f32 order")


@pytest.mark.parametrize("B", [1, 16])
def test_ffn_chain_8b_full_size(g, B):
    """The 8B-class FFN at full size as the benchmark runs it: Q4_K gate/up
    14336x4096 with the SwiGLU and the Q8_0 quantisation of h
    (qmv_launch_gateup_swiglu_q8), then the Q6_K down 4096x14336 on that
    quantisation.  h and its Q8_0 blocks bit-exact against the oracle chain
    (all 14336 rows of gate and up); down on 200 sampled rows bitwise in the
    f32 order and within tolerance of f64."""
    N, K = 14336, 4096
    wg, wu = _pair(synth.Q4_K, N, K, 700 + B)
    wd, _ = synth.weights(synth.Q6_K, K, N, 702 + B, dscale=0.02)
    x = synth.activations(B, K, 703 + B)
    print(f"ffn chain 8b full size B={B}", flush=True)
    h, hq = g.gateup_swiglu_q8(synth.Q4_K, dev(wg), dev(wu), N, K, x=dev(x))
    y = g.matvec(synth.Q6_K, dev(wd), K, N, xq=hq, B=B)
    torch.cuda.synchronize()
    h_o = _oracle_h(synth.Q4_K, wg, wu, N, K, x)
    assert_bitwise(h.cpu().numpy(), h_o, "h")
    xq_o = oracle.quantize_act(h_o)
    assert_bitwise(hq.cpu().numpy()[: xq_o.size], xq_o, "Q8_0 of h")
    rng = np.random.Generator(np.random.PCG64(704))
    rows = np.unique(np.concatenate([[0, K - 1], rng.choice(K, 200, replace=False)]))
    R = synth.row_bytes(synth.Q6_K, N)
    sub = np.ascontiguousarray(wd.reshape(K, R)[rows]).reshape(-1)
    got = np.ascontiguousarray(y.cpu().numpy()[:, rows])
    y64, A = oracle.matmul_f64(synth.Q6_K, sub, len(rows), N, xq_o, B)
    assert_tol(got, y64, A, what="down, full size")
    assert_bitwise(got, oracle.matmul_canon_f32(synth.Q6_K, sub, len(rows), N, xq_o, B), "down f32")


def test_ffn_chain_8b_full_size_q8k(g):
    """The same FFN at 16 rows on the Q8_K path as the benchmark runs it:
    qmv_launch_gateup_swiglu_q8k, then qmv_launch_q8k on h (quantised by
    the launch).  h bit-exact against the oracle's SwiGLU of its Q8_K-order
    gate and up (all rows); down on sampled rows bitwise in the Q8_K f32
    order and within tolerance of f64."""
    N, K, B = 14336, 4096, 16
    wg, wu = _pair(synth.Q4_K, N, K, 710)
    wd, _ = synth.weights(synth.Q6_K, K, N, 712, dscale=0.02)
    x = synth.activations(B, K, 713)
    print("ffn chain 8b full size q8k", flush=True)
    h = g.gateup_swiglu_q8k(synth.Q4_K, dev(wg), dev(wu), N, K, x=dev(x))
    y = g.matmul_q8k(synth.Q6_K, dev(wd), K, N, x=h)
    torch.cuda.synchronize()
    xq = oracle.quantize_act_q8k(x)
    gate = oracle.matmul_q8k_canon_f32(synth.Q4_K, wg, N, K, xq, B)
    up = oracle.matmul_q8k_canon_f32(synth.Q4_K, wu, N, K, xq, B)
    h_o = oracle.swiglu(gate, up)
    assert_bitwise(h.cpu().numpy(), h_o, "h")
    xq_h = oracle.quantize_act_q8k(h_o)
    rng = np.random.Generator(np.random.PCG64(714))
    rows = np.unique(np.concatenate([[0, K - 1], rng.choice(K, 200, replace=False)]))
    R = synth.row_bytes(synth.Q6_K, N)
    sub = np.ascontiguousarray(wd.reshape(K, R)[rows]).reshape(-1)
    got = np.ascontiguousarray(y.cpu().numpy()[:, rows])
    y64, A = oracle.matmul_q8k_f64(synth.Q6_K, sub, len(rows), N, xq_h, B)
    assert_tol(got, y64, A, what="down q8k, full size")
    assert_bitwise(got, oracle.matmul_q8k_canon_f32(synth.Q6_K, sub, len(rows), N, xq_h, B),
                   "down q8k f32")
