"""qmv_launch_noalloc (the decode GEMV whose activation scratch is a fixed
array inside the library) against qmv_launch with a caller-supplied xq,
through the C-ABI: bit-identical y on two calls in a row, the second with a
smaller input, and also against the CPU oracle's tolerance and f32 order."""
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


def _case(g, fmt, N, K, B, seed):
    blob, _ = synth.weights(fmt, N, K, seed)
    x = synth.activations(B, K, seed + 1)
    w = torch.from_numpy(blob).cuda()
    xd = torch.from_numpy(x).cuda()
    s = torch.cuda.current_stream().cuda_stream
    y_ref = torch.empty(B, N, dtype=torch.float32, device="cuda")
    xq = g.act_buffer(B, K)
    g.qmv_launch(fmt, w.data_ptr(), N, K, xd.data_ptr(), B, xq.data_ptr(), y_ref.data_ptr(), s)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    print(f"noalloc case fmt={fmt} N={N} K={K} B={B}", flush=True)
    g.qmv_launch_noalloc(fmt, w.data_ptr(), N, K, xd.data_ptr(), B, y.data_ptr(), s)
    torch.cuda.synchronize()
    return blob, x, y_ref.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # the MFMA path (B = 16, long K) then the fused lane-per-chunk path (B = 1)
    ((synth.Q4_K, 4864, 4096, 16), (synth.Q4_0, 896, 896, 1)),
    # the lane-per-chunk path at B = 4 with a long row, then a shorter B = 3
    ((synth.Q6_K, 1000, 14336, 4), (synth.Q8_0, 300, 1024, 3)),
])
def test_noalloc_matches_qmv_launch(g, first, second):
    for fmt, N, K, B in (first, second):
        blob, x, y_ref, y = _case(g, fmt, N, K, B, 40 + N)
        assert_bitwise(y, y_ref, f"noalloc vs qmv_launch {synth.NAMES[fmt]} {N}x{K} B={B}")
        xq = oracle.quantize_act(x)
        y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
        assert_tol(y, y64, A, what="noalloc vs oracle")
        assert_bitwise(y, oracle.matmul_canon_f32(fmt, blob, N, K, xq, B), "noalloc f32 order")
