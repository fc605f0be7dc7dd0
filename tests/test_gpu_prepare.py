"""GPU parity of the load-time repack for the Q8_K prefill GEMM:

* qmv_prepare's bytes against the oracle's repack, byte for byte (ragged
  row tiles, several superblocks, scales at the edges of their ranges);
* the exact superblock partials of the GEMM on repacked weights against the
  oracle's partials of the GGUF blob, for every tile shape the launch picks
  (32, 64 and 128 activation rows), including partials above 2^24;
* y bit-identical to qmm_launch_q8k on the GGUF blob and to the oracle's
  replay of the Q8_K f32 order; at the 8B-class sizes (M = 2048) over the
  whole output against the direct GEMM.
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


FMTS = [synth.Q4_K, synth.Q6_K]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(1, 256), (32, 512), (45, 768), (300, 4096 + 256)])
def test_prepare_bytes_equal_the_oracle(g, fmt, N, K):
    blob, _ = synth.weights(fmt, N, K, 3000 + N + K, s_range=(-128, 127))
    print(f"prepare fmt={fmt} N={N} K={K}", flush=True)
    wp = host(g.prepare(fmt, dev(blob), N, K))
    assert_bitwise(wp, oracle.prepare_q8k(fmt, blob, N, K), "repacked bytes")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(37, 256), (130, 1024), (300, 4096 + 256)])
@pytest.mark.parametrize("M", [1, 5, 33, 70, 200])
def test_partials_on_repacked_weights(g, fmt, N, K, M):
    blob, _ = synth.weights(fmt, N, K, 3100 + N + M, s_range=(-128, 127))
    x = synth.activations(M, K, 3101 + K)
    print(f"prepared partials fmt={fmt} N={N} K={K} M={M}", flush=True)
    wp = g.prepare(fmt, dev(blob), N, K)
    P = host(g.partials_q8k_prepared(fmt, wp, N, K, g.quantize_q8k(dev(x)), M))
    assert_bitwise(P, oracle.partials_q8k(fmt, blob, N, K, oracle.quantize_act_q8k(x), M),
                   "prepared partials")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [3, 40])
def test_repacked_partials_above_2_24(g, fmt, M):
    N, K = 64, 1024
    f = synth.draw_fields(fmt, N, K, 3200, s_range=(-128, 127))
    if fmt == synth.Q4_K:
        f["sc"] = np.maximum(f["sc"], 56)
        f["q"] = np.maximum(f["q"], 12)
    else:
        f["s"] = np.where(np.abs(f["s"]) < 100, np.int8(-128), f["s"]).astype(np.int8)
        f["q"] = np.minimum(f["q"], 3)
    blob = synth.encode(f)
    x = (np.abs(synth.activations(M, K, 3201)) * 0.2 + 4).astype(np.float32)
    xq_o = oracle.quantize_act_q8k(x)
    P_o = oracle.partials_q8k(fmt, blob, N, K, xq_o, M)
    assert np.abs(P_o[..., 0] if fmt == synth.Q4_K else P_o).max() > 2 ** 24
    print(f"prepared large partials fmt={fmt} M={M}", flush=True)
    wp = g.prepare(fmt, dev(blob), N, K)
    xd = dev(x)
    assert_bitwise(host(g.partials_q8k_prepared(fmt, wp, N, K, g.quantize_q8k(xd), M)), P_o,
                   "prepared partials > 2^24")
    assert_bitwise(host(g.matmul_q8k_prepared(fmt, wp, N, K, x=xd)),
                   oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq_o, M), "y")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K,M", [(45, 1024, 1), (96, 4352, 3), (129, 1024, 17),
                                   (250, 2048, 64), (130, 512, 65), (70, 4096, 200)])
def test_repacked_y_against_oracle_and_direct(g, fmt, N, K, M):
    blob, _ = synth.weights(fmt, N, K, 3300 + N, s_range=(-128, 127))
    x = synth.activations(M, K, 3301 + M)
    print(f"prepared y fmt={fmt} N={N} K={K} M={M}", flush=True)
    w, xd = dev(blob), dev(x)
    y = host(g.matmul_q8k_prepared(fmt, g.prepare(fmt, w, N, K), N, K, x=xd))
    xq = oracle.quantize_act_q8k(x)
    y64, A = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, M)
    assert_tol(y, y64, A, what="repacked vs f64")
    assert_bitwise(y, oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq, M), "repacked f32 order")
    assert_bitwise(y, host(g.matmul_q8k(fmt, w, N, K, x=xd)), "repacked vs direct")


@pytest.mark.parametrize("fmt", FMTS)
def test_repacked_wide_grid_ragged(g, fmt):
    """A grid of 64-row tiles with ragged M and N (130 tokens, 32805 rows):
    sampled rows against the oracle, all of y against the direct GEMM (there
    on 128-row tiles), partials on sampled rows."""
    N, K, M = 32805, 512, 130
    blob, _ = synth.weights(fmt, N, K, 3400 + fmt, s_range=(-128, 127))
    x = synth.activations(M, K, 3401)
    w, xd = dev(blob), dev(x)
    print(f"prepared wide ragged fmt={fmt}", flush=True)
    wp = g.prepare(fmt, w, N, K)
    y = host(g.matmul_q8k_prepared(fmt, wp, N, K, x=xd))
    assert_bitwise(y, host(g.matmul_q8k(fmt, w, N, K, x=xd)), "repacked vs direct")
    rng = np.random.Generator(np.random.PCG64(3402))
    rows = np.unique(np.concatenate([[0, 31, 32, 127, 128, N - 38, N - 1],
                                     rng.choice(N, 300, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xq = oracle.quantize_act_q8k(x)
    assert_bitwise(np.ascontiguousarray(y[:, rows]),
                   oracle.matmul_q8k_canon_f32(fmt, sub, len(rows), K, xq, M), "f32 order")
    P = host(g.partials_q8k_prepared(fmt, wp, N, K, g.quantize_q8k(xd), M))
    assert_bitwise(np.ascontiguousarray(P[:, rows]),
                   oracle.partials_q8k(fmt, sub, len(rows), K, xq, M), "partials")


@pytest.mark.parametrize("fmt,N,K", [(synth.Q4_K, 14336, 4096), (synth.Q6_K, 4096, 14336),
                                     (synth.Q4_K, 1024, 4096), (synth.Q4_K, 4096, 4096)])
def test_repacked_8b_class_full_size(g, fmt, N, K):
    """The 8B-class shapes at 2048 tokens in the benchmark's launch
    configuration: all of y against the direct GEMM (itself checked against
    the oracle at this size), sampled tokens x rows against the oracle."""
    M = 2048
    idx = {(synth.Q4_K, 4096): 0, (synth.Q4_K, 1024): 1, (synth.Q4_K, 14336): 2,
           (synth.Q6_K, 4096): 3}[(fmt, N)]
    blob, _ = synth.weights(fmt, N, K, synth.seed_for(4, idx), dscale=0.02)
    x = synth.activations(M, K, synth.act_seed_for(4, M))
    w, xd = dev(blob), dev(x)
    print(f"prepared full size fmt={fmt} N={N} K={K}", flush=True)
    y = host(g.matmul_q8k_prepared(fmt, g.prepare(fmt, w, N, K), N, K, x=xd))
    assert_bitwise(y, host(g.matmul_q8k(fmt, w, N, K, x=xd)), "repacked vs direct, full size")
    rng = np.random.Generator(np.random.PCG64(3500 + N))
    toks = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.choice(M, 6, replace=False)]))
    rows = np.unique(np.concatenate([[0, 31, 32, N - 1], rng.choice(N, 100, replace=False)]))
    R = synth.row_bytes(fmt, K)
    sub = np.ascontiguousarray(blob.reshape(N, R)[rows]).reshape(-1)
    xq = oracle.quantize_act_q8k(x[toks])
    assert_bitwise(np.ascontiguousarray(y[toks][:, rows]),
                   oracle.matmul_q8k_canon_f32(fmt, sub, len(rows), K, xq, len(toks)),
                   "full size f32 order")
