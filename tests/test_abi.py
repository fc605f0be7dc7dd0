"""CPU tests of the C-ABI library: it loads, exports every declared entry
point, and refuses bad arguments on the host before touching the GPU."""
import os
import re

import pytest

import gguf_quantized_matvec_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(g.LIB_PATH), reason="libqmv.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(g.EXPORTS), names
    L = g.lib()
    for n in names:
        assert hasattr(L, n), n


def test_act_bytes():
    # worked by hand from the layout in qmv_internal.h (every part 256-aligned):
    # 1 row, K = 896 (28 blocks): Q8_0 blocks 952 B; MFMA staging 14336 + 3*1792;
    # row-major staging 896 + 3*112; f16 staging 1792 + 56 -> 24576 bytes
    assert g.qmv_act_bytes(1, 896) == 24576
    # 17 rows, K = 64: blocks 1156 B; 2 groups -> 2048 + 3*256; rows 1088 + 3*136;
    # f16 rows 2176 + 68 -> 8704 bytes
    assert g.qmv_act_bytes(17, 64) == 8704
    for rows, K in [(0, 32), (1, 31), (1, 0), (1, 48), (-1, 32), (1, (1 << 20) + 32)]:
        assert g.qmv_act_bytes(rows, K) == 0


FAKE = 1 << 20  # a 16-byte aligned non-NULL address; never dereferenced


@pytest.mark.parametrize("args,code", [
    ((4, FAKE, 16, 32, FAKE, 1, FAKE, FAKE), -1),            # unknown type (GGUF 4, 5: retired)
    ((5, FAKE, 16, 32, FAKE, 1, FAKE, FAKE), -1),
    ((10, FAKE, 16, 256, FAKE, 1, FAKE, FAKE), -1),          # Q2_K: not accepted
    ((g.Q5_0, FAKE, 16, 48, FAKE, 1, FAKE, FAKE), -2),       # Q5_0 accepted: K % 32
    ((g.Q5_0, FAKE + 8, 16, 32, FAKE, 1, FAKE, FAKE), -3),   # Q5_0 accepted: w misaligned
    ((g.Q4_1, FAKE + 8, 16, 32, FAKE, 1, FAKE, FAKE), -3),   # Q4_1, Q5_1, Q8_1 accepted
    ((g.Q5_1, FAKE + 8, 16, 32, FAKE, 1, FAKE, FAKE), -3),
    ((g.Q8_1, FAKE, 16, 48, FAKE, 1, FAKE, FAKE), -2),
    ((g.Q8_0, FAKE, 16, 48, FAKE, 1, FAKE, FAKE), -2),       # K % 32
    ((g.Q4_K, FAKE, 16, 896, FAKE, 1, FAKE, FAKE), -2),      # K-quant K % 256
    ((g.Q6_K, FAKE, 16, 4864 + 32, FAKE, 1, FAKE, FAKE), -2),
    ((g.Q8_0, FAKE, 0, 32, FAKE, 1, FAKE, FAKE), -2),        # N
    ((g.Q8_0, FAKE, 16, 32, FAKE, 0, FAKE, FAKE), -2),       # B = 0
    ((g.Q8_0, FAKE, 16, 32, FAKE, 17, FAKE, FAKE), -2),      # B > 16: use qmm
    ((g.Q8_0, FAKE, 16, (1 << 20) + 32, FAKE, 1, FAKE, FAKE), -2),
    ((g.Q8_0, None, 16, 32, FAKE, 1, FAKE, FAKE), -3),       # w NULL
    ((g.Q8_0, FAKE + 8, 16, 32, FAKE, 1, FAKE, FAKE), -3),   # w misaligned
    ((g.Q8_0, FAKE, 16, 32, FAKE + 2, 1, FAKE, FAKE), -3),   # x not 4-byte aligned
    ((g.Q8_0, FAKE, 16, 32, FAKE, 1, None, FAKE), -3),       # xq NULL
    ((g.Q8_0, FAKE, 16, 32, FAKE, 1, FAKE + 8, FAKE), -3),   # xq misaligned
    ((g.Q8_0, FAKE, 16, 32, FAKE, 1, FAKE, FAKE + 2), -3),   # y misaligned
])
def test_qmv_refusals(args, code):
    assert g.lib().qmv_launch(*args, None) == code


def test_qmm_and_partials_refusals():
    L = g.lib()
    assert L.qmm_launch(g.Q4_0, FAKE, 16, 32, FAKE, 0, FAKE, FAKE, None) == -2
    assert L.qmm_launch(g.Q4_0, FAKE, 16, 32, FAKE, (1 << 24) + 1, FAKE, FAKE, None) == -2
    assert L.qmm_launch(g.Q4_K, FAKE, 16, 512 + 32, FAKE, 4, FAKE, FAKE, None) == -2
    assert L.qmv_partials_launch(g.Q8_0, FAKE, 16, 32, FAKE, 17, FAKE, None) == -2
    assert L.qmv_partials_launch(g.Q8_0, FAKE, 16, 32, None, 1, FAKE, None) == -3
    assert L.qmv_partials_launch(5, FAKE, 16, 32, FAKE, 1, FAKE, None) == -1
    assert L.quantize_act_q8_0(FAKE, FAKE, 1, 40, None) == -2
    assert L.quantize_act_q8_0(FAKE + 2, FAKE, 1, 32, None) == -3   # x 4-byte aligned at least
    assert L.quantize_act_q8_0(FAKE, FAKE + 4, 1, 32, None) == -3   # xq 16-byte aligned


def test_group_refusals():
    L = g.lib()
    G = g.Gemv
    ok = G(16, 1, 32, 16, None, 16)
    arr = (G * 1)(ok)
    assert L.qmv_launch_group(4, 1, arr, 1, None) == -1                    # type
    assert L.qmv_launch_group(8, 1, arr, 0, None) == -2                    # count
    assert L.qmv_launch_group(8, 1, arr, 9, None) == -2
    assert L.qmv_launch_group(8, 17, arr, 1, None) == -2                   # batch
    assert L.qmv_launch_group(8, 1, None, 1, None) == -3
    two = (G * 2)(ok, G(16, 1, 32, None, 16, 16))                          # x given for one only
    assert L.qmv_launch_group(8, 1, two, 2, None) == -3
    assert L.qmv_launch_group(8, 1, (G * 1)(G(16, 1, 32, None, None, 16)), 1, None) == -3
    assert L.qmv_launch_group(12, 1, (G * 1)(G(16, 1, 96, 16, None, 16)), 1, None) == -2
    # xq may be NULL only for a single fused launch (B <= 4); B = 5 quantises into xq
    assert L.qmv_launch_group(8, 5, (G * 1)(G(16, 1, 32, 16, None, 16)), 1, None) == -3
    # ... decided for the whole group: an entry whose K is too long for the
    # one-launch kernel (activation rows beyond its LDS) makes the group run
    # one GEMV after another, so the small entry's NULL xq is refused too
    mixed = (G * 2)(G(16, 1, 32, 16, None, 16), G(16, 1, 1 << 17, 16, 16, 16))
    assert L.qmv_launch_group(8, 1, mixed, 2, None) == -3
    # an x only 4-byte aligned is quantised by a launch of its own: needs xq
    assert L.qmv_launch_group(8, 1, (G * 1)(G(16, 1, 32, 20, None, 16)), 1, None) == -3
    assert L.qmv_launch_group(8, 1, (G * 1)(G(16, 1, 32, 18, 16, 16)), 1, None) == -3


def test_q8k_refusals_and_scratch_size():
    L = g.lib()
    # Q8_K blocks 292 B per 256 elements come first in the scratch
    assert g.qmv_act_bytes_q8k(3, 1024) >= 3 * 4 * 292
    for rows, K in [(0, 256), (1, 128), (1, 896), (1, (1 << 20) + 256), ((1 << 24) + 1, 256)]:
        assert g.qmv_act_bytes_q8k(rows, K) == 0
    assert L.quantize_act_q8_k(FAKE, FAKE, 1, 896, None) == -2
    assert L.quantize_act_q8_k(FAKE + 2, FAKE, 1, 256, None) == -3
    assert L.quantize_act_q8_k(FAKE, FAKE + 4, 1, 256, None) == -3
    for f, cap in ((L.qmv_launch_q8k, 16), (L.qmm_launch_q8k, 1 << 24)):
        assert f(g.Q4_0, FAKE, 16, 256, FAKE, 1, FAKE, FAKE, None) == -1   # K-quants only
        assert f(g.Q8_0, FAKE, 16, 256, FAKE, 1, FAKE, FAKE, None) == -1
        assert f(g.Q4_K, FAKE, 16, 896, FAKE, 1, FAKE, FAKE, None) == -2
        assert f(g.Q6_K, FAKE, 16, 256, FAKE, 0, FAKE, FAKE, None) == -2
        assert f(g.Q6_K, FAKE, 16, 256, FAKE, cap + 1, FAKE, FAKE, None) == -2
        assert f(g.Q6_K, FAKE + 8, 16, 256, FAKE, 1, FAKE, FAKE, None) == -3
        assert f(g.Q6_K, FAKE, 16, 256, FAKE + 2, 1, FAKE, FAKE, None) == -3
        assert f(g.Q6_K, FAKE, 16, 256, FAKE, 1, FAKE + 8, FAKE, None) == -3
        assert f(g.Q6_K, FAKE, 16, 256, FAKE, 1, FAKE, None, None) == -3
    assert L.qmv_partials_q8k_launch(g.Q4_K, FAKE, 16, 256, FAKE, 1, None, None) == -3
    assert L.qmv_partials_q8k_launch(g.Q4_0, FAKE, 16, 256, FAKE, 1, FAKE, None) == -1


def test_prepare_refusals_and_size():
    L = g.lib()
    # 16896-byte regions per 32-row tile and superblock
    assert g.qmv_prepared_bytes(g.Q4_K, 33, 512) == 2 * 2 * 16896
    assert g.qmv_prepared_bytes(g.Q6_K, 32, 256) == 16896
    for t, N, K in [(g.Q4_0, 32, 256), (g.Q8_0, 32, 256), (g.Q4_K, 32, 896), (g.Q6_K, 0, 256),
                    (g.Q6_K, 32, (1 << 20) + 256)]:
        assert g.qmv_prepared_bytes(t, N, K) == 0
    assert L.qmv_prepare(g.Q4_0, FAKE, 16, 256, FAKE, None) == -1
    assert L.qmv_prepare(g.Q4_K, FAKE, 16, 896, FAKE, None) == -2
    assert L.qmv_prepare(g.Q4_K, FAKE, 16, 256, None, None) == -3
    assert L.qmv_prepare(g.Q4_K, FAKE, 16, 256, FAKE + 8, None) == -3
    assert L.qmv_prepare(g.Q4_K, FAKE + 8, 16, 256, FAKE, None) == -3
    f = L.qmm_launch_q8k_prepared
    assert f(g.Q4_0, FAKE, 16, 256, FAKE, 1, FAKE, FAKE, None) == -1
    assert f(g.Q6_K, FAKE, 16, 4096 + 32, FAKE, 1, FAKE, FAKE, None) == -2
    assert f(g.Q6_K, FAKE, 16, 256, FAKE, 0, FAKE, FAKE, None) == -2
    assert f(g.Q6_K, FAKE, 16, 256, FAKE, (1 << 24) + 1, FAKE, FAKE, None) == -2
    assert f(g.Q6_K, FAKE + 8, 16, 256, FAKE, 1, FAKE, FAKE, None) == -3
    assert f(g.Q6_K, FAKE, 16, 256, FAKE, 1, None, FAKE, None) == -3
    assert f(g.Q6_K, FAKE, 16, 256, FAKE, 1, FAKE, FAKE + 2, None) == -3
    p = L.qmm_partials_q8k_prepared_launch
    assert p(g.Q4_K, FAKE, 16, 256, FAKE, 1, None, None) == -3
    assert p(g.Q4_1, FAKE, 16, 256, FAKE, 1, FAKE, None) == -1


def test_gateup_q8_refusals():
    f = g.lib().qmv_launch_gateup_swiglu_q8
    assert f(4, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, FAKE, FAKE, None) == -1
    assert f(g.Q4_K, FAKE, FAKE, 64 + 16, 4096, FAKE, 1, FAKE, FAKE, FAKE, None) == -2  # N % 32
    assert f(g.Q4_K, FAKE, FAKE, 16, 4096, FAKE, 1, FAKE, FAKE, FAKE, None) == -2       # N < 32
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE, 17, FAKE, FAKE, FAKE, None) == -2
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, FAKE, None, None) == -3       # hq NULL
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, FAKE, FAKE + 4, None) == -3   # hq align
    assert f(g.Q4_K, FAKE, FAKE + 8, 64, 4096, FAKE, 1, FAKE, FAKE, FAKE, None) == -3


def test_gateup_q8k_refusals():
    f = g.lib().qmv_launch_gateup_swiglu_q8k
    assert f(g.Q8_0, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, FAKE, None) == -1       # not a K-quant
    assert f(4, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, FAKE, None) == -1
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096 + 32, FAKE, 1, FAKE, FAKE, None) == -2  # K % 256
    assert f(g.Q4_K, FAKE, FAKE, 0, 4096, FAKE, 1, FAKE, FAKE, None) == -2
    assert f(g.Q6_K, FAKE, FAKE, 64, 4096, FAKE, 0, FAKE, FAKE, None) == -2
    assert f(g.Q6_K, FAKE, FAKE, 64, 4096, FAKE, 17, FAKE, FAKE, None) == -2
    assert f(g.Q4_K, FAKE, FAKE + 8, 64, 4096, FAKE, 1, FAKE, FAKE, None) == -3   # w_up align
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE + 2, 1, FAKE, FAKE, None) == -3   # x align
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE + 4, FAKE, None) == -3   # xq align
    assert f(g.Q4_K, FAKE, FAKE, 64, 4096, FAKE, 1, FAKE, None, None) == -3       # h NULL


def test_group_q8k_refusals():
    L, G = g.lib(), g.Gemv
    ok = (G * 2)(G(FAKE, 16, 1024, None, FAKE, FAKE), G(FAKE, 32, 1024, None, FAKE, FAKE))
    assert L.qmv_launch_group_q8k(g.Q8_0, 16, ok, 2, None) == -1             # not a K-quant
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, None, 2, None) == -3
    assert L.qmv_launch_group_q8k(g.Q4_K, 17, ok, 2, None) == -2
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, ok, 0, None) == -2
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, ok, 9, None) == -2
    bad_k = (G * 1)(G(FAKE, 16, 1024 + 32, None, FAKE, FAKE))
    assert L.qmv_launch_group_q8k(g.Q6_K, 16, bad_k, 1, None) == -2          # K % 256
    no_xq = (G * 1)(G(FAKE, 16, 1024, FAKE, None, FAKE))
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, no_xq, 1, None) == -3          # xq required
    mixed = (G * 2)(G(FAKE, 16, 1024, FAKE, FAKE, FAKE), G(FAKE, 16, 1024, None, FAKE, FAKE))
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, mixed, 2, None) == -3          # x all or none
    unal = (G * 1)(G(FAKE, 16, 1024, None, FAKE + 8, FAKE))
    assert L.qmv_launch_group_q8k(g.Q4_K, 16, unal, 1, None) == -3


def test_noalloc_refusals():
    L = g.lib()
    # the fixed scratch admits every K <= 65536 at B = 16 (and no more at K = 2^17)
    assert g.qmv_act_bytes(16, 65536) <= 8 << 20 < g.qmv_act_bytes(16, 1 << 17)
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 1 << 17, FAKE, 16, FAKE, None) == -6
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 1 << 19, FAKE, 1, FAKE, None) == -6
    assert L.qmv_launch_noalloc(4, FAKE, 16, 32, FAKE, 1, FAKE, None) == -1
    assert L.qmv_launch_noalloc(g.Q4_K, FAKE, 16, 896, FAKE, 1, FAKE, None) == -2
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 32, FAKE, 0, FAKE, None) == -2
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 32, FAKE, 17, FAKE, None) == -2
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 32, None, 1, FAKE, None) == -3   # x required
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 32, FAKE + 2, 1, FAKE, None) == -3
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE, 16, 32, FAKE, 1, None, None) == -3
    assert L.qmv_launch_noalloc(g.Q8_0, FAKE + 8, 16, 32, FAKE, 1, FAKE, None) == -3
    assert "QMV_NOALLOC_MAX_ACT_BYTES" in g.strerror(-6)


def test_gateup_refusals_and_scratch_size():
    L = g.lib()
    # the activation scratch of qmv_launch (24576 B at 1 x 896), then two
    # 256-aligned [B][N] f32 products: 4864 * 4 = 19456 B each
    assert g.qmv_gateup_act_bytes(1, 4864, 896) == 24576 + 2 * 19456
    assert g.qmv_gateup_act_bytes(17, 16, 32) == 0 and g.qmv_gateup_act_bytes(1, 0, 32) == 0
    f = L.qmv_launch_gateup_swiglu
    assert f(4, FAKE, FAKE, 16, 32, FAKE, 1, FAKE, FAKE, None) == -1
    assert f(g.Q4_K, FAKE, FAKE, 16, 896, FAKE, 1, FAKE, FAKE, None) == -2
    assert f(g.Q4_0, FAKE, None, 16, 32, FAKE, 1, FAKE, FAKE, None) == -3   # up blob NULL
    assert f(g.Q4_0, FAKE, FAKE + 8, 16, 32, FAKE, 1, FAKE, FAKE, None) == -3
    assert f(g.Q4_0, FAKE, FAKE, 16, 32, FAKE, 17, FAKE, FAKE, None) == -2
    assert f(g.Q4_0, FAKE, FAKE, 16, 32, FAKE, 1, None, FAKE, None) == -3
    assert f(g.Q4_0, FAKE, FAKE, 16, 32, FAKE, 1, FAKE, FAKE + 2, None) == -3
    assert f(g.Q4_0, FAKE, FAKE, 16, 32, FAKE + 2, 1, FAKE, FAKE, None) == -3


def test_strerror_names_what_works():
    assert all(t in g.strerror(-1) for t in ("Q4_0", "Q4_1", "Q5_0", "Q5_1", "Q8_0", "Q8_1",
                                              "Q4_K", "Q6_K"))
    assert "K % 256" in g.strerror(-2) and "qmm_launch" in g.strerror(-2)
    assert "gfx950" in g.strerror(-5)
    assert g.strerror(0) == "ok" and "unknown" in g.strerror(-99)
    with pytest.raises(g.QmvError) as e:
        g.qmv_launch(4, FAKE, 16, 32, FAKE, 1, FAKE, FAKE, 0)
    assert e.value.code == -1


def test_ceilings_library_exports_its_header():
    import ctypes
    lib_path = os.path.join(ROOT, "gguf_quantized_matvec_amd", "libqmv_ceilings.so")
    if not os.path.exists(lib_path):
        pytest.skip("libqmv_ceilings.so not built")
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qmv_ceilings.h")).read(),
                 flags=re.S)
    names = set(re.findall(r"^\s*int\s+([a-z_0-9]+)\s*\(", src, re.M))
    assert names == {"qmv_ceil_stream_read", "qmv_ceil_stream_read_nt", "qmv_ceil_mfma_i8",
                     "qmv_ceil_mfma_f16", "qmv_ceil_epilogue", "qmv_ceil_chunk_read"}
    L = ctypes.CDLL(lib_path)
    for n in names:
        assert hasattr(L, n), n
    # host-side refusals (nothing is launched): sizes that are not whole slices
    L.qmv_ceil_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_void_p]
    assert L.qmv_ceil_stream_read(FAKE, 1000, FAKE, None) == -2
    assert L.qmv_ceil_stream_read(None, 65536, FAKE, None) == -2
    L.qmv_ceil_stream_read_nt.argtypes = L.qmv_ceil_stream_read.argtypes
    assert L.qmv_ceil_stream_read_nt(FAKE, 32768 + 16384, FAKE, None) == -2
    assert L.qmv_ceil_stream_read_nt(FAKE + 4, 32768, FAKE, None) == -2
    I64 = ctypes.c_int64
    L.qmv_ceil_chunk_read.argtypes = [ctypes.c_void_p, I64, I64, I64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    assert L.qmv_ceil_chunk_read(FAKE, 16, 16, 160, FAKE, None) == -2   # chunk size
    assert L.qmv_ceil_chunk_read(FAKE, 16, 65, 144, FAKE, None) == -2   # > 64 chunks a row
    assert L.qmv_ceil_chunk_read(FAKE, 0, 16, 144, FAKE, None) == -2    # no rows
    assert L.qmv_ceil_chunk_read(FAKE + 8, 16, 16, 144, FAKE, None) == -2
    assert L.qmv_ceil_chunk_read(FAKE, 16, 16, 272, None, None) == -2
