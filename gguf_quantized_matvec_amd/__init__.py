"""Python binding of libqmv.so (include/qmv.h): the same entry points, argument
marshalling only.  Every step of the multiply runs in the HIP kernels.

Raw pointers and sizes go straight through; the torch-tensor helpers below
only turn tensors into (pointer, stream) and check shapes/dtypes.  There is no
CPU fallback: if the library is missing or the device is not gfx950 the calls
raise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmv.so")

Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1, Q4_K, Q6_K = 2, 3, 6, 7, 8, 9, 12, 14
TYPES = {"Q4_0": Q4_0, "Q4_1": Q4_1, "Q5_0": Q5_0, "Q5_1": Q5_1, "Q8_0": Q8_0, "Q8_1": Q8_1,
         "Q4_K": Q4_K, "Q6_K": Q6_K}
BLOCK = {Q8_0: (32, 34), Q4_0: (32, 18), Q5_0: (32, 22), Q4_1: (32, 20), Q5_1: (32, 24),
         Q8_1: (32, 36), Q4_K: (256, 144), Q6_K: (256, 210)}
EXPORTS = ("qmv_act_bytes", "quantize_act_q8_0", "qmv_launch", "qmv_launch_group", "qmm_launch",
           "qmv_partials_launch", "qmm_partials_launch", "qmv_launch_noalloc", "qmv_gateup_act_bytes",
           "qmv_launch_gateup_swiglu", "qmv_launch_gateup_swiglu_q8", "qmv_act_bytes_q8k", "quantize_act_q8_k", "qmv_launch_q8k",
           "qmv_launch_gateup_swiglu_q8k", "qmv_launch_group_q8k", "qmm_launch_q8k", "qmv_partials_q8k_launch", "qmv_prepared_bytes", "qmv_prepare",
           "qmm_launch_q8k_prepared", "qmm_partials_q8k_prepared_launch", "qmv_strerror")
MAX_BATCH = 16
MAX_GROUP = 8


class Gemv(ctypes.Structure):
    """struct qmv_gemv: one GEMV of qmv_launch_group (pointers as integers)."""
    _fields_ = [("w", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("x", ctypes.c_void_p), ("xq", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class QmvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} (status {code})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libqmv.so (built in-tree by build.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run python -m gguf_quantized_matvec_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qmv_act_bytes.argtypes = [I64, I64]
        L.qmv_act_bytes.restype = ctypes.c_size_t
        L.quantize_act_q8_0.argtypes = [P, P, I64, I64, P]
        L.qmv_launch.argtypes = [I, P, I64, I64, P, I64, P, P, P]
        L.qmm_launch.argtypes = [I, P, I64, I64, P, I64, P, P, P]
        L.qmv_launch_group.argtypes = [I, I64, ctypes.POINTER(Gemv), I, P]
        L.qmv_partials_launch.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.qmv_launch_noalloc.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.qmm_partials_launch.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.qmv_act_bytes_q8k.argtypes = [I64, I64]
        L.qmv_act_bytes_q8k.restype = ctypes.c_size_t
        L.quantize_act_q8_k.argtypes = [P, P, I64, I64, P]
        L.qmv_launch_q8k.argtypes = [I, P, I64, I64, P, I64, P, P, P]
        L.qmm_launch_q8k.argtypes = [I, P, I64, I64, P, I64, P, P, P]
        L.qmv_partials_q8k_launch.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.qmv_prepared_bytes.argtypes = [I, I64, I64]
        L.qmv_prepared_bytes.restype = ctypes.c_size_t
        L.qmv_prepare.argtypes = [I, P, I64, I64, P, P]
        L.qmm_launch_q8k_prepared.argtypes = [I, P, I64, I64, P, I64, P, P, P]
        L.qmm_partials_q8k_prepared_launch.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.qmv_gateup_act_bytes.argtypes = [I64, I64, I64]
        L.qmv_gateup_act_bytes.restype = ctypes.c_size_t
        L.qmv_launch_gateup_swiglu.argtypes = [I, P, P, I64, I64, P, I64, P, P, P]
        L.qmv_launch_gateup_swiglu_q8.argtypes = [I, P, P, I64, I64, P, I64, P, P, P, P]
        L.qmv_launch_gateup_swiglu_q8k.argtypes = [I, P, P, I64, I64, P, I64, P, P, P]
        L.qmv_launch_group_q8k.argtypes = [I, I64, ctypes.POINTER(Gemv), I, P]
        for f in ("quantize_act_q8_0", "qmv_launch", "qmv_launch_group", "qmm_launch",
                  "qmv_partials_launch", "qmm_partials_launch", "qmv_launch_noalloc",
                  "qmv_launch_gateup_swiglu", "qmv_launch_gateup_swiglu_q8", "quantize_act_q8_k", "qmv_launch_q8k",
                  "qmv_launch_gateup_swiglu_q8k", "qmv_launch_group_q8k", "qmm_launch_q8k", "qmv_partials_q8k_launch", "qmv_prepare",
                  "qmm_launch_q8k_prepared", "qmm_partials_q8k_prepared_launch"):
            getattr(L, f).restype = I
        L.qmv_strerror.argtypes = [I]
        L.qmv_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().qmv_strerror(int(code)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise QmvError(rc, what)


# ---------------------------------------------------------------- raw C-ABI --

def qmv_act_bytes(rows: int, K: int) -> int:
    return int(lib().qmv_act_bytes(rows, K))


def quantize_act_q8_0(x, xq: int, rows: int, K: int, stream: int = 0) -> None:
    _check(lib().quantize_act_q8_0(x, xq, rows, K, stream), "quantize_act_q8_0")


def qmv_launch(type: int, w: int, N: int, K: int, x, B: int, xq: int, y: int,
               stream: int = 0) -> None:
    _check(lib().qmv_launch(type, w, N, K, x, B, xq, y, stream), "qmv_launch")


def qmv_launch_group(type: int, B: int, gemvs, stream: int = 0) -> None:
    """gemvs: a sequence of Gemv (or of (w, N, K, x, xq, y) tuples)."""
    arr = (Gemv * len(gemvs))(*[gv if isinstance(gv, Gemv) else Gemv(*gv) for gv in gemvs])
    _check(lib().qmv_launch_group(type, B, arr, len(gemvs), stream), "qmv_launch_group")


def qmv_launch_group_q8k(type: int, B: int, gemvs, stream: int = 0) -> None:
    """gemvs: a sequence of Gemv (or of (w, N, K, x, xq, y) tuples), Q8_K path."""
    arr = (Gemv * len(gemvs))(*[gv if isinstance(gv, Gemv) else Gemv(*gv) for gv in gemvs])
    _check(lib().qmv_launch_group_q8k(type, B, arr, len(gemvs), stream), "qmv_launch_group_q8k")


def qmm_launch(type: int, w: int, N: int, K: int, x, M: int, xq: int, y: int,
               stream: int = 0) -> None:
    _check(lib().qmm_launch(type, w, N, K, x, M, xq, y, stream), "qmm_launch")


def qmv_partials_launch(type: int, w: int, N: int, K: int, xq: int, B: int, P: int,
                        stream: int = 0) -> None:
    _check(lib().qmv_partials_launch(type, w, N, K, xq, B, P, stream), "qmv_partials_launch")


def qmm_partials_launch(type: int, w: int, N: int, K: int, xq: int, M: int, P: int,
                        stream: int = 0) -> None:
    _check(lib().qmm_partials_launch(type, w, N, K, xq, M, P, stream), "qmm_partials_launch")


def qmv_launch_noalloc(type: int, w: int, N: int, K: int, x: int, B: int, y: int,
                       stream: int = 0) -> None:
    _check(lib().qmv_launch_noalloc(type, w, N, K, x, B, y, stream), "qmv_launch_noalloc")


def qmv_gateup_act_bytes(B: int, N: int, K: int) -> int:
    return int(lib().qmv_gateup_act_bytes(B, N, K))


def qmv_launch_gateup_swiglu(type: int, w_gate: int, w_up: int, N: int, K: int, x, B: int,
                             xq: int, h: int, stream: int = 0) -> None:
    _check(lib().qmv_launch_gateup_swiglu(type, w_gate, w_up, N, K, x, B, xq, h, stream),
           "qmv_launch_gateup_swiglu")


def qmv_launch_gateup_swiglu_q8(type: int, w_gate: int, w_up: int, N: int, K: int, x, B: int,
                                xq: int, h: int, hq: int, stream: int = 0) -> None:
    _check(lib().qmv_launch_gateup_swiglu_q8(type, w_gate, w_up, N, K, x, B, xq, h, hq, stream),
           "qmv_launch_gateup_swiglu_q8")


def qmv_launch_gateup_swiglu_q8k(type: int, w_gate: int, w_up: int, N: int, K: int, x, B: int,
                                 xq: int, h: int, stream: int = 0) -> None:
    _check(lib().qmv_launch_gateup_swiglu_q8k(type, w_gate, w_up, N, K, x, B, xq, h, stream),
           "qmv_launch_gateup_swiglu_q8k")


def qmv_act_bytes_q8k(rows: int, K: int) -> int:
    return int(lib().qmv_act_bytes_q8k(rows, K))


def quantize_act_q8_k(x, xq: int, rows: int, K: int, stream: int = 0) -> None:
    _check(lib().quantize_act_q8_k(x, xq, rows, K, stream), "quantize_act_q8_k")


def qmv_launch_q8k(type: int, w: int, N: int, K: int, x, B: int, xq: int, y: int,
                   stream: int = 0) -> None:
    _check(lib().qmv_launch_q8k(type, w, N, K, x, B, xq, y, stream), "qmv_launch_q8k")


def qmm_launch_q8k(type: int, w: int, N: int, K: int, x, M: int, xq: int, y: int,
                   stream: int = 0) -> None:
    _check(lib().qmm_launch_q8k(type, w, N, K, x, M, xq, y, stream), "qmm_launch_q8k")


def qmv_partials_q8k_launch(type: int, w: int, N: int, K: int, xq: int, M: int, P: int,
                            stream: int = 0) -> None:
    _check(lib().qmv_partials_q8k_launch(type, w, N, K, xq, M, P, stream),
           "qmv_partials_q8k_launch")


def qmv_prepared_bytes(type: int, N: int, K: int) -> int:
    return int(lib().qmv_prepared_bytes(type, N, K))


def qmv_prepare(type: int, w: int, N: int, K: int, wp: int, stream: int = 0) -> None:
    _check(lib().qmv_prepare(type, w, N, K, wp, stream), "qmv_prepare")


def qmm_launch_q8k_prepared(type: int, wp: int, N: int, K: int, x, M: int, xq: int, y: int,
                            stream: int = 0) -> None:
    _check(lib().qmm_launch_q8k_prepared(type, wp, N, K, x, M, xq, y, stream),
           "qmm_launch_q8k_prepared")


def qmm_partials_q8k_prepared_launch(type: int, wp: int, N: int, K: int, xq: int, M: int,
                                     P: int, stream: int = 0) -> None:
    _check(lib().qmm_partials_q8k_prepared_launch(type, wp, N, K, xq, M, P, stream),
           "qmm_partials_q8k_prepared_launch")


def qmv_strerror(code: int) -> str:
    return strerror(code)


# ------------------------------------------------------------ torch helpers --

def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t, dtype, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t.data_ptr()


def row_bytes(type: int, K: int) -> int:
    qk, nbytes = BLOCK[type]
    return (K // qk) * nbytes


def act_buffer(rows: int, K: int, device="cuda"):
    """Allocate an activation scratch tensor of qmv_act_bytes(rows, K) bytes."""
    import torch
    n = qmv_act_bytes(rows, K)
    if n == 0:
        raise ValueError(f"bad activation shape rows={rows} K={K}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def quantize(x, xq=None, stream=None, rows=None, K=None):
    """x: f32 [rows, K] device tensor -> xq scratch (Q8_0 blocks first).
    x None: re-stage the Q8_0 blocks already in xq (rows, K given)."""
    import torch
    if x is not None:
        rows, K = x.shape
    if xq is None:
        xq = act_buffer(rows, K, x.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    quantize_act_q8_0(xp, _dev(xq, torch.uint8, "xq"), rows, K, _stream(stream))
    return xq


def matvec(type: int, w, N: int, K: int, x=None, xq=None, B=None, y=None, stream=None):
    """Decode GEMV: y [B, N] f32 = x [B, K] @ W^T, B <= 16 (x None: reuse xq)."""
    import torch
    if x is not None:
        B = x.shape[0]
    if xq is None:
        xq = act_buffer(B, K, w.device)
    if y is None:
        y = torch.empty(B, N, dtype=torch.float32, device=w.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmv_launch(type, _dev(w, torch.uint8, "w"), N, K, xp, B, _dev(xq, torch.uint8, "xq"),
               _dev(y, torch.float32, "y"), _stream(stream))
    return y


def matvec_group(type: int, items, stream=None):
    """Grouped decode GEMVs: items are dicts with w, N, K and x (f32 [B, K])
    or xq (staged), optional xq / y.  Returns the list of y [B, N]."""
    import torch
    B = None
    descs, ys = [], []
    for it in items:
        x, xq = it.get("x"), it.get("xq")
        b = x.shape[0] if x is not None else it["B"]
        if B is None:
            B = b
        elif b != B:
            raise ValueError("all GEMVs of a group take the same number of rows")
        w = it["w"]
        y = it.get("y")
        if y is None:
            y = torch.empty(B, it["N"], dtype=torch.float32, device=w.device)
        xp = _dev(x, torch.float32, "x") if x is not None else None
        qp = _dev(xq, torch.uint8, "xq") if xq is not None else None
        descs.append(Gemv(_dev(w, torch.uint8, "w"), it["N"], it["K"], xp, qp,
                          _dev(y, torch.float32, "y")))
        ys.append(y)
    qmv_launch_group(type, B, descs, _stream(stream))
    return ys


def gateup_swiglu(type: int, w_gate, w_up, N: int, K: int, x=None, xq=None, B=None, h=None,
                  stream=None):
    """h [B, N] f32 = silu(x @ Wg^T) * (x @ Wu^T) (x None: use the staged xq)."""
    import torch
    if x is not None:
        B = x.shape[0]
    if xq is None:
        n = qmv_gateup_act_bytes(B, N, K)
        if n == 0:
            raise ValueError(f"bad shape B={B} N={N} K={K}")
        xq = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    if h is None:
        h = torch.empty(B, N, dtype=torch.float32, device=w_gate.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmv_launch_gateup_swiglu(type, _dev(w_gate, torch.uint8, "w_gate"),
                             _dev(w_up, torch.uint8, "w_up"), N, K, xp, B,
                             _dev(xq, torch.uint8, "xq"), _dev(h, torch.float32, "h"),
                             _stream(stream))
    return h


def gateup_swiglu_q8(type: int, w_gate, w_up, N: int, K: int, x=None, xq=None, B=None, h=None,
                     hq=None, stream=None):
    """(h [B, N] f32, hq) with hq the Q8_0 scratch of h for the down GEMV."""
    import torch
    if x is not None:
        B = x.shape[0]
    if xq is None:
        n = qmv_gateup_act_bytes(B, N, K)
        if n == 0:
            raise ValueError(f"bad shape B={B} N={N} K={K}")
        xq = torch.empty(n, dtype=torch.uint8, device=w_gate.device)
    if h is None:
        h = torch.empty(B, N, dtype=torch.float32, device=w_gate.device)
    if hq is None:
        hq = act_buffer(B, N, w_gate.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmv_launch_gateup_swiglu_q8(type, _dev(w_gate, torch.uint8, "w_gate"),
                                _dev(w_up, torch.uint8, "w_up"), N, K, xp, B,
                                _dev(xq, torch.uint8, "xq"), _dev(h, torch.float32, "h"),
                                _dev(hq, torch.uint8, "hq"), _stream(stream))
    return h, hq


def matmul(type: int, w, N: int, K: int, x=None, xq=None, M=None, y=None, stream=None):
    """Prefill GEMM: y [M, N] f32 = x [M, K] @ W^T."""
    import torch
    if x is not None:
        M = x.shape[0]
    if xq is None:
        xq = act_buffer(M, K, w.device)
    if y is None:
        y = torch.empty(M, N, dtype=torch.float32, device=w.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmm_launch(type, _dev(w, torch.uint8, "w"), N, K, xp, M, _dev(xq, torch.uint8, "xq"),
               _dev(y, torch.float32, "y"), _stream(stream))
    return y


def partials(type: int, w, N: int, K: int, xq, B: int, P=None, stream=None, gemm=False):
    """Test hook: int32 per-block partials [B, N, K/32] (Q4_K, Q4_1, Q5_1: [B, N, K/32, 2])
    of the kernel that qmv_launch (gemm: qmm_launch) runs for B rows."""
    import torch
    shape = (B, N, K // 32, 2) if type in (Q4_K, Q4_1, Q5_1) else (B, N, K // 32)
    if P is None:
        P = torch.empty(shape, dtype=torch.int32, device=w.device)
    fn = qmm_partials_launch if gemm else qmv_partials_launch
    fn(type, _dev(w, torch.uint8, "w"), N, K, _dev(xq, torch.uint8, "xq"), B,
       _dev(P, torch.int32, "P"), _stream(stream))
    return P


# ------------------------------------------- K-quants x Q8_K activations --

def quantize_q8k(x, xq=None, stream=None, rows=None, K=None):
    """x: f32 [rows, K] (K % 256 == 0) -> Q8_K scratch (blocks first); x None:
    rebuild the staging from the Q8_K blocks already in xq."""
    import torch
    if x is not None:
        rows, K = x.shape
    if xq is None:
        n = qmv_act_bytes_q8k(rows, K)
        if n == 0:
            raise ValueError(f"bad shape rows={rows} K={K}")
        xq = torch.empty(n, dtype=torch.uint8, device=x.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    quantize_act_q8_k(xp, _dev(xq, torch.uint8, "xq"), rows, K, _stream(stream))
    return xq


def matmul_q8k(type: int, w, N: int, K: int, x=None, xq=None, M=None, y=None, stream=None):
    """y [M, N] f32 = x [M, K] @ W^T on the Q8_K path (any M; x None: staged xq)."""
    import torch
    if x is not None:
        M = x.shape[0]
    if xq is None:
        xq = torch.empty(qmv_act_bytes_q8k(M, K), dtype=torch.uint8, device=w.device)
    if y is None:
        y = torch.empty(M, N, dtype=torch.float32, device=w.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmm_launch_q8k(type, _dev(w, torch.uint8, "w"), N, K, xp, M, _dev(xq, torch.uint8, "xq"),
                   _dev(y, torch.float32, "y"), _stream(stream))
    return y


def gateup_swiglu_q8k(type: int, w_gate, w_up, N: int, K: int, x=None, xq=None, B=None, h=None,
                      stream=None):
    """h [B, N] f32 = silu(x Wg^T) * (x Wu^T) on the Q8_K path (x None: staged xq)."""
    import torch
    if x is not None:
        B = x.shape[0]
    if xq is None:
        xq = torch.empty(qmv_act_bytes_q8k(B, K), dtype=torch.uint8, device=w_gate.device)
    if h is None:
        h = torch.empty(B, N, dtype=torch.float32, device=w_gate.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmv_launch_gateup_swiglu_q8k(type, _dev(w_gate, torch.uint8, "w_gate"),
                                 _dev(w_up, torch.uint8, "w_up"), N, K, xp, B,
                                 _dev(xq, torch.uint8, "xq"), _dev(h, torch.float32, "h"),
                                 _stream(stream))
    return h


def partials_q8k(type: int, w, N: int, K: int, xq, M: int, P=None, stream=None):
    """Superblock partials of the Q8_K path: Q4_K [M, N, K/256, 2], Q6_K [M, N, K/256]."""
    import torch
    shape = (M, N, K // 256, 2) if type == Q4_K else (M, N, K // 256)
    if P is None:
        P = torch.empty(shape, dtype=torch.int32, device=w.device)
    qmv_partials_q8k_launch(type, _dev(w, torch.uint8, "w"), N, K, _dev(xq, torch.uint8, "xq"), M,
                            _dev(P, torch.int32, "P"), _stream(stream))
    return P


def prepare(type: int, w, N: int, K: int, wp=None, stream=None):
    """The load-time repack of a Q4_K / Q6_K blob for the Q8_K prefill GEMM."""
    import torch
    n = qmv_prepared_bytes(type, N, K)
    if n == 0:
        raise ValueError(f"no repacked layout for type {type} N={N} K={K}")
    if wp is None:
        wp = torch.empty(n, dtype=torch.uint8, device=w.device)
    qmv_prepare(type, _dev(w, torch.uint8, "w"), N, K, _dev(wp, torch.uint8, "wp"), _stream(stream))
    return wp


def matmul_q8k_prepared(type: int, wp, N: int, K: int, x=None, xq=None, M=None, y=None,
                        stream=None):
    """y [M, N] f32 = x [M, K] @ W^T from repacked weights (x None: staged xq)."""
    import torch
    if x is not None:
        M = x.shape[0]
    if xq is None:
        xq = torch.empty(qmv_act_bytes_q8k(M, K), dtype=torch.uint8, device=wp.device)
    if y is None:
        y = torch.empty(M, N, dtype=torch.float32, device=wp.device)
    xp = _dev(x, torch.float32, "x") if x is not None else None
    qmm_launch_q8k_prepared(type, _dev(wp, torch.uint8, "wp"), N, K, xp, M,
                            _dev(xq, torch.uint8, "xq"), _dev(y, torch.float32, "y"),
                            _stream(stream))
    return y


def partials_q8k_prepared(type: int, wp, N: int, K: int, xq, M: int, P=None, stream=None):
    import torch
    shape = (M, N, K // 256, 2) if type == Q4_K else (M, N, K // 256)
    if P is None:
        P = torch.empty(shape, dtype=torch.int32, device=wp.device)
    qmm_partials_q8k_prepared_launch(type, _dev(wp, torch.uint8, "wp"), N, K,
                                     _dev(xq, torch.uint8, "xq"), M, _dev(P, torch.int32, "P"),
                                     _stream(stream))
    return P
