"""ctypes wrapper of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product library never loads
it.  Functions take and return numpy arrays; see oracle.h for the definitions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1, Q4_K, Q6_K = 2, 3, 6, 7, 8, 9, 12, 14


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, no fast-math, no contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_float_to_half.argtypes = [ctypes.c_float]
        L.oracle_float_to_half.restype = ctypes.c_uint16
        L.oracle_quantize_act.argtypes = [P, I64, I64, P]
        L.oracle_unpack.argtypes = [I, P, I64, I64, P, P, P, P, P]
        L.oracle_dequant.argtypes = [I, P, I64, I64, P]
        L.oracle_dequant_act.argtypes = [P, I64, I64, P]
        L.oracle_partials.argtypes = [I, P, I64, I64, P, I64, P]
        L.oracle_matmul_f64.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.oracle_dense_f64.argtypes = [I, P, I64, I64, P, I64, P]
        L.oracle_matmul_canon_f32.argtypes = [I, P, I64, I64, P, I64, P]
        L.oracle_swiglu.argtypes = [P, P, I64, P]
        L.oracle_quantize_act_q8k.argtypes = [P, I64, I64, P]
        L.oracle_dequant_act_q8k.argtypes = [P, I64, I64, P]
        L.oracle_partials_q8k.argtypes = [I, P, I64, I64, P, I64, P]
        L.oracle_matmul_q8k_f64.argtypes = [I, P, I64, I64, P, I64, P, P]
        L.oracle_matmul_q8k_canon_f32.argtypes = [I, P, I64, I64, P, I64, P]
        L.oracle_prepared_bytes.argtypes = [I, I64, I64]
        L.oracle_prepared_bytes.restype = I64
        L.oracle_prepare_q8k.argtypes = [I, P, I64, I64, P]
        for name in ("oracle_quantize_act", "oracle_unpack", "oracle_dequant",
                     "oracle_dequant_act", "oracle_partials", "oracle_matmul_f64",
                     "oracle_dense_f64", "oracle_matmul_canon_f32", "oracle_swiglu",
                     "oracle_quantize_act_q8k", "oracle_dequant_act_q8k", "oracle_partials_q8k",
                     "oracle_matmul_q8k_f64", "oracle_matmul_q8k_canon_f32",
                     "oracle_prepare_q8k"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"{what} failed with code {rc}")


QK = {Q8_0: 32, Q4_0: 32, Q5_0: 32, Q4_1: 32, Q5_1: 32, Q8_1: 32, Q4_K: 256, Q6_K: 256}


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def float_to_half(f: float) -> int:
    return lib().oracle_float_to_half(float(f))


def quantize_act(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] -> Q8_0 blocks uint8 [rows * K/32 * 34]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    out = np.zeros(rows * (K // 32) * 34, dtype=np.uint8)
    _ok(lib().oracle_quantize_act(_p(x), rows, K, _p(out)), "quantize_act")
    return out


def unpack(fmt: int, blob: np.ndarray, N: int, K: int) -> dict:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    nbq = K // QK[fmt]
    q = np.zeros(N * K, np.int32)
    sc = np.zeros(N * K, np.int32)
    mn = np.zeros(N * K, np.int32)
    d = np.zeros(N * nbq, np.float64)
    dmin = np.zeros(N * nbq, np.float64)
    _ok(lib().oracle_unpack(fmt, _p(blob), N, K, _p(q), _p(sc), _p(mn), _p(d), _p(dmin)),
        "unpack")
    return dict(q=q.reshape(N, K), sub_scale=sc.reshape(N, K), sub_min=mn.reshape(N, K),
                d=d.reshape(N, nbq), dmin=dmin.reshape(N, nbq))


def dequant(fmt: int, blob: np.ndarray, N: int, K: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.zeros(N * K, np.float64)
    _ok(lib().oracle_dequant(fmt, _p(blob), N, K, _p(out)), "dequant")
    return out.reshape(N, K)


def dequant_act(xq: np.ndarray, rows: int, K: int) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    out = np.zeros(rows * K, np.float64)
    _ok(lib().oracle_dequant_act(_p(xq), rows, K, _p(out)), "dequant_act")
    return out.reshape(rows, K)


def partials(fmt: int, blob, N: int, K: int, xq, B: int) -> np.ndarray:
    """[B, N, K/32] int32 (Q4_K, Q4_1, Q5_1: [B, N, K/32, 2])."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    per = 2 if fmt in (Q4_K, Q4_1, Q5_1) else 1
    P = np.zeros(B * N * (K // 32) * per, np.int32)
    _ok(lib().oracle_partials(fmt, _p(blob), N, K, _p(xq), B, _p(P)), "partials")
    return P.reshape((B, N, K // 32, 2) if per == 2 else (B, N, K // 32))


def matmul_f64(fmt: int, blob, N: int, K: int, xq, B: int, want_abs: bool = True):
    """(y [B, N] f64, A [B, N] f64 = sum |w^ x^|)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.zeros(B * N, np.float64)
    A = np.zeros(B * N, np.float64) if want_abs else None
    _ok(lib().oracle_matmul_f64(fmt, _p(blob), N, K, _p(xq), B, _p(y), _p(A)), "matmul_f64")
    return y.reshape(B, N), (A.reshape(B, N) if want_abs else None)


def dense_f64(fmt: int, blob, N: int, K: int, xq, B: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.zeros(B * N, np.float64)
    _ok(lib().oracle_dense_f64(fmt, _p(blob), N, K, _p(xq), B, _p(y)), "dense_f64")
    return y.reshape(B, N)


def matmul_canon_f32(fmt: int, blob, N: int, K: int, xq, B: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.zeros(B * N, np.float32)
    _ok(lib().oracle_matmul_canon_f32(fmt, _p(blob), N, K, _p(xq), B, _p(y)),
        "matmul_canon_f32")
    return y.reshape(B, N)


def swiglu(g, u) -> np.ndarray:
    """h = silu(g) * u element by element (f64 evaluation, one rounding to f32)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    if g.shape != u.shape:
        raise ValueError("g and u differ in shape")
    h = np.zeros(g.shape, np.float32)
    _ok(lib().oracle_swiglu(_p(g), _p(u), g.size, _p(h)), "swiglu")
    return h


# ------------------------------------------ K-quants x Q8_K activations --

Q8K_BYTES = 292


def quantize_act_q8k(x: np.ndarray) -> np.ndarray:
    """f32 [rows, K] (K % 256 == 0) -> Q8_K blocks uint8 [rows * K/256 * 292]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    out = np.zeros(rows * (K // 256) * Q8K_BYTES, dtype=np.uint8)
    _ok(lib().oracle_quantize_act_q8k(_p(x), rows, K, _p(out)), "quantize_act_q8k")
    return out


def dequant_act_q8k(xq, rows: int, K: int) -> np.ndarray:
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    out = np.zeros(rows * K, np.float64)
    _ok(lib().oracle_dequant_act_q8k(_p(xq), rows, K, _p(out)), "dequant_act_q8k")
    return out.reshape(rows, K)


def partials_q8k(fmt: int, blob, N: int, K: int, xq, B: int) -> np.ndarray:
    """Q4_K [B, N, K/256, 2] (P, Q); Q6_K [B, N, K/256]."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    per = 2 if fmt == Q4_K else 1
    P = np.zeros(B * N * (K // 256) * per, np.int32)
    _ok(lib().oracle_partials_q8k(fmt, _p(blob), N, K, _p(xq), B, _p(P)), "partials_q8k")
    return P.reshape((B, N, K // 256, 2) if per == 2 else (B, N, K // 256))


def matmul_q8k_f64(fmt: int, blob, N: int, K: int, xq, B: int, want_abs: bool = True):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.zeros(B * N, np.float64)
    A = np.zeros(B * N, np.float64) if want_abs else None
    _ok(lib().oracle_matmul_q8k_f64(fmt, _p(blob), N, K, _p(xq), B, _p(y), _p(A)),
        "matmul_q8k_f64")
    return y.reshape(B, N), (A.reshape(B, N) if want_abs else None)


def matmul_q8k_canon_f32(fmt: int, blob, N: int, K: int, xq, B: int) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    y = np.zeros(B * N, np.float32)
    _ok(lib().oracle_matmul_q8k_canon_f32(fmt, _p(blob), N, K, _p(xq), B, _p(y)),
        "matmul_q8k_canon_f32")
    return y.reshape(B, N)


def prepared_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().oracle_prepared_bytes(fmt, N, K))


def prepare_q8k(fmt: int, blob, N: int, K: int) -> np.ndarray:
    """The load-time repack of a Q4_K / Q6_K blob (uint8 [prepared_bytes])."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    n = prepared_bytes(fmt, N, K)
    if n < 0:
        raise ValueError(f"oracle prepare: type {fmt} N={N} K={K} refused ({n})")
    out = np.zeros(n, np.uint8)
    _ok(lib().oracle_prepare_q8k(fmt, _p(blob), N, K, _p(out)), "prepare_q8k")
    return out
