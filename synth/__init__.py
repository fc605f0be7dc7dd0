"""Seeded synthetic inputs: GGUF block-quantised weight blobs and f32 activations.

This module is shared by the tests, the benchmark and the smoke check. It holds
no arithmetic of the multiply itself: it draws integer codes and fp16 scales
and *encodes* them into the GGUF block byte layout (the inverse direction of a
decoder), and it draws f32 activations. Neither the CPU oracle nor the HIP
library imports it, and it imports neither of them.

Block layouts encoded here (little-endian; fp16 = IEEE binary16).  The pages
name the formats only (llamay "Models and formats", section "Tensor formats");
the byte layouts below are the published GGUF ones:

  Q8_0  32 elems, 34 B : d f16 | qs int8[32]              value d*qs[e]
  Q4_0  32 elems, 18 B : d f16 | qs u8[16]                e<16: lo nibble of qs[e];
                                                          e>=16: hi nibble of qs[e-16];
                                                          value d*(q-8)
  Q5_0  32 elems, 22 B : d f16 | qh u32 | qs u8[16]       low 4 bits as Q4_0; bit 4 of
                                                          q is bit e of qh (LE u32);
                                                          value d*(q-16)
  Q4_1  32 elems, 20 B : d f16 | m f16 | qs u8[16]        nibbles as Q4_0; value d*q + m
  Q5_1  32 elems, 24 B : d f16 | m f16 | qh u32 | qs[16]  codes as Q5_0; value d*q + m
  Q8_1  32 elems, 36 B : d f16 | s f16 | qs int8[32]      value d*qs[e] (s = d*sum(qs),
                                                          stored, not part of the value)
  Q4_K 256 elems, 144 B: d f16 | dmin f16 | sc12 u8[12] | qs u8[128]
                         element e: c=e//64, r=e%64, byte qs[32c + r%32],
                         lo nibble if r<32 else hi nibble; sub-block j=e//32;
                         6-bit (sc_j, m_j) packed in sc12; value d*sc_j*q - dmin*m_j
  Q6_K 256 elems, 210 B: ql u8[128] | qh u8[64] | s int8[16] | d f16
                         element e: h=e//128, r=e%128, k=r//32, l=r%32;
                         low4 = nibble (k//2) of ql[64h + 32(k%2) + l];
                         high2 = bits 2k..2k+1 of qh[32h + l]; q = low4 | high2<<4;
                         sub-block j=e//16; value d*s_j*(q-32)
"""
from __future__ import annotations

import numpy as np

# GGUF tensor type ids (public GGUF enumeration).
Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q8_1, Q4_K, Q6_K = 2, 3, 6, 7, 8, 9, 12, 14
FORMATS = {"Q4_0": Q4_0, "Q4_1": Q4_1, "Q5_0": Q5_0, "Q5_1": Q5_1, "Q8_0": Q8_0, "Q8_1": Q8_1,
           "Q4_K": Q4_K, "Q6_K": Q6_K}
NAMES = {v: k for k, v in FORMATS.items()}
# (elements per block, bytes per block)
BLOCK = {Q8_0: (32, 34), Q4_0: (32, 18), Q5_0: (32, 22), Q4_1: (32, 20), Q5_1: (32, 24),
         Q8_1: (32, 36), Q4_K: (256, 144), Q6_K: (256, 210)}


def row_bytes(fmt: int, K: int) -> int:
    qk, nbytes = BLOCK[fmt]
    return (K // qk) * nbytes


def blob_bytes(fmt: int, N: int, K: int) -> int:
    return N * row_bytes(fmt, K)


def _f16_scales(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    """|N(0,1)| * scale, rounded to fp16 (numpy's conversion is round-to-nearest-even)."""
    return (np.abs(rng.standard_normal(shape)) * scale).astype(np.float16)


def draw_fields(fmt: int, N: int, K: int, seed: int, dscale: float = 0.01,
                s_range=(-32, 31)) -> dict:
    """Draw the fields of an N x K weight matrix: scales first, then codes.

    Distributions follow the workloads: codes uniform over their full range,
    fp16 d (and dmin) = |N(0,1)|*dscale, Q4_K 6-bit sc/m uniform in [0,63],
    Q6_K int8 sub-scales uniform in s_range (inclusive).
    """
    qk, _ = BLOCK[fmt]
    if K % qk:
        raise ValueError(f"K={K} is not a multiple of {qk}")
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = K // qk
    f: dict = {"fmt": fmt, "N": N, "K": K}
    if fmt in (Q8_0, Q8_1):
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        f["q"] = rng.integers(-127, 128, size=(N, K), dtype=np.int16).astype(np.int8)
    elif fmt == Q4_0:
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        f["q"] = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    elif fmt == Q5_0:
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        f["q"] = rng.integers(0, 32, size=(N, K), dtype=np.uint8)
    elif fmt in (Q4_1, Q5_1):
        # m: the block minimum, negative in practice: -|N(0,1)| * 8 * dscale
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        f["m"] = (-_f16_scales(rng, (N, nb), dscale * 8)).astype(np.float16)
        f["q"] = rng.integers(0, 16 if fmt == Q4_1 else 32, size=(N, K), dtype=np.uint8)
    elif fmt == Q4_K:
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        f["dmin"] = _f16_scales(rng, (N, nb), dscale)
        f["sc"] = rng.integers(0, 64, size=(N, nb, 8), dtype=np.uint8)
        f["m"] = rng.integers(0, 64, size=(N, nb, 8), dtype=np.uint8)
        f["q"] = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    elif fmt == Q6_K:
        f["d"] = _f16_scales(rng, (N, nb), dscale)
        lo, hi = s_range
        f["s"] = rng.integers(lo, hi + 1, size=(N, nb, 16), dtype=np.int16).astype(np.int8)
        f["q"] = rng.integers(0, 64, size=(N, K), dtype=np.uint8)
    else:
        raise ValueError(f"unknown format {fmt}")
    return f


def _f16_bytes(a: np.ndarray) -> np.ndarray:
    """fp16 array [..] -> little-endian bytes [.., 2]."""
    return a.astype("<f2").view(np.uint8).reshape(a.shape + (2,))


def encode(f: dict) -> np.ndarray:
    """Encode drawn fields into a GGUF block blob (uint8, N*row_bytes)."""
    fmt, N, K = f["fmt"], f["N"], f["K"]
    qk, nbytes = BLOCK[fmt]
    nb = K // qk
    out = np.zeros((N, nb, nbytes), dtype=np.uint8)
    if fmt == Q8_0:
        out[:, :, 0:2] = _f16_bytes(f["d"])
        out[:, :, 2:34] = f["q"].reshape(N, nb, 32).view(np.uint8)
    elif fmt == Q8_1:
        q = f["q"].reshape(N, nb, 32)
        out[:, :, 0:2] = _f16_bytes(f["d"])
        s = f["d"].astype(np.float32) * q.astype(np.float32).sum(axis=2)
        out[:, :, 2:4] = _f16_bytes(s.astype(np.float16))
        out[:, :, 4:36] = q.view(np.uint8)
    elif fmt == Q4_0:
        q = f["q"].reshape(N, nb, 32)
        out[:, :, 0:2] = _f16_bytes(f["d"])
        out[:, :, 2:18] = q[:, :, :16] | (q[:, :, 16:] << 4)
    elif fmt in (Q5_0, Q5_1):
        q = f["q"].reshape(N, nb, 32)
        out[:, :, 0:2] = _f16_bytes(f["d"])
        o = 2
        if fmt == Q5_1:
            out[:, :, 2:4] = _f16_bytes(f["m"])
            o = 4
        bits = (q >> 4).astype(np.uint32) << np.arange(32, dtype=np.uint32)
        qh = np.bitwise_or.reduce(bits, axis=2)
        out[:, :, o:o + 4] = qh.astype("<u4").view(np.uint8).reshape(N, nb, 4)
        lo = q & 15
        out[:, :, o + 4:o + 20] = lo[:, :, :16] | (lo[:, :, 16:] << 4)
    elif fmt == Q4_1:
        q = f["q"].reshape(N, nb, 32)
        out[:, :, 0:2] = _f16_bytes(f["d"])
        out[:, :, 2:4] = _f16_bytes(f["m"])
        out[:, :, 4:20] = q[:, :, :16] | (q[:, :, 16:] << 4)
    elif fmt == Q4_K:
        sc, m = f["sc"], f["m"]
        out[:, :, 0:2] = _f16_bytes(f["d"])
        out[:, :, 2:4] = _f16_bytes(f["dmin"])
        s12 = np.zeros((N, nb, 12), dtype=np.uint8)
        # sub-blocks 0..3: 6 bits in place; their top 2 bits carry bits 4..5 of 4..7
        s12[:, :, 0:4] = sc[:, :, 0:4] | ((sc[:, :, 4:8] >> 4) << 6)
        s12[:, :, 4:8] = m[:, :, 0:4] | ((m[:, :, 4:8] >> 4) << 6)
        # sub-blocks 4..7: low nibbles of sc (lo) and m (hi)
        s12[:, :, 8:12] = (sc[:, :, 4:8] & 15) | ((m[:, :, 4:8] & 15) << 4)
        out[:, :, 4:16] = s12
        q = f["q"].reshape(N, nb, 4, 2, 32)  # [.., group c, half, 32]
        out[:, :, 16:144] = (q[:, :, :, 0, :] | (q[:, :, :, 1, :] << 4)).reshape(N, nb, 128)
    elif fmt == Q6_K:
        q = f["q"].reshape(N, nb, 2, 4, 32)  # [.., half h, quarter k, l]
        lo4 = q & 15
        hi2 = q >> 4
        ql = np.zeros((N, nb, 2, 64), dtype=np.uint8)
        ql[:, :, :, 0:32] = lo4[:, :, :, 0, :] | (lo4[:, :, :, 2, :] << 4)
        ql[:, :, :, 32:64] = lo4[:, :, :, 1, :] | (lo4[:, :, :, 3, :] << 4)
        qh = (hi2[:, :, :, 0, :] | (hi2[:, :, :, 1, :] << 2)
              | (hi2[:, :, :, 2, :] << 4) | (hi2[:, :, :, 3, :] << 6))
        out[:, :, 0:128] = ql.reshape(N, nb, 128)
        out[:, :, 128:192] = qh.reshape(N, nb, 64)
        out[:, :, 192:208] = f["s"].view(np.uint8)
        out[:, :, 208:210] = _f16_bytes(f["d"])
    return out.reshape(-1)


def weights(fmt: int, N: int, K: int, seed: int, dscale: float = 0.01, **kw):
    """Return (blob uint8[N*row_bytes], fields dict) for a seeded weight matrix."""
    f = draw_fields(fmt, N, K, seed, dscale, **kw)
    return encode(f), f


def activations(B: int, K: int, seed: int) -> np.ndarray:
    """f32 N(0,1) activations [B, K], from their own PCG64 stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((B, K), dtype=np.float32)


# Workloads (shapes, formats and distributions of the pages' Qwen2.5-0.5B
# decode/prefill and of the 8B-class shapes).  Each entry: a list of matrices
# (fmt, N, K, dscale) and the batch sizes / token counts used with them.
WORKLOADS = {
    "q8_0_896": dict(mats=[(Q8_0, 896, 896, 0.01)], batches=[1]),
    "q4_0_ffn": dict(mats=[(Q4_0, 4864, 896, 0.02), (Q4_0, 4864, 896, 0.02),
                           (Q4_0, 896, 4864, 0.02)], batches=[1]),
    "kquant_lmhead": dict(mats=[(Q6_K, 151936, 1024, 0.01), (Q4_K, 4864, 1024, 0.01),
                                (Q4_K, 896, 4864, 0.01)], batches=[1, 4, 16]),
    "q4_0_prefill512": dict(mats=[(Q4_0, 4864, 896, 0.02), (Q4_0, 896, 4864, 0.02)],
                            batches=[512]),
    "8b_class": dict(mats=[(Q4_K, 4096, 4096, 0.02), (Q4_K, 1024, 4096, 0.02),
                           (Q4_K, 14336, 4096, 0.02), (Q6_K, 4096, 14336, 0.02)],
                     batches=[1, 16, 2048]),
    # the pages' Qwen2.5-0.5B file holds 132 Q5_0 tensors (histogram only);
    # taken here as its 2-D shapes other than ffn_down: gate/up 4864x896,
    # attention q/o 896x896, k/v 128x896 (an inference)
    "q5_0_qwen": dict(mats=[(Q5_0, 4864, 896, 0.02), (Q5_0, 896, 896, 0.02),
                            (Q5_0, 128, 896, 0.02)], batches=[1, 16, 512]),
    # the other 32-element formats the pages list, at the FFN gate shape
    "fmt32_4864x896": dict(mats=[(Q4_1, 4864, 896, 0.02), (Q5_1, 4864, 896, 0.02),
                                 (Q8_1, 4864, 896, 0.02)], batches=[1, 16, 512]),
}


def seed_for(config_index: int, matrix_index: int) -> int:
    """Seed of matrix i in workload c (base seed 0)."""
    return 1000 * config_index + matrix_index


def act_seed_for(config_index: int, batch: int) -> int:
    return 1000 * config_index + 100 + batch
