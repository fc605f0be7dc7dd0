"""Pins of the oracle's K-quant x Q8_K path (Q4_K / Q6_K weights against
activations quantised per 256 elements with an f32 scale).  Each pin is
independent of the oracle's own code: a hand-worked block
(tests/golden/q8k_act_block.json), invariants of the quantiser, partials by
brute force with Python integers from the generator's fields and codes
parsed here from the block bytes, the f64 result against a dense product,
and the f32 order against an exact-rational emulation of every rounding."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from checks import assert_bitwise, assert_tol

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8k_act_block.json")


def _parse(xq, rows, K):
    """(d f32 [rows, K/256], codes int [rows, K], bsums int [rows, K/16]) from the bytes."""
    b = np.asarray(xq, np.uint8).reshape(rows, K // 256, 292)
    d = b[:, :, 0:4].copy().view("<f4")[:, :, 0]
    codes = b[:, :, 4:260].view(np.int8).reshape(rows, K).astype(np.int64)
    bsums = b[:, :, 260:292].copy().view("<i2").reshape(rows, K // 16).astype(np.int64)
    return d, codes, bsums


def test_hand_worked_block():
    g = json.load(open(GOLDEN))
    x = np.zeros((1, 256), np.float32)
    for k, v in g["x_nonzero"].items():
        x[0, int(k)] = v
    xq = oracle.quantize_act_q8k(x)
    assert list(xq[:4]) == g["d_f32_bytes_le"]
    want = np.zeros(256, np.int64)
    for k, v in g["codes_nonzero"].items():
        want[int(k)] = v
    d, codes, bsums = _parse(xq, 1, 256)
    assert np.array_equal(codes[0], want)
    assert list(bsums[0]) == g["bsums"]


def test_quantiser_invariants():
    rng = np.random.Generator(np.random.PCG64(3))
    x = (rng.standard_normal((5, 1024)) * np.exp(rng.standard_normal((5, 1)) * 3)).astype(np.float32)
    x[2, 256:512] = 0.0
    xq = oracle.quantize_act_q8k(x)
    d, codes, bsums = _parse(xq, 5, 1024)
    assert np.all(np.abs(codes) <= 127)
    assert np.array_equal(bsums, codes.reshape(5, 64, 16).sum(axis=2))
    blocks = x.reshape(5, 4, 256)
    for r in range(5):
        for s in range(4):
            amax = np.max(np.abs(blocks[r, s]))
            assert d[r, s] == np.float32(amax) / np.float32(127)
            if amax > 0:
                i = int(np.argmax(np.abs(blocks[r, s])))
                assert codes[r, 256 * s + i] == (127 if blocks[r, s, i] > 0 else -127)
    assert np.all(codes[2, 256:512] == 0) and d[2, 1] == 0
    # sign symmetry and exact 2^k scaling
    n = _parse(oracle.quantize_act_q8k(-x), 5, 1024)
    assert np.array_equal(n[1], -codes) and np.array_equal(n[0], d)
    for k in (-20, 7):
        s = _parse(oracle.quantize_act_q8k(x * np.float32(2.0 ** k)), 5, 1024)
        assert np.array_equal(s[1], codes) and np.array_equal(s[0], d * np.float32(2.0 ** k))
    # half-step bound of the rounding
    xd = d[:, :, None].repeat(256, axis=2).reshape(5, 1024).astype(np.float64) * codes
    assert np.all(np.abs(xd - x) <= 0.5 * np.repeat(d, 256, axis=1) * (1 + 1e-6))


def test_tiny_blocks_quantise_to_zero():
    x = np.zeros((1, 512), np.float32)
    x[0, :256] = np.float32(1e-40)            # 1/d overflows f32
    x[0, 256:] = np.float32(1e-36)            # 1/d finite
    d, codes, _ = _parse(oracle.quantize_act_q8k(x), 1, 512)
    assert np.all(codes[0, :256] == 0)
    assert np.all(codes[0, 256:] == 127)


def _case(fmt, N=3, nsb=2, B=2, seed=0):
    K = 256 * nsb
    blob, f = synth.weights(fmt, N, K, seed, s_range=(-128, 127))
    x = synth.activations(B, K, seed + 50)
    xq = oracle.quantize_act_q8k(x)
    return blob, f, x, xq, N, K, B


def _wint_mint(f):
    N, K, q = f["N"], f["K"], f["q"].astype(np.int64)
    if f["fmt"] == synth.Q4_K:
        wint = np.repeat(f["sc"].reshape(N, -1), 32, axis=1).astype(np.int64) * q
        mint = np.repeat(f["m"].reshape(N, -1), 32, axis=1).astype(np.int64)
    else:
        wint = np.repeat(f["s"].reshape(N, -1), 16, axis=1).astype(np.int64) * (q - 32)
        mint = np.zeros((N, K), np.int64)
    return wint, mint


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
def test_partials_brute_force(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=4, nsb=3, B=3, seed=5)
    P = oracle.partials_q8k(fmt, blob, N, K, xq, B)
    wint, mint = _wint_mint(f)
    _, a, _ = _parse(xq, B, K)
    for m in range(B):
        for n in range(N):
            for s in range(K // 256):
                sl = slice(256 * s, 256 * s + 256)
                I = sum(int(w) * int(v) for w, v in zip(wint[n, sl], a[m, sl]))
                if fmt == synth.Q4_K:
                    Q = sum(int(w) * int(v) for w, v in zip(mint[n, sl], a[m, sl]))
                    assert (P[m, n, s, 0], P[m, n, s, 1]) == (I, Q)
                else:
                    assert P[m, n, s] == I


def test_partials_refuse_other_formats():
    blob, _ = synth.weights(synth.Q4_0, 2, 256, 1)
    xq = oracle.quantize_act_q8k(synth.activations(1, 256, 2))
    with pytest.raises(ValueError):
        oracle.partials_q8k(synth.Q4_0, blob, 2, 256, xq, 1)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
def test_f64_against_dense_product(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=5, nsb=4, B=3, seed=9)
    y, A = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, B)
    d, codes, _ = _parse(xq, B, K)
    xd = np.repeat(d.astype(np.float64), 256, axis=1) * codes
    wd = oracle.dequant(fmt, blob, N, K)
    assert np.all(np.abs(y - xd @ wd.T) <= 1e-12 * A)
    assert np.allclose(A, np.abs(xd) @ np.abs(wd).T, rtol=1e-12)


def _round_f32(fr: Fraction) -> Fraction:
    if fr == 0:
        return Fraction(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if 2 * r > ulp or (2 * r == ulp and q % 2 == 1):
        q += 1
    return sgn * q * ulp


@pytest.mark.parametrize("fmt,nsb", [(synth.Q4_K, 3), (synth.Q6_K, 3)])
def test_canon_f32_against_exact_rational_emulation(fmt, nsb):
    N, K, B = 3, 256 * nsb, 2
    f = synth.draw_fields(fmt, N, K, 21, s_range=(-128, 127))
    if fmt == synth.Q4_K:
        # large scales and codes, so that superblock partials pass 2^24 and (float)P rounds
        f["sc"] = np.maximum(f["sc"], 56)
        f["q"] = np.maximum(f["q"], 12)
    blob = synth.encode(f)
    x = (np.abs(synth.activations(B, K, 22)) * 0.2 + 4).astype(np.float32)
    xq = oracle.quantize_act_q8k(x)
    P = oracle.partials_q8k(fmt, blob, N, K, xq, B)
    u = oracle.unpack(fmt, blob, N, K)
    da, _, _ = _parse(xq, B, K)
    got = oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq, B)
    for m in range(B):
        for n in range(N):
            acc = Fraction(0)
            for s in range(nsb):
                dA = Fraction(float(da[m, s]))
                sd = _round_f32(Fraction(float(u["d"][n, s])) * dA)
                I = int(P[m, n, s, 0] if fmt == synth.Q4_K else P[m, n, s])
                p = _round_f32(_round_f32(Fraction(I)) * sd)
                if fmt == synth.Q4_K:
                    sm = _round_f32(Fraction(float(u["dmin"][n, s])) * dA)
                    p = _round_f32(p - _round_f32(Fraction(int(P[m, n, s, 1]))) * sm)
                acc = _round_f32(acc + p)
            assert got[m, n] == np.float32(float(acc)), (m, n)
    if fmt == synth.Q4_K:
        assert np.any(np.abs(P[..., 0]) > 2 ** 24)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
def test_canon_f32_error_bound(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=16, nsb=16, B=4, seed=33)
    y64, A = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, B)
    assert_tol(oracle.matmul_q8k_canon_f32(fmt, blob, N, K, xq, B), y64, A, what="canon vs f64")


def test_q4k_zero_scales_leave_minus_min_term():
    fmt, N, K, B = synth.Q4_K, 3, 512, 2
    f = synth.draw_fields(fmt, N, K, 40)
    f["sc"][:] = 0
    blob = synth.encode(f)
    x = synth.activations(B, K, 41)
    xq = oracle.quantize_act_q8k(x)
    y, _ = oracle.matmul_q8k_f64(fmt, blob, N, K, xq, B)
    d, codes, _ = _parse(xq, B, K)
    for m in range(B):
        for n in range(N):
            want = Fraction(0)
            for s in range(K // 256):
                for j in range(8):
                    S = int(codes[m, 256 * s + 32 * j: 256 * s + 32 * j + 32].sum())
                    want -= (Fraction(float(d[m, s])) * Fraction(float(f["dmin"][n, s]))
                             * int(f["m"][n, s, j]) * S)
            assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)
