"""Oracle pins: integer partials, f64 result, documented f32 order.

* Partials by brute force with Python integers from the generator's fields.
* Each block's partials reproduce the exact rational dot product of the
  dequantised weights and activations (Fractions).
* f64 result vs a dense f64 product of the dequantised matrices (two ways).
* Closed forms: a hand-worked product, zero-point rows, Q4_K with sc = 0,
  negation, the triangle inequality.
* The documented f32 order vs an exact-rational emulation with explicit
  round-to-nearest-even, and vs its error bound.
* Teeth: the parity checks used on the GPU reject planted mistakes.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from checks import assert_bitwise, assert_tol, tol_violations

FMTS = [synth.Q8_0, synth.Q4_0, synth.Q5_0, synth.Q4_1, synth.Q5_1, synth.Q8_1, synth.Q4_K,
        synth.Q6_K]
MIN_FMTS = (synth.Q4_K, synth.Q4_1, synth.Q5_1)   # partials come in pairs


def _acts(xq, B, K):
    b = xq.reshape(B, K // 32, 34)
    d = b[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    a = b[:, :, 2:].view(np.int8).reshape(B, K).astype(np.int64)
    return d, a


def _case(fmt, N=3, nblk=2, B=2, seed=0):
    qk = synth.BLOCK[fmt][0]
    K = qk * nblk
    blob, f = synth.weights(fmt, N, K, seed, s_range=(-128, 127))
    x = synth.activations(B, K, seed + 50)
    xq = oracle.quantize_act(x)
    return blob, f, x, xq, N, K, B


def _wint_mint(f):
    """Per-element integer weight factor and min factor from generator fields."""
    fmt, N, K = f["fmt"], f["N"], f["K"]
    q = f["q"].astype(np.int64)
    mint = np.zeros((N, K), np.int64)
    if fmt in (synth.Q8_0, synth.Q8_1):
        wint = q
    elif fmt in (synth.Q4_1, synth.Q5_1):
        wint = q
        mint = np.ones((N, K), np.int64)
    elif fmt == synth.Q4_0:
        wint = q - 8
    elif fmt == synth.Q5_0:
        wint = q - 16
    elif fmt == synth.Q4_K:
        wint = np.repeat(f["sc"].reshape(N, -1), 32, axis=1).astype(np.int64) * q
        mint = np.repeat(f["m"].reshape(N, -1), 32, axis=1).astype(np.int64)
    else:
        wint = np.repeat(f["s"].reshape(N, -1), 16, axis=1).astype(np.int64) * (q - 32)
    return wint, mint


@pytest.mark.parametrize("fmt", FMTS)
def test_partials_brute_force(fmt):
    blob, f, x, xq, N, K, B = _case(fmt)
    P = oracle.partials(fmt, blob, N, K, xq, B)
    _, a = _acts(xq, B, K)
    wint, mint = _wint_mint(f)
    for m in range(B):
        for n in range(N):
            for b in range(K // 32):
                sl = slice(32 * b, 32 * b + 32)
                I = sum(int(w) * int(v) for w, v in zip(wint[n, sl], a[m, sl]))
                Q = sum(int(w) * int(v) for w, v in zip(mint[n, sl], a[m, sl]))
                if fmt in MIN_FMTS:
                    assert (P[m, n, b, 0], P[m, n, b, 1]) == (I, Q)
                else:
                    assert P[m, n, b] == I and Q == 0


@pytest.mark.parametrize("fmt", FMTS)
def test_partials_reproduce_exact_block_dot(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=2, nblk=1, B=2, seed=4)
    P = oracle.partials(fmt, blob, N, K, xq, B)
    W = oracle.dequant(fmt, blob, N, K)
    X = oracle.dequant_act(xq, B, K)
    u = oracle.unpack(fmt, blob, N, K)
    da, _ = _acts(xq, B, K)
    qk = synth.BLOCK[fmt][0]
    for m in range(B):
        for n in range(N):
            for b in range(K // 32):
                sl = slice(32 * b, 32 * b + 32)
                exact = sum(Fraction(float(w)) * Fraction(float(v)) for w, v in zip(W[n, sl], X[m, sl]))
                dw = Fraction(float(u["d"][n, (32 * b) // qk]))
                dmw = Fraction(float(u["dmin"][n, (32 * b) // qk]))
                if fmt == synth.Q4_K:
                    got = Fraction(float(da[m, b])) * (dw * int(P[m, n, b, 0]) - dmw * int(P[m, n, b, 1]))
                elif fmt in MIN_FMTS:   # dmin reports the block's m, which is added
                    got = Fraction(float(da[m, b])) * (dw * int(P[m, n, b, 0]) + dmw * int(P[m, n, b, 1]))
                else:
                    got = Fraction(float(da[m, b])) * dw * int(P[m, n, b])
                assert got == exact


@pytest.mark.parametrize("fmt", FMTS)
def test_f64_against_dense_products(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=7, nblk=3, B=3, seed=2)
    y, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    yd = oracle.dense_f64(fmt, blob, N, K, xq, B)
    W = oracle.dequant(fmt, blob, N, K)
    X = oracle.dequant_act(xq, B, K)
    ynp = X @ W.T
    Anp = np.abs(X) @ np.abs(W).T
    assert np.all(np.abs(y - yd) <= 1e-12 * A)
    assert np.all(np.abs(y - ynp) <= 1e-12 * A)
    assert np.allclose(A, Anp, rtol=1e-12, atol=0)
    assert np.all(np.abs(y) <= A * (1 + 1e-12))


def test_hand_worked_q8_0_product():
    """Weights: the hand-assembled Q8_0 block (d=2; codes -127@0, -1@5, 127@31).
    Activations: 127@0, 2@5, -127@31 -> d_a = 1, codes equal x.
    y = 2 * (-127*127 + -1*2 + 127*-127) = -64520."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "weight_blocks.json")))
    blk = np.zeros(34, np.uint8)
    for off, v in g["blocks"]["Q8_0"]["set"].items():
        blk[int(off)] = v
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 5], x[0, 31] = 127, 2, -127
    xq = oracle.quantize_act(x)
    y, A = oracle.matmul_f64(synth.Q8_0, blk, 1, 32, xq, 1)
    assert y[0, 0] == -64520.0 and A[0, 0] == 64520.0
    assert oracle.matmul_canon_f32(synth.Q8_0, blk, 1, 32, xq, 1)[0, 0] == np.float32(-64520.0)
    assert oracle.partials(synth.Q8_0, blk, 1, 32, xq, 1)[0, 0, 0] == -32260


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q5_0, synth.Q4_K, synth.Q6_K])
def test_zero_point_rows_give_exact_zero(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=2, nblk=2, B=2, seed=8)
    if fmt == synth.Q4_0:
        f["q"][:] = 8
    elif fmt == synth.Q5_0:
        f["q"][:] = 16
    elif fmt == synth.Q6_K:
        f["q"][:] = 32
    else:
        f["sc"][:] = 0
        f["m"][:] = 0
    blob = synth.encode(f)
    y, _ = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    assert np.all(y == 0)
    assert np.all(oracle.matmul_canon_f32(fmt, blob, N, K, xq, B) == 0)


@pytest.mark.parametrize("fmt", [synth.Q4_1, synth.Q5_1])
def test_zero_codes_leave_the_block_minimum(fmt):
    """q = 0 everywhere: y = sum_b d_a * m_b * S_b (S_b = sum of activation codes)."""
    blob, f, x, xq, N, K, B = _case(fmt, N=2, nblk=3, B=2, seed=13)
    f["q"][:] = 0
    blob = synth.encode(f)
    y, _ = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    da, a = _acts(xq, B, K)
    S = a.reshape(B, K // 32, 32).sum(axis=2)
    for m in range(B):
        for n in range(N):
            want = sum(Fraction(float(da[m, b])) * Fraction(float(f["m"][n, b])) * int(S[m, b])
                       for b in range(K // 32))
            assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)


def test_q4k_scale_zero_leaves_minus_min_term():
    """sc = 0: y = -sum_b d_a * dmin * m_j * S_b, S_b = sum of activation codes."""
    blob, f, x, xq, N, K, B = _case(synth.Q4_K, N=2, nblk=2, B=2, seed=12)
    f["sc"][:] = 0
    blob = synth.encode(f)
    y, _ = oracle.matmul_f64(synth.Q4_K, blob, N, K, xq, B)
    da, a = _acts(xq, B, K)
    S = a.reshape(B, K // 32, 32).sum(axis=2)
    for m in range(B):
        for n in range(N):
            want = Fraction(0)
            for b in range(K // 32):
                want -= (Fraction(float(da[m, b])) * Fraction(float(f["dmin"][n, b // 8]))
                         * int(f["m"][n, b // 8, b % 8]) * int(S[m, b]))
            assert abs(Fraction(y[m, n]) - want) <= abs(want) * Fraction(1, 2 ** 50)


@pytest.mark.parametrize("fmt", FMTS)
def test_negated_activations_negate_output(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, seed=21)
    y1, _ = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    y2, _ = oracle.matmul_f64(fmt, blob, N, K, oracle.quantize_act(-x), B)
    assert np.array_equal(y1, -y2)


# ---------------------------------------------------- documented f32 order --

def _round_f32(fr: Fraction) -> Fraction:
    """Round an exact rational to the nearest f32 (ties to even)."""
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


def _canon_exact(fmt, blob, N, K, xq, B):
    P = oracle.partials(fmt, blob, N, K, xq, B)
    u = oracle.unpack(fmt, blob, N, K)
    da, _ = _acts(xq, B, K)
    qk = synth.BLOCK[fmt][0]
    nb = K // 32
    y = np.zeros((B, N), np.float32)
    for m in range(B):
        for n in range(N):
            acc = Fraction(0)
            for c0 in range(0, nb, 8):
                p = Fraction(0)
                for b in range(c0, min(nb, c0 + 8)):
                    dA = Fraction(float(da[m, b]))
                    dw = Fraction(float(u["d"][n, (32 * b) // qk]))
                    if fmt in MIN_FMTS:
                        p = _round_f32(p + int(P[m, n, b, 0]) * dw * dA)
                        dmw = Fraction(float(u["dmin"][n, (32 * b) // qk]))
                        sgn = -1 if fmt == synth.Q4_K else 1   # Q4_K subtracts, Q4_1/Q5_1 add
                        p = _round_f32(p + sgn * int(P[m, n, b, 1]) * dmw * dA)
                    else:
                        p = _round_f32(p + int(P[m, n, b]) * dw * dA)
                acc = _round_f32(acc + p)
            y[m, n] = np.float32(float(acc))
    return y


@pytest.mark.parametrize("fmt,nblk", [(synth.Q8_0, 20), (synth.Q4_0, 9), (synth.Q5_0, 11),
                                      (synth.Q4_1, 9), (synth.Q5_1, 10), (synth.Q8_1, 9),
                                      (synth.Q4_K, 2), (synth.Q6_K, 2)])
def test_canon_f32_against_exact_rational_emulation(fmt, nblk):
    blob, f, x, xq, N, K, B = _case(fmt, N=3, nblk=nblk, B=2, seed=31)
    got = oracle.matmul_canon_f32(fmt, blob, N, K, xq, B)
    assert_bitwise(got, _canon_exact(fmt, blob, N, K, xq, B), "canon f32")


@pytest.mark.parametrize("fmt", FMTS)
def test_canon_f32_error_bound(fmt):
    blob, f, x, xq, N, K, B = _case(fmt, N=16, nblk=4 if synth.BLOCK[fmt][0] == 256 else 29,
                                    B=2, seed=40)
    y, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    yc = oracle.matmul_canon_f32(fmt, blob, N, K, xq, B).astype(np.float64)
    nb = K // 32
    rounds = nb * (2 if fmt in MIN_FMTS else 1) + (nb + 7) // 8
    assert np.all(np.abs(yc - y) <= rounds * 2.0 ** -24 * A * 1.0001)


def test_canon_single_block_is_one_rounding():
    blob, f, x, xq, N, K, B = _case(synth.Q8_0, N=9, nblk=1, B=3, seed=5)
    y, _ = oracle.matmul_f64(synth.Q8_0, blob, N, K, xq, B)   # exact: one product
    assert_bitwise(oracle.matmul_canon_f32(synth.Q8_0, blob, N, K, xq, B), y.astype(np.float32))


# ---------------------------------------------------------------- teeth --

def test_teeth_checks_reject_planted_mistakes():
    fmt = synth.Q4_K
    blob, f, x, xq, N, K, B = _case(fmt, N=8, nblk=4, B=2, seed=60)
    y64, A = oracle.matmul_f64(fmt, blob, N, K, xq, B)
    yc = oracle.matmul_canon_f32(fmt, blob, N, K, xq, B)
    P = oracle.partials(fmt, blob, N, K, xq, B)
    assert tol_violations(yc, y64, A).size == 0

    # (1) one weight code changed: the integer partials differ
    f2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in f.items()}
    f2["q"][3, 100] ^= 1
    P2 = oracle.partials(fmt, synth.encode(f2), N, K, xq, B)
    with pytest.raises(AssertionError):
        assert_bitwise(P2, P, "partials")

    # (2) one block scale off by one fp16 ulp: the f32 result differs bitwise
    f3 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in f.items()}
    f3["d"][2, 1] = np.nextafter(f3["d"][2, 1], np.float16(1))
    y3 = oracle.matmul_canon_f32(fmt, synth.encode(f3), N, K, xq, B)
    with pytest.raises(AssertionError):
        assert_bitwise(y3, yc, "canon")

    # (3) two superblocks of a row swapped: outside the 1e-4 tolerance
    b2 = blob.reshape(N, -1, 144).copy()
    b2[5, [0, 1]] = b2[5, [1, 0]]
    y4 = oracle.matmul_canon_f32(fmt, b2.reshape(-1), N, K, xq, B)
    with pytest.raises(AssertionError):
        assert_tol(y4, y64, A, what="swapped blocks")

    # (4) the min term dropped (dmin = 0): outside the tolerance
    f5 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in f.items()}
    f5["dmin"][:] = 0
    y5 = oracle.matmul_canon_f32(fmt, synth.encode(f5), N, K, xq, B)
    with pytest.raises(AssertionError):
        assert_tol(y5, y64, A, what="dropped min term")
