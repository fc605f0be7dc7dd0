"""Pins of the oracle's SwiGLU step, h = silu(g) * u with silu(g) = g/(1+e^-g)
(llamay "Models and formats", architectures table: SwiGLU feed-forward in the
llama baseline).  Each pin comes from outside the oracle's own formula:
printed values of the logistic function, closed forms at the ends of its
range, the odd-part identity silu(g) - silu(-g) = g, and exact scaling."""
import numpy as np
import pytest

import oracle

F32 = np.float32


def h(g, u):
    return oracle.swiglu(np.array(g, F32), np.array(u, F32))


# logistic function sigma(x) = 1/(1+e^-x) at x = 1, 2, 3 (standard tables):
# silu(x) = x * sigma(x), silu(-x) = -x * (1 - sigma(x))
SIGMA = {1.0: 0.7310585786300049, 2.0: 0.8807970779778823, 3.0: 0.9525741268224334}


@pytest.mark.parametrize("x", sorted(SIGMA))
def test_logistic_table_values(x):
    s = SIGMA[x]
    got = h([x, -x], [1.0, 1.0])
    # the true value rounded to f32 (the f64 evaluation is far more precise
    # than half an f32 ulp, unless the value sits on a rounding boundary,
    # which these do not)
    assert got[0] == F32(x * s)
    assert got[1] == F32(-x * (1.0 - s))


def test_zero_gate_gives_zero():
    got = h([0.0, 0.0, -0.0], [3.5, -7.0, 1.0])
    assert np.all(got == 0.0)


def test_large_positive_gate_is_the_product():
    # e^-g < 2^-53 for g > 36.8: 1 + e^-g rounds to 1 and h = fl32(g * u)
    g = np.array([40.0, 100.0, 1e4, 3.0e38], F32)
    u = np.array([1.25, -0.75, 3.0, 0.5], F32)
    assert np.array_equal(h(g, u), (g.astype(np.float64) * u.astype(np.float64)).astype(F32))


def test_large_negative_gate_vanishes():
    # e^-g overflows to infinity for g < -709.8: h = g / inf * u = 0
    got = h([-800.0, -1e30, -3.0e38], [1.0, -2.0, 5.0])
    assert np.all(got == 0.0)
    # at g = -100, silu(g) = -100 e^-100 (1 - ...) ~ -3.7e-42, an f32 subnormal
    assert h([-100.0], [1.0])[0] == F32(-100.0 * np.exp(np.float64(-100.0)))


def test_odd_part_identity():
    # silu(g) - silu(-g) = g exactly in the reals; each side rounds once to f32
    rng = np.random.Generator(np.random.PCG64(11))
    g = (rng.standard_normal(4096) * 4).astype(F32)
    ones = np.ones_like(g)
    d = h(g, ones).astype(np.float64) - h(-g, ones).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(h(g, ones)), np.abs(h(-g, ones))).astype(F32))
    assert np.all(np.abs(d - g.astype(np.float64)) <= ulp.astype(np.float64))


def test_linear_in_u_exact_powers_of_two():
    rng = np.random.Generator(np.random.PCG64(12))
    g = rng.standard_normal(1000).astype(F32)
    u = rng.standard_normal(1000).astype(F32)
    base = h(g, u)
    for k in (-3, 1, 5):
        assert np.array_equal(h(g, u * F32(2.0 ** k)), base * F32(2.0 ** k))
    assert np.array_equal(h(g, -u), -base)


def test_sign_and_monotone_gate():
    # silu > 0 for g > 0, < 0 for g < 0 and increasing for g > -1.28
    g = np.linspace(-1.2, 6.0, 2001).astype(F32)
    y = h(g, np.ones_like(g))
    assert np.all(np.sign(y) == np.sign(g))
    assert np.all(np.diff(y.astype(np.float64)) >= 0)
