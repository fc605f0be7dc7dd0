"""Oracle pins: Q8_0 activation quantisation (hand-worked fixture, invariants)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "q8_0_act_blocks.json")


def _split(xq, rows, K):
    b = xq.reshape(rows, K // 32, 34)
    d = b[:, :, 0:2].copy().view("<u2")[:, :, 0]
    q = b[:, :, 2:].view(np.int8)
    return d, q


def test_golden_blocks_ties_away_from_zero():
    g = json.load(open(GOLD))
    blocks = g["blocks"]
    x = np.zeros((1, 32 * len(blocks)), np.float32)
    for i, blk in enumerate(blocks):
        for k, v in blk["x_nonzero"].items():
            x[0, 32 * i + int(k)] = np.float32(v)
    d, q = _split(oracle.quantize_act(x), 1, x.shape[1])
    for i, blk in enumerate(blocks):
        assert int(d[0, i]) == blk["d_fp16_bits"], blk["why"]
        want = np.zeros(32, np.int8)
        for k, v in blk["codes_nonzero"].items():
            want[int(k)] = v
        assert np.array_equal(q[0, i], want), blk["why"]


@pytest.fixture(scope="module")
def xs():
    return synth.activations(7, 32 * 29, seed=11) * np.float32(3.0)


def test_code_range_and_amax_maps_to_127(xs):
    rows, K = xs.shape
    d, q = _split(oracle.quantize_act(xs), rows, K)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    xb = xs.reshape(rows, K // 32, 32)
    imax = np.argmax(np.abs(xb), axis=2)
    top = np.take_along_axis(q, imax[..., None], axis=2)[..., 0].astype(np.int32)
    sgn = np.sign(np.take_along_axis(xb, imax[..., None], axis=2)[..., 0]).astype(np.int32)
    assert np.array_equal(top, 127 * sgn)


def test_sign_symmetry(xs):
    rows, K = xs.shape
    d1, q1 = _split(oracle.quantize_act(xs), rows, K)
    d2, q2 = _split(oracle.quantize_act(-xs), rows, K)
    assert np.array_equal(d1, d2)
    assert np.array_equal(q1.astype(np.int32), -q2.astype(np.int32))


@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_scaling(xs, k):
    rows, K = xs.shape
    d1, q1 = _split(oracle.quantize_act(xs), rows, K)
    d2, q2 = _split(oracle.quantize_act(xs * np.float32(2.0 ** k)), rows, K)
    assert np.array_equal(q1, q2)
    f1 = d1.view(np.float16).astype(np.float64)
    f2 = d2.view(np.float16).astype(np.float64)
    assert np.array_equal(f1 * 2.0 ** k, f2)


def test_idempotent_on_dequantised_values(xs):
    rows, K = xs.shape
    xq = oracle.quantize_act(xs)
    x2 = oracle.dequant_act(xq, rows, K).astype(np.float32)  # d16*q is exact in f32
    assert np.array_equal(oracle.quantize_act(x2), xq)


def test_rounding_error_bound(xs):
    """|x - d*q| <= d/2 up to the f32 rounding of 1/d and of x*(1/d)."""
    rows, K = xs.shape
    _, q = _split(oracle.quantize_act(xs), rows, K)
    xb = xs.reshape(rows, K // 32, 32).astype(np.float64)
    d = np.abs(xb).max(axis=2, keepdims=True) / 127.0
    err = np.abs(xb - d * q.astype(np.float64))
    assert np.all(err <= d * (0.5 + 1e-5))


def test_zero_rows_and_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, 40] = 1.5
    d, q = _split(oracle.quantize_act(x), 2, 64)
    assert np.all(d[0] == 0) and np.all(q[0] == 0)
    assert d[1, 0] == 0 and np.all(q[1, 0] == 0)
    assert q[1, 1, 8] == 127 and np.count_nonzero(q[1, 1]) == 1
    assert oracle.quantize_act(np.zeros((0, 32), np.float32)).size == 0


def test_blocks_too_small_for_a_finite_reciprocal_scale():
    """A block whose d = amax/127 is so small that 1/d overflows f32 (d below
    about 2^-128; subnormal amax, as a SwiGLU gate far below zero yields) is
    quantised like an all-zero block: codes 0 (its fp16 scale is 0 anyway).
    One just above that edge is quantised normally: its amax element maps
    to +-127."""
    x = np.zeros((1, 96), np.float32)
    x[0, 0:32] = np.linspace(-1e-40, 7e-41, 32, dtype=np.float32)     # subnormal amax
    x[0, 32:64] = np.linspace(2.0e-37, -2.5e-37, 32, dtype=np.float32)  # d ~ 2e-39: 1/d = inf
    x[0, 64:96] = np.linspace(-1e-36, 4e-37, 32, dtype=np.float32)     # d ~ 7.9e-39: 1/d finite
    q = oracle.quantize_act(x).reshape(3, 34)
    assert np.all(q[0] == 0) and np.all(q[1] == 0)
    assert q[2, 0] == 0 and q[2, 1] == 0                  # fp16(d) underflows to 0
    codes = q[2, 2:].view(np.int8)
    assert codes[0] == -127 and codes[-1] == 51           # -1e-36 -> -127, 4e-37 -> 50.8 -> 51
    # the edge itself: 1/d is finite exactly when d >= 1/FLT_MAX (to rounding)
    fmax = np.finfo(np.float32).max
    for amax in (np.float32(127.0) / fmax * np.float32(0.999), np.float32(127.0) / fmax * np.float32(1.001)):
        xb = np.zeros((1, 32), np.float32)
        xb[0, 0] = amax
        d = np.float32(amax) / np.float32(127.0)
        with np.errstate(over="ignore", divide="ignore"):
            finite = np.isfinite(np.float32(1.0) / d)
        c = oracle.quantize_act(xb)[2:].view(np.int8)
        assert c[0] == (127 if finite else 0)
