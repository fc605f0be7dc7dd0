"""Oracle pins: fp16 <-> f32/f64 conversion against numpy's IEEE binary16 routines."""
import numpy as np

import oracle


def test_half_to_double_every_bit_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(v)) for v in h])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _cases():
    h = np.arange(0x7c00, dtype=np.uint16)            # every finite non-negative half
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                         # exact ties (12 significant bits)
    f32 = [v.astype(np.float32), mids.astype(np.float32)]
    m32 = mids.astype(np.float32)
    f32.append(np.nextafter(m32, np.float32(np.inf)))
    f32.append(np.nextafter(m32, np.float32(0)))
    rng = np.random.default_rng(7)
    f32.append((rng.standard_normal(100000) * 0.01).astype(np.float32))
    f32.append(np.exp2(rng.uniform(-30, 17, 100000)).astype(np.float32))
    f32.append(np.array([0.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30, np.inf,
                         2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
                         2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12), 1e-40], np.float32))
    x = np.concatenate(f32)
    return np.concatenate([x, -x])


def test_float_to_half_matches_numpy_rne_with_subnormals():
    x = _cases()
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.float_to_half(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} got {got[bad[0]]:#06x} want {ref[bad[0]]:#06x}"
