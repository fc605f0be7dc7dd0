"""Oracle pins: block layouts.

* Hand-assembled blocks (tests/golden/weight_blocks.json) with values worked out
  by hand from the element formulas.
* Round trip: fields drawn by the seeded generator, encoded by its own encoder,
  decoded by the oracle, must come back unchanged -- including an exhaustive
  sweep of every code and sub-scale value at every position.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "weight_blocks.json")
FMTS = [synth.Q8_0, synth.Q4_0, synth.Q5_0, synth.Q4_1, synth.Q5_1, synth.Q8_1, synth.Q4_K,
        synth.Q6_K]


def _golden():
    return json.load(open(GOLD))["blocks"]


@pytest.mark.parametrize("name", ["Q8_0", "Q4_0", "Q5_0", "Q4_1", "Q5_1", "Q8_1", "Q4_K", "Q6_K"])
def test_hand_assembled_block(name):
    g = _golden()[name]
    blk = np.zeros(g["nbytes"], np.uint8)
    for s, e, v in g["fill"]:
        blk[s:e] = v
    for off, v in g["set"].items():
        blk[int(off)] = v
    qk = synth.BLOCK[g["type"]][0]
    vals = oracle.dequant(g["type"], blk, 1, qk)[0]
    for e, v in g["expect"].items():
        assert vals[int(e)] == v, f"{name} element {e}: {vals[int(e)]} != {v} ({g['why']})"
    if g["default"] is not None:
        rest = np.ones(qk, bool)
        rest[[int(e) for e in g["expect"]]] = False
        assert np.all(vals[rest] == g["default"])
    u = oracle.unpack(g["type"], blk, 1, qk)
    if name == "Q4_K":
        assert np.array_equal(u["sub_scale"][0].reshape(8, 32)[:, 0], g["sc"])
        assert np.array_equal(u["sub_min"][0].reshape(8, 32)[:, 0], g["m"])
        assert u["d"][0, 0] == 1.0 and u["dmin"][0, 0] == 0.5
    if name == "Q6_K":
        assert np.array_equal(u["sub_scale"][0].reshape(16, 16)[:, 0], g["s"])
        assert u["d"][0, 0] == 0.25
    if name in ("Q4_1", "Q5_1"):
        assert u["dmin"][0, 0] == {"Q4_1": -1.0, "Q5_1": 2.0}[name]
        assert np.all(u["sub_min"][0] == 1)


def _expected_fields(f):
    """What oracle.unpack must return for generator fields f."""
    fmt, N, K = f["fmt"], f["N"], f["K"]
    q = f["q"].astype(np.int32)
    sc = np.ones((N, K), np.int32)
    mn = np.zeros((N, K), np.int32)
    dmin = np.zeros_like(f["d"], dtype=np.float64)
    if fmt == synth.Q4_K:
        sc = np.repeat(f["sc"].reshape(N, -1), 32, axis=1).astype(np.int32)
        mn = np.repeat(f["m"].reshape(N, -1), 32, axis=1).astype(np.int32)
        dmin = f["dmin"].astype(np.float64)
    if fmt in (synth.Q4_1, synth.Q5_1):
        mn = np.ones((N, K), np.int32)
        dmin = f["m"].astype(np.float64)
    if fmt == synth.Q6_K:
        sc = np.repeat(f["s"].reshape(N, -1), 16, axis=1).astype(np.int32)
    return q, sc, mn, f["d"].astype(np.float64), dmin


def _check_roundtrip(f):
    blob = synth.encode(f)
    assert blob.size == synth.blob_bytes(f["fmt"], f["N"], f["K"])
    u = oracle.unpack(f["fmt"], blob, f["N"], f["K"])
    q, sc, mn, d, dmin = _expected_fields(f)
    assert np.array_equal(u["q"], q)
    assert np.array_equal(u["sub_scale"], sc)
    assert np.array_equal(u["sub_min"], mn)
    assert np.array_equal(u["d"], d)
    assert np.array_equal(u["dmin"], dmin)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("seed", [0, 1])
def test_roundtrip_random(fmt, seed):
    qk = synth.BLOCK[fmt][0]
    f = synth.draw_fields(fmt, 5, qk * 3, seed, s_range=(-128, 127))
    _check_roundtrip(f)


@pytest.mark.parametrize("fmt", FMTS)
def test_roundtrip_exhaustive_codes_and_subscales(fmt):
    """Row n gets code (n + e) mod range at element e, so across the rows every
    position carries every code value; sub-scales/mins sweep the same way."""
    qk = synth.BLOCK[fmt][0]
    K = qk * 2
    f = synth.draw_fields(fmt, 1, K, 0)
    rng_codes = {synth.Q8_0: 256, synth.Q4_0: 16, synth.Q5_0: 32, synth.Q4_1: 16, synth.Q5_1: 32,
                 synth.Q8_1: 256, synth.Q4_K: 16, synth.Q6_K: 64}[fmt]
    N = max(rng_codes, 64 if fmt == synth.Q4_K else 1, 256 if fmt == synth.Q6_K else 1)
    f = synth.draw_fields(fmt, N, K, 3)
    n = np.arange(N)[:, None]
    e = np.arange(K)[None, :]
    codes = (n + e) % rng_codes
    if fmt in (synth.Q8_0, synth.Q8_1):
        f["q"] = (codes - 128).astype(np.int8)
    else:
        f["q"] = codes.astype(np.uint8)
    if fmt == synth.Q4_K:
        j = np.arange(8)[None, None, :]
        sb = np.arange(K // 256)[None, :, None]
        f["sc"] = ((n[:, :, None] + j + sb) % 64).astype(np.uint8)
        f["m"] = ((n[:, :, None] + 3 * j + sb + 1) % 64).astype(np.uint8)
    if fmt == synth.Q6_K:
        j = np.arange(16)[None, None, :]
        sb = np.arange(K // 256)[None, :, None]
        f["s"] = (((n[:, :, None] + j + sb) % 256) - 128).astype(np.int8)
    _check_roundtrip(f)


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_element_position(fmt):
    """A single non-neutral code lands on exactly its own element."""
    qk = synth.BLOCK[fmt][0]
    neutral = {synth.Q8_0: 0, synth.Q4_0: 8, synth.Q5_0: 16, synth.Q4_1: 0, synth.Q5_1: 0,
               synth.Q8_1: 0, synth.Q4_K: 0, synth.Q6_K: 32}[fmt]
    for e in [0, 1, 15, 16, 31, qk - 1] + ([32, 63, 64, 127, 128, 200] if qk == 256 else []):
        f = synth.draw_fields(fmt, 1, qk, 5)
        f["q"][:] = neutral
        f["q"][0, e] = neutral + 3
        if "m" in f:
            f["m"][:] = 0
        if fmt == synth.Q4_K:
            f["sc"][:] = 1
        if fmt == synth.Q6_K:
            f["s"][:] = 1
        f["d"][:] = 1.0
        vals = oracle.dequant(fmt, synth.encode(f), 1, qk)[0]
        assert np.count_nonzero(vals) == 1 and vals[e] == 3.0, (fmt, e)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_matches_element_formulas(fmt):
    """Dequantised values vs the element formulas applied to the drawn fields."""
    qk = synth.BLOCK[fmt][0]
    f = synth.draw_fields(fmt, 4, qk * 2, 9, s_range=(-128, 127))
    N, K = 4, qk * 2
    q = f["q"].astype(np.float64)
    d = np.repeat(f["d"].astype(np.float64), qk, axis=1)
    if fmt == synth.Q8_0:
        want = d * q
    elif fmt == synth.Q4_0:
        want = d * (q - 8)
    elif fmt == synth.Q5_0:
        want = d * (q - 16)
    elif fmt in (synth.Q4_1, synth.Q5_1):
        want = d * q + np.repeat(f["m"].astype(np.float64), qk, axis=1)
    elif fmt == synth.Q8_1:
        want = d * q
    elif fmt == synth.Q4_K:
        sc = np.repeat(f["sc"].reshape(N, -1), 32, axis=1)
        mm = np.repeat(f["m"].reshape(N, -1), 32, axis=1)
        dmin = np.repeat(f["dmin"].astype(np.float64), qk, axis=1)
        want = d * sc * q - dmin * mm
    else:
        s = np.repeat(f["s"].reshape(N, -1), 16, axis=1)
        want = d * s * (q - 32)
    got = oracle.dequant(fmt, synth.encode(f), N, K)
    assert np.array_equal(got, want)


def test_refusals():
    with pytest.raises(ValueError):
        oracle.dequant(4, np.zeros(64, np.uint8), 1, 32)        # unknown type
    with pytest.raises(ValueError):
        oracle.dequant(synth.Q4_K, np.zeros(144, np.uint8), 1, 128)  # K % 256
