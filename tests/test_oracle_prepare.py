"""Pins of the oracle's load-time repack of Q4_K / Q6_K weights for the Q8_K
path, each independent of the oracle's own decoders: the digit rule on
hand-worked values (closed form: v = 64 hi + lo, lo = v mod 64, floor
division for negative v), every element's recombined digits against the
generator's fields (sc * q, s * (q - 32)), the scale records against the
generator's d / dmin / mins, zero padding rows, and the superblock partials
summed from the repacked digits by brute force against the oracle's partials
of the GGUF blob."""
import numpy as np
import pytest

import oracle
import synth

REGION, REC = 16896, 16384


def _parse(buf, N, K):
    """(lo [T*32, K], hi [T*32, K], d, dmin [T*32, nsb], mins [T*32, nsb, 8])
    read back by the layout's index formula."""
    nsb, T = K // 256, (N + 31) // 32
    reg = np.asarray(buf, np.uint8).reshape(T, nsb, REGION)
    dig = reg[:, :, :REC].reshape(T, nsb, 8, 2, 2, 32, 16)    # t s j g h r i
    dig = dig.transpose(0, 5, 1, 2, 4, 6, 3).reshape(T * 32, K, 2)  # (t r) (s j h i) g
    lo = dig[..., 0].astype(np.int64)
    hi = dig[..., 1].view(np.int8).astype(np.int64)
    rec = reg[:, :, REC:].reshape(T, nsb, 32, 16).transpose(0, 2, 1, 3).reshape(T * 32, nsb, 16)
    d = rec[..., 0:4].copy().view("<f4")[..., 0]
    dmin = rec[..., 4:8].copy().view("<f4")[..., 0]
    return lo, hi, d, dmin, rec[..., 8:16]


def _wint(f):
    N, K = f["N"], f["K"]
    q = f["q"].astype(np.int64)
    if f["fmt"] == synth.Q4_K:
        sc = np.repeat(f["sc"].astype(np.int64).reshape(N, -1), 32, axis=1)
        return sc * q
    s = np.repeat(f["s"].astype(np.int64).reshape(N, -1), 16, axis=1)
    return s * (q - 32)


def test_digit_rule_hand_worked():
    """Q6_K values at the ends of the range: 4096 = 64*64 + 0, 3937 = 64*61 + 33,
    -1 = 64*(-1) + 63, -3968 = 64*(-62) + 0, 0."""
    N, K = 1, 256
    f = synth.draw_fields(synth.Q6_K, N, K, 5, s_range=(-128, 127))
    f["s"][0, 0, :5] = [-128, 127, -1, -128, 7]
    f["q"][0, [0, 16, 32, 48, 64]] = [0, 63, 33, 63, 32]
    buf = oracle.prepare_q8k(synth.Q6_K, synth.encode(f), N, K)
    # element e = 32 j + 16 h + i of row 0 (r = 0): lo at 1024*2j + 16*32h + i
    for e, (hi, lo) in {0: (64, 0), 16: (61, 33), 32: (-1, 63), 48: (-62, 0), 64: (0, 0)}.items():
        j, h, i = e // 32, (e % 32) // 16, e % 16
        assert buf[1024 * 2 * j + 512 * h + i] == lo, e
        assert np.int8(buf[1024 * (2 * j + 1) + 512 * h + i].view(np.int8)) == hi, e


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
@pytest.mark.parametrize("N,K", [(1, 256), (32, 512), (45, 768), (70, 256)])
def test_digits_and_records_against_the_fields(fmt, N, K):
    f = synth.draw_fields(fmt, N, K, 40 + N + K, s_range=(-128, 127))
    buf = oracle.prepare_q8k(fmt, synth.encode(f), N, K)
    assert buf.size == oracle.prepared_bytes(fmt, N, K) == (N + 31) // 32 * (K // 256) * REGION
    lo, hi, d, dmin, mins = _parse(buf, N, K)
    assert lo.min() >= 0 and lo.max() <= 63
    assert np.array_equal((64 * hi + lo)[:N], _wint(f))
    assert np.array_equal(d[:N], f["d"].astype(np.float32))
    if fmt == synth.Q4_K:
        assert np.array_equal(dmin[:N], f["dmin"].astype(np.float32))
        assert np.array_equal(mins[:N], f["m"])
    else:
        assert np.all(dmin == 0) and np.all(mins == 0)
    assert np.all(lo[N:] == 0) and np.all(hi[N:] == 0) and np.all(d[N:] == 0)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q6_K])
def test_partials_from_the_digits(fmt):
    N, K, B = 37, 768, 3
    blob, f = synth.weights(fmt, N, K, 60, s_range=(-128, 127))
    x = synth.activations(B, K, 61)
    xq = oracle.quantize_act_q8k(x)
    a = np.asarray(xq, np.uint8).reshape(B, K // 256, 292)[:, :, 4:260].view(np.int8)
    a = a.reshape(B, K).astype(np.int64)
    lo, hi, _, _, mins = _parse(oracle.prepare_q8k(fmt, blob, N, K), N, K)
    v = (64 * hi + lo)[:N].reshape(N, K // 256, 256)
    P = np.einsum("nsk,bsk->bns", v, a.reshape(B, K // 256, 256))
    want = oracle.partials_q8k(fmt, blob, N, K, xq, B)
    if fmt == synth.Q4_K:
        S = a.reshape(B, K // 256, 8, 32).sum(axis=3)
        Q = np.einsum("nsj,bsj->bns", mins[:N].astype(np.int64), S)
        assert np.array_equal(P, want[..., 0]) and np.array_equal(Q, want[..., 1])
    else:
        assert np.array_equal(P, want)


def test_refusals():
    assert oracle.prepared_bytes(synth.Q4_0, 32, 256) == -1
    assert oracle.prepared_bytes(synth.Q4_K, 32, 100) == -2
    with pytest.raises(ValueError):
        oracle.prepare_q8k(synth.Q8_0, np.zeros(34, np.uint8), 1, 32)
