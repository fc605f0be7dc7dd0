"""CPU checks of arithmetic the GPU kernels rely on that can be verified
exhaustively on the host (no GPU, no library calls).

* The lane-per-chunk GEMV finds a lane's row (lane / C) and an output's
  batch row (t / G) as floor((a + 1/2) * rcp(b)) in f32, for a < 4096 and
  b <= 64, with the hardware reciprocal within 1 ulp.  Checked for every
  such (a, b) and for the correctly rounded reciprocal and its neighbours
  one ulp away.
"""
import numpy as np


def test_small_div_through_f32_reciprocal_is_exact():
    a = np.arange(4096, dtype=np.float32)
    exact = np.arange(4096)[None, :] // np.arange(1, 65)[:, None]
    for b in range(1, 65):
        r = np.float32(1.0) / np.float32(b)
        for rr in (r, np.nextafter(r, np.float32(0)), np.nextafter(r, np.float32(1))):
            q = ((a + np.float32(0.5)) * rr).astype(np.int32)
            assert np.array_equal(q, exact[b - 1]), f"b={b}, rcp={rr!r}"
