"""Comparison helpers shared by the parity tests (no arithmetic of the method)."""
import numpy as np

# Tolerance on final f32 outputs: |y - y_f64| <= RTOL * sum_k |w^ x^| per element.
RTOL = 1e-4


def tol_violations(y, y64, A, rtol=RTOL):
    """Indices where |y - y64| > rtol*A (A = sum |w^ x^|)."""
    y = np.asarray(y, np.float64)
    err = np.abs(y - y64)
    bad = ~(err <= rtol * A)
    return np.argwhere(bad)


def assert_tol(y, y64, A, rtol=RTOL, what=""):
    bad = tol_violations(y, y64, A, rtol)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(
            f"{what}: {len(bad)} elements outside {rtol}*sum|w x|; first at {i}: "
            f"got {np.asarray(y)[i]!r}, f64 {y64[i]!r}, bound {rtol * A[i]!r}")


def assert_bitwise(a, b, what=""):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    av = a.view(np.uint8).reshape(-1)
    bv = b.view(np.uint8).reshape(-1)
    if not np.array_equal(av, bv):
        diff = np.argwhere(a.reshape(-1).view(np.uint8 if a.dtype.itemsize == 1 else
                                               {2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])
                           != b.reshape(-1).view(np.uint8 if b.dtype.itemsize == 1 else
                                                 {2: np.uint16, 4: np.uint32, 8: np.uint64}[b.dtype.itemsize]))
        j = int(diff[0][0])
        raise AssertionError(f"{what}: {len(diff)} of {a.size} elements differ bitwise; "
                             f"first at flat {j}: {a.reshape(-1)[j]!r} vs {b.reshape(-1)[j]!r}")
