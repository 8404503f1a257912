"""CPU checks of the closed-form arithmetic the kernels' epilogues use in
place of library calls (no GPU, no oracle: pure IEEE reasoning in numpy).

div448 (csrc/moe_device.h) computes x / 448 as q0 = RN(x c), c = RN(1/448),
r = fma(-q0, 448, x), q = fma(r, c, q0).  For a normal x the quotient
depends on the significand only, so checking every significand of a binade
covers every finite x the requant scale sees (x >= 1e-10)."""
import numpy as np


def _div448_fma(x):
    c = np.float32(1.0) / np.float32(448.0)
    c64 = np.float64(c)
    x64 = x.astype(np.float64)
    q0 = (x64 * c64).astype(np.float32)            # one rounding of an exact product
    q064 = q0.astype(np.float64)
    r64 = x64 - q064 * 448.0                       # exact in f64 (27-bit product, cancelling)
    r = r64.astype(np.float32)
    assert np.array_equal(r.astype(np.float64), r64), "the residual is not exact in f32"
    s64 = r64 * c64 + q064                         # within 2^-53 of the exact sum
    q = s64.astype(np.float32)
    # the f32 rounding of s64 is that of the exact sum unless s64 lies within
    # its own error of a rounding midpoint: there are none (asserted)
    qn = np.nextafter(q, np.float32(np.inf)).astype(np.float64)
    qp = np.nextafter(q, np.float32(-np.inf)).astype(np.float64)
    q64 = q.astype(np.float64)
    tol = np.abs(s64) * 2.0 ** -50
    assert not np.any(np.abs(s64 - (q64 + qn) / 2) <= tol)
    assert not np.any(np.abs(s64 - (q64 + qp) / 2) <= tol)
    return q


def test_div448_equals_ieee_division_on_every_significand():
    m = np.arange(2 ** 23, 2 ** 24, dtype=np.int64)
    for e in (0, -34, 20):   # [1, 2), the binade of 1e-10, a large one
        x = (m.astype(np.float64) * 2.0 ** (e - 23)).astype(np.float32)
        q = _div448_fma(x)
        ref = x / np.float32(448.0)
        assert np.array_equal(q.view(np.uint32), ref.view(np.uint32)), e
