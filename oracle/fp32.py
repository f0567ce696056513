"""Single-precision operations the scheme specifies, emulated exactly.

numpy's float32 add, subtract, multiply and divide are IEEE binary32 with
round-to-nearest-even, so the oracle uses them directly.  The one operation
numpy lacks is a fused multiply-add with a single rounding; ``fma_f32``
provides it: the product of two float32 values is exact in float64 (24 + 24
significant bits, exponents well inside float64's range), so an error-free
sum and one correction give the correctly rounded float32 result.
"""

import numpy as np

_F32_MAX = float(np.finfo(np.float32).max)


def _twosum(a, b):
    """Error-free sum (Knuth): a + b == s + err exactly, s = fl64(a + b)."""
    s = a + b
    bb = s - a
    err = (a - (s - bb)) + (b - bb)
    return s, err


def fma_f32(a, b, c):
    """fp32(a*b + c) with one rounding (RNE), for float32 operands.

    Precondition: every operand is exactly a float32 value (integers
    |a| < 2^24 included); then a*b is exact in float64.

    Method: p = a*b exactly; s + err = p + c exactly (two-sum).  Rounding s
    to float32 gives the correctly rounded result unless s lies exactly on a
    midpoint between two float32 neighbours while err != 0; the sign of
    (s - midpoint) + err -- exact in sign because s - midpoint is exact
    (Sterbenz) -- then decides the direction.
    """
    a0, b0, c0 = (np.asarray(t) for t in (a, b, c))
    a = a0.astype(np.float32)
    b = b0.astype(np.float32)
    c = c0.astype(np.float32)
    for t0, t in ((a0, a), (b0, b), (c0, c)):
        if np.any(t0.astype(np.float64) != t.astype(np.float64)):
            raise ValueError("fma_f32: operands must be float32 values")
    p = a.astype(np.float64) * b.astype(np.float64)
    s, err = _twosum(p, c.astype(np.float64))
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.nextafter(r, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float32(-np.inf)).astype(np.float64)
    mid_up = 0.5 * (r64 + up)
    mid_dn = 0.5 * (r64 + dn)
    t_up = (s - mid_up) + err
    t_dn = (s - mid_dn) + err
    r_bits = r.view(np.uint32) if r.ndim else np.array(r).view(np.uint32)
    r_even = (r_bits & 1) == 0
    go_up = (t_up > 0) | ((t_up == 0) & ~r_even)
    go_dn = (t_dn < 0) | ((t_dn == 0) & ~r_even)
    out = np.where(go_up, up, np.where(go_dn, dn, r64)).astype(np.float32)
    # s == 0 exactly means p + c == 0 exactly (err is 0 as well)
    return np.where(s == 0, np.float32(0.0), out).astype(np.float32)
