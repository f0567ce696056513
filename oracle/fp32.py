"""Single-precision operations the scheme specifies, emulated exactly.

numpy's float32 add, subtract, multiply and divide are IEEE binary32 with
round-to-nearest-even, so the oracle uses them directly.  The one operation
numpy lacks is a fused multiply-add with a single rounding; ``fma_f32``
provides it for the case the scheme needs, where the product is exact in
float64.
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

    Precondition: a*b is exact in float64, which holds when ``a`` holds
    integers with |a| < 2^29 and ``b`` is float32 (24 + 29 <= 53 bits).

    Method: p = a*b exactly; s + err = p + c exactly (two-sum).  Rounding s
    to float32 gives the correctly rounded result unless s lies exactly on a
    midpoint between two float32 neighbours while err != 0; the sign of
    (s - midpoint) + err -- exact in sign because s - midpoint is exact
    (Sterbenz) -- then decides the direction.
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    c = np.asarray(c, dtype=np.float32)
    ai = a.astype(np.float64)
    if np.any(np.abs(ai) >= 2.0 ** 29) or np.any(ai != np.round(ai)):
        raise ValueError("fma_f32: first operand must be integer-valued, |a| < 2^29")
    p = ai * b.astype(np.float64)
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
