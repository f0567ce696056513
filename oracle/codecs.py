"""Number formats used by the quantized path, written from their definitions.

* bfloat16: the top 16 bits of an IEEE binary32, rounded to nearest, ties to
  even (RNE).
* float16: IEEE binary16; numpy's float32 -> float16 conversion (RNE) is used
  as a library primitive and pinned by the tests against a brute-force
  nearest-value search.
* OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities,
  only S.1111.111 is NaN, so the largest finite value is 448; subnormals have
  exponent -6 and step 2^-9.
* E8M0: an unsigned byte e + 127 standing for the scale 2^e.

The pages name none of these formats (they say only "low-bit", podcast notes
section "02:48 There were clearly faster compute units on the hardware"); they
are the formats of the library's stated scheme.
"""

import numpy as np

# ----------------------------------------------------------------- bfloat16


def bf16_bits(x):
    """RNE-round float32 values to bfloat16; return the 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(x)
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_bf16(x):
    """float32 -> nearest bfloat16 value, returned as float32 (exact)."""
    return bf16_to_f32(bf16_bits(x))


# ----------------------------------------------------------------- float16


def round_f16(x):
    """float32 -> nearest float16 value (RNE), returned as float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(x, dtype):
    """RNE-round float32 values to the named 16-bit type ('bf16'|'f16')."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f16":
        return round_f16(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------- e4m3fn


def e4m3_decode(code):
    """Decode OCP e4m3fn bytes to float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    out = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def _e4m3_positive_table():
    """The 127 finite non-negative e4m3fn values, ascending (code == index)."""
    return e4m3_decode(np.arange(127, dtype=np.uint8))


_E4M3_POS = _e4m3_positive_table()


def e4m3_encode(x):
    """RNE-encode finite float values with |x| <= 448 into e4m3fn bytes.

    Rounds to the nearest representable value; a value exactly halfway
    between two neighbours goes to the one with an even code (mantissa LSB
    0).  Magnitudes above 448 are rejected: the scheme scales every operand
    so that they never occur.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("e4m3_encode: input outside [-448, 448]")
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    vhi = _E4M3_POS[hi]
    vlo = _E4M3_POS[lo]
    dhi = vhi - a
    dlo = a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a == vhi, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


def round_e4m3(x):
    """x -> nearest e4m3fn value (RNE), as float64."""
    return e4m3_decode(e4m3_encode(x))


# ----------------------------------------------------------------- E8M0


E8M0_MIN = -127  # the smallest scale an E8M0 byte holds: byte 0 is 2^-127


def e8m0_exponent(amax):
    """Smallest integer e >= -127 with amax * 2^-e <= 448 (e = 0 when
    amax == 0).

    With amax = m * 2^k, m in [0.5, 1): amax * 2^-e <= 0.875 * 2^9 holds for
    e >= k - 9 when m <= 0.875 and for e >= k - 8 otherwise.  A block whose
    amax lies below 448 * 2^-127 keeps the scale 2^-127 (byte 0): its values
    then round to e4m3 subnormals or zero.
    """
    a = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(a)
    e = np.maximum(np.where(m <= 0.875, k - 9, k - 8), E8M0_MIN)
    return np.where(a == 0, 0, e).astype(np.int64)
