"""Pins for oracle/codecs.py and oracle/fp32.py against independent definitions.

The number formats are those of the library's stated scheme (the pages name
none: podcast notes, section "02:48 There were clearly faster compute units on
the hardware").  Each codec is checked against something other than itself:
exhaustive tables built from the format definition, exact rational
arithmetic, or torch's independent CPU casts.
"""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle.fp32 import fma_f32


# ------------------------------------------------------------------ e4m3fn

def _e4m3_value_from_definition(code):
    """Decode one byte straight from the OCP e4m3fn definition (Fraction)."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None  # NaN
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def test_e4m3_decode_all_256_codes():
    dec = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = _e4m3_value_from_definition(c)
        if ref is None:
            assert np.isnan(dec[c]), c
        else:
            assert dec[c] == float(ref), c
    assert dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9


def test_e4m3_encode_roundtrip_and_midpoints():
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = codecs.e4m3_decode(np.array(finite, dtype=np.uint8))
    enc = codecs.e4m3_encode(vals)
    np.testing.assert_array_equal(enc, np.array(finite, dtype=np.uint8))
    pos = [float(_e4m3_value_from_definition(c)) for c in range(0x7F)]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert codecs.e4m3_encode(np.array([mid]))[0] == even
        assert codecs.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)
        assert codecs.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == c
        assert codecs.e4m3_encode(np.array([np.nextafter(mid, 1e9)]))[0] == c + 1


def test_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = codecs.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.array([449.0]))


# ------------------------------------------------------------------ bf16 / f16

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-30, 30, 200000)).astype(np.float32)
    # exact ties: low 16 bits == 0x8000
    u = rng.integers(0, 2 ** 31, 5000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0x7F7F0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = codecs.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_f16_round_is_nearest_even_by_search():
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    rng = np.random.default_rng(3)
    x = rng.uniform(0, 65000, 5000)
    mids = (allh[1:] + allh[:-1]) / 2
    x = np.concatenate([x, mids[::37]]).astype(np.float32)
    got = codecs.round_f16(x).astype(np.float64)
    for xi, gi in zip(x.astype(np.float64), got):
        i = np.searchsorted(allh, xi)
        cands = [allh[j] for j in (i - 1, i) if 0 <= j < len(allh)]
        best = min(abs(c - xi) for c in cands)
        near = [c for c in cands if abs(c - xi) == best]
        if len(near) == 2:  # tie: the even bit pattern
            near = [c for c in near if np.float16(c).view(np.uint16) % 2 == 0]
        assert gi == near[0], (xi, gi, near)


# ------------------------------------------------------------------ E8M0

def test_e8m0_exponent_is_smallest_fitting_power():
    rng = np.random.default_rng(4)
    ks = rng.integers(-40, 40, 4000)
    m = rng.uniform(0.5, 1.0, 4000)
    special = np.array([0.875, 0.8750001, 0.87499994, 0.5, 0.99999994])
    a = np.concatenate([np.ldexp(m, ks), np.ldexp(np.repeat(special, 10), np.tile(np.arange(-5, 5), 5))])
    a = a.astype(np.float32).astype(np.float64)
    e = codecs.e8m0_exponent(a)
    for ai, ei in zip(a, e):
        assert Fraction(ai) * Fraction(2) ** (-int(ei)) <= 448
        assert Fraction(ai) * Fraction(2) ** (-int(ei) + 1) > 448
    assert codecs.e8m0_exponent(np.array([0.0]))[0] == 0
    # below 448 * 2^-127 the scale stays at the E8M0 minimum 2^-127 (byte 0)
    tiny = np.array([448 * 2.0 ** -127, np.nextafter(448 * 2.0 ** -127, 0), 1e-37, 2.0 ** -149])
    assert list(codecs.e8m0_exponent(tiny)) == [-127, -127, -127, -127]
    assert codecs.e8m0_exponent(np.array([np.nextafter(448 * 2.0 ** -127, 1)]))[0] == -126


# ------------------------------------------------------------------ fp32 FMA

def _round_fraction_to_f32(x):
    """Correct RNE rounding of a Fraction to binary32 (normal range)."""
    if x == 0:
        return 0.0
    f = float(x)                     # nearest double
    c = np.float32(f)
    cands = {float(c), float(np.nextafter(c, np.float32(np.inf))),
             float(np.nextafter(c, np.float32(-np.inf)))}
    best = min(abs(Fraction(v) - x) for v in cands)
    near = sorted(v for v in cands if abs(Fraction(v) - x) == best)
    if len(near) == 2:
        near = [v for v in near if struct.unpack("<I", struct.pack("<f", v))[0] % 2 == 0]
    return near[0]


def test_fma_f32_single_rounding_against_fractions():
    rng = np.random.default_rng(5)
    n = 3000
    a = rng.integers(-2 ** 21, 2 ** 21, n).astype(np.float32)
    b = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    c = (rng.standard_normal(n) * 30).astype(np.float32)
    got = fma_f32(a, b, c)
    for i in range(n):
        ref = _round_fraction_to_f32(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert float(got[i]) == ref, i


def test_fma_f32_double_rounding_cases():
    # a*b + c lands exactly on a float32 midpoint plus a tiny tail that a
    # float64 rounding would lose: only a single rounding gets these right.
    cases = []
    for k in range(200):
        c = np.float32(1.0 + k * 2.0 ** -20)
        # target = c + half ulp(c) + 2^-60  ->  must round up
        b = np.float32(2.0 ** -24)
        a = np.float32(1.0)
        cases.append((a, b, c))
    a, b, c = (np.array(x, dtype=np.float32) for x in zip(*cases))
    got = fma_f32(a, b, c)
    for i in range(len(a)):
        ref = _round_fraction_to_f32(Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i])))
        assert float(got[i]) == ref
    # explicit tail beyond float64: a*b has 45 significant bits far below c
    a2 = np.array([2 ** 21 + 1], dtype=np.float32)
    b2 = np.array([np.float32(2.0 ** -45) * np.float32(1.0000001)], dtype=np.float32)
    c2 = np.array([np.float32(1.0)], dtype=np.float32)
    ref = _round_fraction_to_f32(Fraction(float(a2[0])) * Fraction(float(b2[0])) + Fraction(1))
    assert float(fma_f32(a2, b2, c2)[0]) == ref
    assert math.isfinite(ref)


def test_exponent_argument_is_rounded_once():
    """Step 5 of the emulation: x = fp32(S c - mref) is the float32 nearest to
    the exact rational S c - mref (ties to even), over the whole score range
    (|S| <= 127^2 d for d <= 128) and scales from 1e-8 to 1e-1, including
    cases where a float64 evaluation followed by a float32 rounding would
    round twice (tiny c against a large mref)."""
    from fractions import Fraction
    from oracle.emulate import exponent_arg
    rng = np.random.default_rng(32)
    n = 3000
    S = rng.integers(-2_064_512, 2_064_513, (n, 1)).astype(np.float64)
    c = (10.0 ** rng.uniform(-8, -1, n)).astype(np.float32)
    mref = rng.uniform(-40, 40, n).astype(np.float32)
    # double-rounding traps: S c = (2^22 + a)(2^22 - a) 2^-68 = 2^-24 - a^2 2^-68
    # lies just below half an ulp of -mref = 1 + (2k+1) 2^-23 (odd last bit);
    # a float64 sum rounds to the midpoint, whose float32 rounding then goes
    # up to the even neighbour, while the exact value rounds down
    a = np.arange(1, 51)
    S[:50, 0] = 2 ** 22 + a
    c[:50] = ((2 ** 22 - a) * 2.0 ** -68).astype(np.float32)
    mref[:50] = -(1.0 + (2 * a + 1) * 2.0 ** -23)
    twice = ((S[:50, 0] * c[:50].astype(np.float64) - mref[:50].astype(np.float64))).astype(np.float32)
    x = exponent_arg(S, c, mref)[:, 0]
    assert np.all(twice != x[:50])
    for i in range(n):
        exact = Fraction(int(S[i, 0])) * Fraction(float(c[i])) - Fraction(float(mref[i]))
        assert float(x[i]) == _round_fraction_to_f32(exact), i
    # c = 0 gives x = -mref; a power-of-two c with mref = 0 gives S c exactly
    z = exponent_arg(S[:5], np.zeros(5, np.float32), mref[:5])[:, 0]
    assert np.array_equal(z, -mref[:5])
    w = exponent_arg(S[:5], np.full(5, 2.0 ** -20, np.float32), np.zeros(5, np.float32))[:, 0]
    assert np.array_equal(w.astype(np.float64), S[:5, 0] * 2.0 ** -20)
    with pytest.raises(ValueError):
        exponent_arg(np.array([[2.0 ** 24]]), np.ones(1, np.float32), np.zeros(1, np.float32))
