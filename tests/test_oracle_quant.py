"""Pins for oracle/quant.py: mean, channel balance and block quantization.

Checked against exact sums (math.fsum), exact rationals, a per-element scalar
implementation in plain Python floats, closed forms and symmetries -- never
against the vectorized code itself.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, codecs
from oracle.constants import BQ, BK, VB, KMEAN_CHUNK


def _bf16_values(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return codecs.round_bf16(x)


def test_k_mean_equals_exact_mean():
    rng = np.random.default_rng(10)
    K = _bf16_values(rng, (2, 3, 700, 8), 2.0) + 3.0
    K = codecs.round_bf16(K.astype(np.float32))
    kv = np.array([700, 333])
    mu = quant.k_mean(K, kv)
    for b in range(2):
        for h in range(3):
            for c in range(8):
                col = [float(v) for v in K[b, h, :kv[b], c]]
                exact = Fraction(math.fsum(col)) / kv[b]
                # the float64 sum of these bf16 values is exact, so mu is
                # the float32 rounding of the float64 rounding of the mean
                assert mu[b, h, c] == np.float32(float(exact)), (b, h, c)


def test_k_mean_ignores_padding_and_order():
    rng = np.random.default_rng(11)
    K = _bf16_values(rng, (1, 2, 300, 4))
    K2 = K.copy()
    K2[:, :, 250:, :] = 1e3                          # padding must not matter
    np.testing.assert_array_equal(quant.k_mean(K, [250]), quant.k_mean(K2, [250]))
    perm = rng.permutation(250)
    K3 = K.copy()
    K3[:, :, :250] = K[:, :, perm]
    np.testing.assert_array_equal(quant.k_mean(K, [250]), quant.k_mean(K3, [250]))
    assert KMEAN_CHUNK == 128


def _scalar_quant_block(vals):
    """One block, element by element, with numpy float32 scalars."""
    f = np.float32
    amax = f(0)
    for v in vals:
        amax = max(amax, abs(f(v)))
    if amax == 0:
        return [0] * len(vals), f(0)
    delta = f(amax) / f(127)
    inv = f(127) / f(amax)
    out = []
    for v in vals:
        y = f(f(v) * inv)
        r = round(float(y))                      # Python round: ties to even
        out.append(int(min(127, max(-127, r))))
    return out, delta


def test_block_quant_matches_scalar_loop():
    rng = np.random.default_rng(12)
    X = (rng.standard_normal((1, 2, 200, 16)) * 3).astype(np.float32)
    X[0, 1, 64:128] = 0                             # an all-zero block
    codes, delta = quant.quant_int8_blocks(X, 64, [200])
    assert delta.shape == (1, 2, 4)
    for h in range(2):
        for t in range(4):
            lo, hi = 64 * t, min(64 * t + 64, 200)
            blk = X[0, h, lo:hi].reshape(-1)
            ref, dref = _scalar_quant_block(blk)
            assert delta[0, h, t] == dref
            np.testing.assert_array_equal(codes[0, h, lo:hi].reshape(-1), np.array(ref, np.int8))
    assert delta[0, 1, 1] == 0 and not codes[0, 1, 64:128].any()


def test_block_quant_closed_form_power_of_two():
    rng = np.random.default_rng(13)
    for k in (-6, 0, 3):
        ints = rng.integers(-127, 128, (1, 1, BQ, 32))
        ints[0, 0, 5, 7] = -127
        X = np.ldexp(ints.astype(np.float32), k).astype(np.float32)
        codes, delta = quant.quant_int8_blocks(X, BQ)
        assert delta[0, 0, 0] == np.float32(2.0 ** k)
        np.testing.assert_array_equal(codes, ints.astype(np.int8))


def test_block_quant_symmetries():
    rng = np.random.default_rng(14)
    X = (rng.standard_normal((1, 2, 150, 8)) * 2).astype(np.float32)
    c1, d1 = quant.quant_int8_blocks(X, BK)
    c2, d2 = quant.quant_int8_blocks(-X, BK)
    np.testing.assert_array_equal(c2, -c1)
    np.testing.assert_array_equal(d1, d2)
    c3, d3 = quant.quant_int8_blocks(np.ldexp(X, 5).astype(np.float32), BK)
    np.testing.assert_array_equal(c3, c1)
    np.testing.assert_array_equal(d3, np.ldexp(d1, 5).astype(np.float32))
    assert np.abs(c1).max() <= 127 and c1.min() >= -127


def test_padding_keys_have_zero_codes_and_no_influence():
    rng = np.random.default_rng(15)
    K = _bf16_values(rng, (1, 1, 130, 8))
    K2 = K.copy()
    K2[:, :, 100:] = 50.0
    mu = quant.k_mean(K, [100])
    c1, d1 = quant.quantize_k(K, mu, [100])
    c2, d2 = quant.quantize_k(K2, mu, [100])
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(d1, d2)
    assert not c1[0, 0, 100:].any()
    assert d1.shape == (1, 1, 3) and d1[0, 0, 2] == 0


def test_channel_shift_definition():
    rng = np.random.default_rng(16)
    Q = _bf16_values(rng, (1, 4, 256, 32))
    K = _bf16_values(rng, (1, 4, 256, 32))
    gains = 2.0 ** rng.uniform(-6, 6, (4, 32))
    K = codecs.round_bf16((K * gains[None, :, None, :]).astype(np.float32))
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    Ks = quant.smooth_k(K, mu)
    for h in range(4):
        for c in range(32):
            A = Fraction(float(np.abs(Q[0, h, :, c]).max()))
            Bv = Fraction(float(np.abs(Ks[0, h, :, c]).max()))
            r = Bv / A
            ai = int(a[0, h, c])
            assert Fraction(2) ** (2 * ai - 1) <= r < Fraction(2) ** (2 * ai + 1), (h, c, ai, float(r))


def test_channel_balance_keeps_products_exact():
    rng = np.random.default_rng(17)
    Q = _bf16_values(rng, (1, 1, 64, 16))
    K = _bf16_values(rng, (1, 1, 64, 16))
    K[..., 3] *= 8
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    assert a[0, 0, 3] >= 1
    Qs = np.ldexp(Q, a[:, :, None, :])
    Ks = np.ldexp(quant.smooth_k(K, mu), -a[:, :, None, :])
    lhs = Qs[0, 0].astype(np.float64) @ Ks[0, 0].astype(np.float64).T
    rhs = Q[0, 0].astype(np.float64) @ quant.smooth_k(K, mu)[0, 0].astype(np.float64).T
    np.testing.assert_array_equal(lhs, rhs)


def test_v_fp8_scales_and_codes():
    rng = np.random.default_rng(18)
    V = _bf16_values(rng, (1, 2, 100, 8), 3.0)
    V[0, 0, 32:64, 2] = 0
    codes, e, e8 = quant.quantize_v_fp8(V, [90])
    assert e.shape == (1, 2, 4, 8)
    np.testing.assert_array_equal(e8, (e + 127).astype(np.uint8))
    deq = quant.dequant_v_fp8(codes, e)
    for h in range(2):
        for t in range(4):
            lo, hi = VB * t, min(VB * t + VB, 90)
            if hi <= lo:                            # a block of padding only
                assert not e[0, h, t].any()
                continue
            for c in range(8):
                blk = V[0, h, lo:hi, c].astype(np.float64)
                amax = np.abs(blk).max()
                ee = int(e[0, h, t, c])
                if amax == 0:
                    assert ee == 0 and not codes[0, h, lo:hi, c].any()
                    continue
                scaled = np.ldexp(amax, -ee)
                assert 224 < scaled <= 448          # the smallest fitting power
                # each element is the nearest e4m3 value times 2^e
                ref = np.ldexp(codecs.round_e4m3(np.ldexp(blk, -ee)), ee)
                np.testing.assert_array_equal(deq[0, h, lo:hi, c], ref)
    assert not codes[0, :, 90:].any()


def test_v_fp8_tiny_block_keeps_the_smallest_scale():
    """A V block whose amax is below 448 * 2^-127 (bf16 goes down to 2^-133)
    gets E8M0 byte 0 (2^-127), finite codes, and values rounded to e4m3 at
    that scale -- never a wrapped byte or a NaN."""
    V = np.zeros((1, 1, 64, 4), np.float32)
    V[0, 0, :32, 0] = codecs.round_bf16(np.float32(1e-37))
    V[0, 0, :32, 1] = codecs.round_bf16(np.linspace(-3e-38, 3e-38, 32).astype(np.float32))
    V[0, 0, 32:, 2] = codecs.round_bf16(np.float32(2.0 ** -133))
    codes, e, e8 = quant.quantize_v_fp8(V)
    assert e[0, 0, 0, 0] == -127 and e[0, 0, 0, 1] == -127 and e[0, 0, 1, 2] == -127
    assert e8[0, 0, 0, 0] == 0 and e8[0, 0, 1, 2] == 0
    deq = quant.dequant_v_fp8(codes, e)
    assert np.all(np.isfinite(deq))
    for c in range(3):
        blk = V[0, 0, :, c].astype(np.float64)
        ee = np.repeat(e[0, 0, :, c], 32)
        ref = np.ldexp(codecs.round_e4m3(np.ldexp(blk, -ee)), ee)
        np.testing.assert_array_equal(deq[0, 0, :, c], ref)
    # bf16's smallest subnormal 2^-133 is 2^-6 at this scale: an e4m3 normal, kept exactly
    assert deq[0, 0, 0, 0] > 0 and deq[0, 0, 32, 2] == 2.0 ** -133
