"""Pins for the per-head P.V mode (PV_AUTO): the rule that picks each head's
mode, and the emulation running every head in its own mode.

The pages fix no bit widths (podcast notes, section "02:48 There were clearly
faster compute units on the hardware"); the rule is the library's reading:
FP8 P.V for a head whose channel-balance exponents are all 0, 16-bit P.V for
a head with an outlier channel.  Checked against hand-built exponents, the
exact amax ratios at which channel balance starts to move a channel, and the
single-mode emulations (themselves pinned elsewhere) head by head.
"""

import numpy as np

from oracle import quant, emulate, attention, codecs
from oracle.constants import PV_16, PV_FP8, PV_AUTO


def test_rule_on_hand_built_exponents():
    a = np.zeros((2, 3, 8), np.int64)
    a[0, 1, 5] = 2       # an outlier channel of K
    a[1, 2, 0] = -1      # a channel where Q's range is the larger one
    m = quant.pv_modes_auto(a)
    assert m.shape == (2, 3)
    want = np.full((2, 3), PV_FP8)
    want[0, 1] = PV_16
    want[1, 2] = PV_16
    np.testing.assert_array_equal(m, want)


def _head(kval, qval, n=64, d=8):
    """One head whose channel 3 has amax |K| = kval and |Q| = qval; K is
    symmetric in every channel, so its mean is 0 and K~ = K exactly; every
    other channel has K and Q amax 1."""
    Q = np.ones((1, 1, n, d), np.float32)
    Q[..., 1::2, :] = -1
    K = Q.copy()
    Q[..., 3] *= qval
    K[..., 3] *= kval
    return Q, K


def test_rule_switches_at_the_exact_ratios():
    # a_c != 0 exactly when amax_c(K~)/amax_c(Q) >= 2 or < 1/2 (channel_shift:
    # the nearest integer to half its log2, halves up)
    for kval, qval, mode in [(1.0, 1.0, PV_FP8), (1.9921875, 1.0, PV_FP8), (2.0, 1.0, PV_16),
                             (8.0, 1.0, PV_16), (0.5, 1.0, PV_FP8), (0.4921875, 1.0, PV_16)]:
        Q, K = _head(kval, qval)
        mu = quant.k_mean(K)
        assert not mu.any()
        a = quant.channel_shift(Q, K, mu)
        assert quant.pv_modes_auto(a)[0, 0] == mode, (kval, qval, a[0, 0])


def _inputs(seed, B=2, H=3, N=320, d=64):
    rng = np.random.default_rng(seed)
    Q = codecs.round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    K = rng.standard_normal((B, H, N, d)).astype(np.float32)
    K[0, 1, :, 7] *= 8          # outlier channels in (0,1) and (1,0)
    if B > 1:
        K[1, 0, :, 20] *= 8
    V = codecs.round_bf16(rng.standard_normal((B, H, N, d)).astype(np.float32))
    return Q, codecs.round_bf16(K), V


def test_auto_is_each_head_in_its_own_mode():
    Q, K, V = _inputs(3)
    kv = [320, 257]
    rows = np.array([0, 1, 63, 64, 127, 128, 200, 319])
    mu = quant.k_mean(K, kv)
    a = quant.channel_shift(Q, K, mu, kv)
    modes = quant.pv_modes_auto(a)
    want = np.full((2, 3), PV_FP8)
    want[0, 1] = want[1, 0] = PV_16
    np.testing.assert_array_equal(modes, want)
    got, got_r = emulate.emulate_from_inputs(Q, K, V, PV_AUTO, "bf16", kv_len=kv, rows=rows)
    o16, r16 = emulate.emulate_from_inputs(Q, K, V, PV_16, "bf16", kv_len=kv, rows=rows)
    o8, r8 = emulate.emulate_from_inputs(Q, K, V, PV_FP8, "bf16", kv_len=kv, rows=rows)
    for b in range(2):
        for h in range(3):
            ref, ref_r = (o8, r8) if modes[b, h] == PV_FP8 else (o16, r16)
            np.testing.assert_array_equal(got[b, h], ref[b, h])
            np.testing.assert_array_equal(got_r[b, h], ref_r[b, h])


def test_auto_with_splits_reports_modes_and_stays_accurate():
    Q, K, V = _inputs(4, B=1)
    sp = [emulate.split_ranges(320, 2)]
    rows = np.arange(0, 320, 7)
    o, _, aux = emulate.emulate_from_inputs(Q, K, V, PV_AUTO, "bf16", rows=rows, splits=sp,
                                            slack=emulate.Slack(lambda c, m, x: np.zeros(np.shape(x)), 0.0))
    np.testing.assert_array_equal(aux["pv_modes"], [[PV_FP8, PV_16, PV_FP8]])
    # and the result stays close to exact attention
    ref = attention.attention_fp64(Q, K, V)[:, :, rows]
    cos = float((o.ravel() @ ref.ravel()) / np.sqrt((o.ravel() @ o.ravel()) * (ref.ravel() @ ref.ravel())))
    assert cos > 0.999
