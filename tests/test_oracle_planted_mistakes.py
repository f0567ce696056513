"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle, on the CPU (a wrong variant
swapped into an oracle module for the duration of the case), runs the pin
that should see it, and requires that pin to fail: a dropped mask term, a
truncation for a rounding, a mean over padding, a tie rule, an exponent
rounded twice, the lazy-max threshold ignored, a reversed block index, the
caller's softmax scale ignored, a block mask ignored, a sliding window one
frame short or without its sink frames, the per-head P.V rule inverted or
blind to channels moved towards Q.  A pin that still
passed would not be pinning anything."""

import numpy as np
import pytest

from oracle import attention, codecs, emulate, quant, w8a8
from oracle.constants import PV_16, PV_FP8

import test_oracle_attention as TA
import test_oracle_auto as TAUTO
import test_oracle_codecs as TC
import test_oracle_quant as TQ
import test_oracle_sparse as TS
import test_oracle_w8a8 as TW
import test_oracle_window as TWIN


class _NumpyWithTruncation:
    """numpy, except that rint truncates (the planted mistake)."""

    def __getattr__(self, name):
        return getattr(np, name)

    rint = staticmethod(np.trunc)


def _e4m3_ties_away(x):
    """e4m3_encode with halfway values rounded away from zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    pos = codecs._E4M3_POS
    hi = np.minimum(np.searchsorted(pos, a, side="left"), 126)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (pos[hi] - a) <= (a - pos[lo])
    code = np.where(a == pos[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return (code | (np.signbit(x).astype(np.uint8) << 7)).astype(np.uint8)


def _exponent_rounded_twice(S, c_t, mref):
    """fp32(fp32(S c) - mref): two roundings instead of one."""
    S = np.asarray(S, dtype=np.float64)
    sc = (S.astype(np.float32) * np.asarray(c_t, np.float32)[:, None]).astype(np.float32)
    return (sc - np.asarray(mref, np.float32)[:, None]).astype(np.float32)


def _cases():
    k_mean, row_end, attn = quant.k_mean, attention.row_end, attention.attention_fp64
    gemm, block_visible = w8a8.gemm_exact, attention.block_visible

    def window_one_short(fk, fq, sink_frames=0, window_frames=0):
        # the window's oldest frame dropped: > where >= belongs
        fk, fq = np.asarray(fk, dtype=np.int64), np.asarray(fq, dtype=np.int64)
        ok = fk <= fq
        if window_frames:
            ok = ok & ((fk < int(sink_frames)) | (fk > fq - int(window_frames)))
        return ok

    def sinks_ignored(fk, fq, sink_frames=0, window_frames=0):
        fk, fq = np.asarray(fk, dtype=np.int64), np.asarray(fq, dtype=np.int64)
        ok = fk <= fq
        if window_frames:
            ok = ok & (fk >= fq - int(window_frames))
        return ok

    return [
        ("K mean over padding tokens", quant, "k_mean",
         lambda K, kv_len=None: k_mean(K, None), TQ.test_k_mean_ignores_padding_and_order, {}),
        ("block codes truncated, not rounded", quant, "np", _NumpyWithTruncation(),
         TQ.test_block_quant_matches_scalar_loop, {}),
        ("mask drops the last key of the row's frame", attention, "row_end",
         lambda i, kv, qp, F: row_end(i, kv, qp, F) - (1 if F else 0), TA.test_mask_rule_by_enumeration, {}),
        ("softmax scale of the caller ignored", attention, "attention_fp64",
         lambda Q, K, V, sm_scale=None, *a, **k: attn(Q, K, V, None, *a, **k),
         TA.test_fp64_attention_matches_python_loops, {"frame_len": 0}),
        ("lazy running max without its threshold", emulate, "TAU", 0.0,
         TA.test_lazy_running_max_policy_by_hand, {}),
        ("exponent argument rounded twice", emulate, "exponent_arg", _exponent_rounded_twice,
         TC.test_exponent_argument_is_rounded_once, {}),
        ("e4m3 halfway values away from zero", codecs, "e4m3_encode", _e4m3_ties_away,
         TC.test_e4m3_encode_roundtrip_and_midpoints, {}),
        ("W8A8 activation scales of the reversed K block", w8a8, "gemm_exact",
         lambda xq, dx, wq, dw, bias=None: gemm(xq, dx[:, ::-1], wq, dw, bias),
         TW.test_gemm_matches_brute_force_and_bias, {}),
        ("block mask ignored", attention, "block_visible",
         lambda vis, rows, m: vis, TS.test_fp64_block_mask_equals_brute_force_softmax, {}),
        ("window one frame short", attention, "frame_visible", window_one_short,
         TWIN.test_full_window_has_constant_frame_count, {}),
        ("sink frames ignored", attention, "frame_visible", sinks_ignored,
         TWIN.test_full_window_has_constant_frame_count, {}),
        ("per-head P.V rule inverted", quant, "pv_modes_auto",
         lambda a: np.where(np.all(np.asarray(a) == 0, axis=-1), PV_16, PV_FP8),
         TAUTO.test_auto_is_each_head_in_its_own_mode, {}),
        ("per-head P.V rule blind to channels moved towards Q", quant, "pv_modes_auto",
         lambda a: np.where(np.all(np.asarray(a) <= 0, axis=-1), PV_FP8, PV_16),
         TAUTO.test_rule_switches_at_the_exact_ratios, {}),
    ]


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pin_fails_on_planted_mistake(case, monkeypatch):
    _, module, name, wrong, pin, kwargs = case
    assert hasattr(module, name)
    monkeypatch.setattr(module, name, wrong)
    with pytest.raises(AssertionError):
        pin(**kwargs)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pin_passes_on_the_oracle(case):
    """The same pins pass on the oracle as it is (the failure above is the
    planted mistake's, not the pin's)."""
    *_, pin, kwargs = case
    pin(**kwargs)
