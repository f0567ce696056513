"""Pins for the float64 reference attention and the quantized emulation.

Reference attention (oracle/attention.py) is checked against pure-Python
loops with math.exp, closed forms (two keys reduce to a sigmoid, constant V,
Q = 0) and invariants (rows sum to 1, key permutation, subtracting a vector
from every key).  The emulation (oracle/emulate.py) is checked against closed
forms that fix its mask count and normalisation (Q = 0), against textbook
attention on exactly representable inputs, and against textbook attention on
the dequantized operands, where only the rounding of P may separate them.
"""

import math

import numpy as np
import pytest

from oracle import attention, emulate, quant, codecs
from oracle.constants import PV_16, PV_FP8, BK


def _loops_attention(Q, K, V, scale, vis):
    R, d = Q.shape
    out = np.zeros((R, V.shape[1]))
    for i in range(R):
        logits = [sum(Q[i, c] * K[j, c] for c in range(d)) * scale if vis[i, j] else None
                  for j in range(K.shape[0])]
        mx = max(x for x in logits if x is not None)
        w = [math.exp(x - mx) if x is not None else 0.0 for x in logits]
        s = sum(w)
        for j, wj in enumerate(w):
            out[i] += wj / s * V[j]
    return out


@pytest.mark.parametrize("frame_len", [0, 3])
def test_fp64_attention_matches_python_loops(frame_len):
    rng = np.random.default_rng(20)
    Nq, Nkv, d = 5, 12, 4
    Q, K, V = (rng.standard_normal((1, 1, n, d)) for n in (Nq, Nkv, Nkv))
    kv = [11]
    qp = [4]
    got = attention.attention_fp64(Q, K, V, 0.7, frame_len, kv, qp)
    vis = attention.visible(np.arange(Nq), Nkv, kv[0], qp[0], frame_len)
    ref = _loops_attention(Q[0, 0], K[0, 0], V[0, 0], 0.7, vis)
    np.testing.assert_allclose(got[0, 0], ref, rtol=0, atol=1e-12)


def test_mask_rule_by_enumeration():
    F, kv, qp = 4, 14, 5
    rows = np.arange(6)
    vis = attention.visible(rows, 16, kv, qp, F)
    for i in rows:
        for j in range(16):
            expect = j < kv and (j // F) <= ((qp + i) // F)
            assert vis[i, j] == expect
        assert attention.row_end([i], kv, qp, F)[0] == vis[i].sum()


def test_fp64_attention_invariants():
    rng = np.random.default_rng(21)
    Q, K, V = (rng.standard_normal((1, 2, 9, 6)) for _ in range(3))
    ones = np.ones_like(V)
    np.testing.assert_allclose(attention.attention_fp64(Q, K, ones), 1.0, atol=1e-12)
    const = np.broadcast_to(rng.standard_normal(6), V.shape)
    np.testing.assert_allclose(attention.attention_fp64(Q, K, const),
                               np.broadcast_to(const[:, :, :9], (1, 2, 9, 6)), atol=1e-12)
    perm = rng.permutation(9)
    np.testing.assert_allclose(attention.attention_fp64(Q, K[:, :, perm], V[:, :, perm]),
                               attention.attention_fp64(Q, K, V), atol=1e-12)
    shift = rng.standard_normal((1, 2, 1, 6)) * 5
    np.testing.assert_allclose(attention.attention_fp64(Q, K - shift, V),
                               attention.attention_fp64(Q, K, V), atol=1e-12)


def test_fp64_attention_two_keys_is_sigmoid():
    q = np.array([[[[0.3, -1.2]]]])
    k = np.array([[[[1.0, 0.5], [-0.4, 2.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    out = attention.attention_fp64(q, k, v, 1.0)
    z = (q[0, 0, 0] @ k[0, 0, 0]) - (q[0, 0, 0] @ k[0, 0, 1])
    w0 = 1 / (1 + math.exp(-z))
    np.testing.assert_allclose(out[0, 0, 0], [w0, 1 - w0], atol=1e-15)


# --------------------------------------------------------------- emulation

def _inputs(rng, B, H, Nq, Nkv, d, dtype):
    rnd = codecs.round_bf16 if dtype == "bf16" else codecs.round_f16
    Q = rnd(rng.standard_normal((B, H, Nq, d)).astype(np.float32))
    K = rnd((rng.standard_normal((B, H, Nkv, d)) + rng.standard_normal((1, H, 1, d))).astype(np.float32))
    V = rnd(rng.standard_normal((B, H, Nkv, d)).astype(np.float32))
    return Q, K, V


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
@pytest.mark.parametrize("frame_len", [0, 50])
def test_emulation_q_zero_is_mean_of_visible_v(pv_mode, frame_len):
    """Q = 0: every logit is 0, p = 2^s exactly, O = mean of visible V^ rows."""
    rng = np.random.default_rng(22)
    B, H, Nq, Nkv, d = 2, 2, 70, 260, 16
    _, K, V = _inputs(rng, B, H, Nq, Nkv, d, "bf16")
    Q = np.zeros((B, H, Nq, d), np.float32)
    kv = [260, 199]
    mu = quant.k_mean(K, kv)
    qc, dq = quant.quantize_q(Q)
    kc, dk = quant.quantize_k(K, mu, kv)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(V, kv)
        Vh = quant.dequant_v_fp8(vc, ve)
    else:
        Vh = V.astype(np.float64)
    qp = [kv[0] - Nq, kv[1] - Nq]
    o64, _ = emulate.sage_attention_emulated(qc, dq, kc, dk, Vh, pv_mode, "bf16",
                                             frame_len=frame_len, kv_len=kv, q_pos0=qp)
    for b in range(B):
        ends = attention.row_end(np.arange(Nq), kv[b], qp[b], frame_len)
        for i in range(Nq):
            ref = Vh[b, :, :ends[i]].mean(axis=1)
            np.testing.assert_allclose(o64[b, :, i], ref, rtol=0, atol=1e-12)


def test_emulation_exact_inputs_match_textbook_attention():
    """Inputs whose quantization is exact (integers times 2^k, zero-mean K
    columns, balanced channel ranges): the emulation differs from float64
    attention only by the rounding of P (fp16 here, relative 2^-11)."""
    rng = np.random.default_rng(23)
    Nq = Nkv = 192
    d = 16
    q = rng.integers(-127, 128, (1, 1, Nq, d))
    q[0, 0, 0, :] = 127
    k = rng.integers(-127, 128, (1, 1, Nkv // 2, d))
    k = np.concatenate([k, -k], axis=2)             # zero column means
    k[0, 0, 0, :] = 127
    k[0, 0, Nkv // 2, :] = -127
    Q = np.ldexp(q.astype(np.float32), -7)
    K = np.ldexp(k.astype(np.float32), -7)
    V = codecs.round_f16(rng.standard_normal((1, 1, Nkv, d)).astype(np.float32))
    mu = quant.k_mean(K)
    assert not mu.any()
    a = quant.channel_shift(Q, K, mu)
    assert not a.any()
    o64, _ = emulate.emulate_from_inputs(Q, K, V, PV_16, "f16", sm_scale=0.05)
    ref = attention.attention_fp64(Q, K, V, 0.05)
    np.testing.assert_allclose(o64, ref, rtol=0, atol=4 * 2.0 ** -11 * np.abs(V).max())


@pytest.mark.parametrize("pv_mode,dtype,eps", [(PV_16, "f16", 2.0 ** -11), (PV_16, "bf16", 2.0 ** -8),
                                               (PV_FP8, "bf16", 2.0 ** -4)])
def test_emulation_equals_attention_on_dequantized_operands(pv_mode, dtype, eps):
    """Textbook attention on Q'=dq*qcodes, K'=dk*kcodes, V^ differs from the
    emulation only by P's rounding.  With p~ = p (1 + e_j), |e_j| <= eps, and l
    summing p~, diff_i = sum_j p_j e_j (v_j - ref_i) / sum_j p~_j, so
    |diff| <= eps / (1 - eps) * max_j |v_j - ref_i| <= 2 eps max|V^| (1 + eps)."""
    rng = np.random.default_rng(24)
    B, H, Nq, Nkv, d = 1, 2, 150, 333, 32
    Q, K, V = _inputs(rng, B, H, Nq, Nkv, d, dtype)
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    qc, dq = quant.quantize_q(Q, a)
    kc, dk = quant.quantize_k(K, mu, None, a)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(V)
        Vh = quant.dequant_v_fp8(vc, ve)
    else:
        Vh = V.astype(np.float64)
    o64, _ = emulate.sage_attention_emulated(qc, dq, kc, dk, Vh, pv_mode, dtype, sm_scale=0.3)
    Qd = qc * np.repeat(dq, 128, axis=2)[:, :, :Nq, None].astype(np.float64)
    Kd = kc * np.repeat(dk, 64, axis=2)[:, :, :Nkv, None].astype(np.float64)
    ref = attention.attention_fp64(Qd, Kd, Vh, 0.3)
    bound = 2 * eps * np.abs(Vh).max() * 1.01 + 1e-12
    assert np.abs(o64 - ref).max() <= bound
    # and the difference is real rounding noise, not a systematic error
    assert np.abs(o64 - ref).mean() < 0.25 * bound


def test_emulation_splits_agree_and_p_stays_in_range():
    rng = np.random.default_rng(25)
    Q, K, V = _inputs(rng, 1, 1, 64, 1000, 16, "bf16")
    Q *= 4                                          # peaky rows: the lazy max moves
    one, _ = emulate.emulate_from_inputs(Q, K, V, PV_FP8, "bf16")
    nch = -(-1000 // BK)
    two, _ = emulate.emulate_from_inputs(Q, K, V, PV_FP8, "bf16",
                                         splits=[(0, 5), (5, 11), (11, nch)])
    assert np.abs(one - two).max() <= 2.0 ** -4 * np.abs(V).max()
    ref = attention.attention_fp64(Q, K, V)
    cos = (one * ref).sum() / np.sqrt((one ** 2).sum() * (ref ** 2).sum())
    assert cos > 0.998


def test_scores_int_brute_force():
    rng = np.random.default_rng(26)
    q = rng.integers(-127, 128, (7, 64)).astype(np.int8)
    k = rng.integers(-127, 128, (9, 64)).astype(np.int8)
    s = emulate.scores_int(q, k)
    for i in range(7):
        for j in range(9):
            assert s[i, j] == sum(int(a) * int(b) for a, b in zip(q[i], k[j]))
    assert np.abs(emulate.scores_int(np.full((1, 128), -127, np.int8),
                                     np.full((1, 128), 127, np.int8))) == 127 * 127 * 128


def test_lazy_running_max_policy_by_hand():
    """Chunk maxima 0, 3, 6, 5, 11, 14.5 (log2 units) with TAU = 4: the row
    keeps m = 0 through the 3, adopts 6 (> 0 + 4), keeps it through 5,
    adopts 11, keeps it through 14.5 (not > 15).  Values worked out by hand
    from the rule in the module docstring."""
    from oracle.emulate import _run_rows
    maxima = [0.0, 3.0, 6.0, 5.0, 11.0, 14.5]
    S = np.full((1, 64 * len(maxima)), -40.0)
    for t, mx in enumerate(maxima):
        S[0, 64 * t + 7] = mx * 2                  # integer scores, c = 0.5
    trace = []
    V = np.ones((S.shape[1], 4))
    st = _run_rows(S, np.array([0.5], np.float32), np.ones(len(maxima), np.float32),
                   np.array([S.shape[1]]), V, 0, len(maxima), PV_16, "bf16", trace)
    l, acc = st.l, st.acc
    assert [float(x[0]) for x in trace] == [0.0, 0.0, 6.0, 6.0, 11.0, 11.0]
    # l sums the rounded weights: all-ones V gives exactly 1
    np.testing.assert_allclose(acc / l[:, None], 1.0, rtol=0, atol=1e-15)


@pytest.mark.parametrize("pv_mode,dtype", [(PV_16, "bf16"), (PV_16, "f16"), (PV_FP8, "bf16")])
@pytest.mark.parametrize("frame_len", [0, 64])
def test_emulation_constant_v_columns_pass_through(pv_mode, dtype, frame_len):
    """l sums exactly the weights that multiply V^, so each output row is a
    convex combination of visible V^ rows: a V whose every key row is the
    same vector comes out as that vector's V^ (FP8: its e4m3 x E8M0 value),
    bit-exactly after rounding to the output type, whatever Q and K are."""
    rng = np.random.default_rng(27)
    B, H, Nq, Nkv, d = 1, 2, 100, 300, 32
    Q, K, _ = _inputs(rng, B, H, Nq, Nkv, d, dtype)
    Q *= 3                                          # peaky rows: the lazy max moves
    row = codecs.round_to(rng.standard_normal((1, H, 1, d)).astype(np.float32), dtype)
    V = np.broadcast_to(row, (B, H, Nkv, d)).copy()
    kv = [Nkv]
    o64, o = emulate.emulate_from_inputs(Q, K, V, pv_mode, dtype, frame_len=frame_len, kv_len=kv)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(V, kv)
        want = quant.dequant_v_fp8(vc, ve)[:, :, :1]
    else:
        want = V[:, :, :1].astype(np.float64)
    want = codecs.round_to(want.astype(np.float32), dtype)
    assert np.array_equal(o, np.broadcast_to(want, o.shape))


@pytest.mark.parametrize("pv_mode,dtype", [(PV_16, "bf16"), (PV_16, "f16"), (PV_FP8, "bf16")])
def test_sensitivity_bound_holds_under_perturbed_exponents(pv_mode, dtype):
    """An implementation whose exponent argument is off by up to dx and whose
    2^x is off by up to rel_exp (relative) rounds some p differently; the
    emulation's 'flip' bound must contain every such output.  The perturbed
    runs push each x towards a rounding boundary by (almost) the full slack,
    in random directions, with splits and frames, and the slack is made
    large (many flips) so that a missing term of the bound shows."""
    rng = np.random.default_rng(28)
    B, H, Nq, Nkv, d = 2, 2, 70, 400, 32
    Q, K, V = _inputs(rng, B, H, Nq, Nkv, d, dtype)
    Q *= 2
    kv, F = [400, 333], 64
    slack = emulate.Slack(lambda c, mref, x: 2e-3 + 1e-4 * np.abs(x), 1e-3)
    sp = [emulate.split_ranges(k, 3) for k in kv]
    o, _, aux = emulate.emulate_from_inputs(Q, K, V, pv_mode, dtype, frame_len=F, kv_len=kv,
                                            splits=sp, slack=slack)
    flip = aux["flip"]
    assert np.all(flip >= 0) and flip.max() > 0
    worst = 0.0
    for trial in range(4):
        r = np.random.default_rng(100 + trial)

        def perturb(x, c, mref):
            x64 = x.astype(np.float64)
            dx = 0.999 * (2e-3 + 1e-4 * np.abs(x64))
            sgn = r.choice([-1.0, 1.0], size=x.shape)
            eps = r.uniform(-0.999e-3, 0.999e-3, size=x.shape)
            # float32 rounding of x' stays inside the slack (0.1% margin)
            return (x64 + sgn * dx + np.log2(1 + eps)).astype(np.float32)

        o2, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, dtype, frame_len=F, kv_len=kv,
                                            splits=sp, perturb=perturb)
        d_ = np.abs(o2 - o)
        assert np.all(d_ <= flip * (1 + 1e-9) + 1e-15)
        worst = max(worst, float((d_ / np.where(flip > 0, flip, 1)).max()))
    assert worst > 0.02       # the perturbations really moved outputs towards the bound


def test_sensitivity_sums_match_their_definitions():
    """'a' is the emulation run on |V| (the same weights times |V^|); with no
    slack nothing can flip; nvis counts each row's visible keys."""
    rng = np.random.default_rng(29)
    Q, K, V = _inputs(rng, 1, 2, 50, 300, 16, "bf16")
    kv, F = [290], 64
    zero = emulate.Slack(lambda c, mref, x: np.zeros_like(x, dtype=np.float64), 0.0, flush=False)
    for pv_mode in (PV_16, PV_FP8):
        o, _, aux = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", frame_len=F, kv_len=kv, slack=zero)
        oa, _ = emulate.emulate_from_inputs(Q, K, np.abs(V), pv_mode, "bf16", frame_len=F, kv_len=kv)
        assert np.array_equal(aux["a"], oa)
        assert not aux["flip"].any()
        assert np.array_equal(aux["nvis"][0, 0], attention.row_end(np.arange(50), 290, 240, F))


def test_sensitivity_bound_ignores_masked_keys():
    """Under a causal frame mask a row's invisible keys may score far above
    its running max (their exponent argument exceeds the range of P); they
    take no part in the bound.  Keys of later frames are made to dominate."""
    rng = np.random.default_rng(30)
    Q, K, V = _inputs(rng, 1, 1, 200, 300, 16, "bf16")
    Q[..., 0] = 8.0
    K[0, 0, 200:, 0] = 12.0      # frame 2: seen by the rows of frame 2 only, in chunks shared with frame 1
    slack = emulate.Slack(lambda c, mref, x: 1e-3 + 0 * x, 1e-4)
    for pv_mode in (PV_16, PV_FP8):
        o, _, aux = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", frame_len=100, kv_len=[300],
                                                q_pos0=[100], slack=slack)
        assert np.isfinite(aux["flip"]).all()
