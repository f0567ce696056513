"""Pins of the oracle's sliding-window / sink mask and its frame cache (whole
frames quantized once into padded slots).  Streaming decoding attends to a
fixed window -- sink frames, the most recent history frames and the current
frame -- over cached history (Vidu S1 blog, section "Infra")."""

import numpy as np
import pytest

from oracle import attention, quant, emulate, codecs
from oracle.constants import PV_16, PV_FP8, BK


def _rnd16(x, dtype="bf16"):
    return codecs.round_to(np.asarray(x, np.float32), dtype)


def test_window_covering_all_history_is_the_causal_mask():
    F, kv = 10, 95
    rows = np.arange(60)
    base = attention.visible(rows, 100, kv, 35, F)
    for S in (0, 1, 3):
        wide = attention.visible(rows, 100, kv, 35, F, sink_frames=S, window_frames=10)
        assert np.array_equal(base, wide)


def test_full_window_has_constant_frame_count():
    """Once the query frame is past the sinks and the window, exactly
    S + W + 1 frames are visible, whatever the frame index."""
    F, S, W = 7, 2, 3
    for fq in range(S + W, 40):
        i = np.arange(F) + fq * F                      # the rows of query frame fq
        vis = attention.visible(i - 0, (fq + 1) * F, (fq + 1) * F, 0, F, S, W)
        frames = {int(j) // F for j in np.nonzero(vis[0])[0]}
        assert len(frames) == S + W + 1
        assert frames == set(range(S)) | set(range(fq - W, fq + 1))
        assert (vis == vis[0]).all()                   # same for every row of the frame


def test_window_attention_equals_softmax_over_gathered_frames():
    rng = np.random.default_rng(41)
    F, S, W, nf, d = 6, 1, 2, 9, 8
    K = rng.standard_normal((1, 1, nf * F, d))
    V = rng.standard_normal((1, 1, nf * F, d))
    Q = rng.standard_normal((1, 1, 2 * F, d))           # the last two frames' queries
    q0 = (nf - 2) * F
    got = attention.attention_fp64(Q, K, V, 0.4, frame_len=F, kv_len=[nf * F], q_pos0=[q0],
                                   sink_frames=S, window_frames=W)
    for i in range(2 * F):
        fq = (q0 + i) // F
        frames = sorted(set(range(S)) | set(range(max(0, fq - W), fq + 1)))
        idx = np.concatenate([np.arange(f * F, f * F + F) for f in frames])
        s = Q[0, 0, i] @ K[0, 0, idx].T * 0.4
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ V[0, 0, idx]
        np.testing.assert_allclose(got[0, 0, i], ref, rtol=0, atol=1e-13)


def test_frame_cache_without_padding_equals_contiguous_quantization():
    rng = np.random.default_rng(42)
    F = 2 * BK
    K = _rnd16(rng.standard_normal((2, 3, 5 * F, 16)) + rng.standard_normal((1, 3, 1, 16)))
    V = _rnd16(rng.standard_normal((2, 3, 5 * F, 16)))
    mu = quant.k_mean(K)
    a = rng.integers(-2, 3, (2, 3, 16))
    c1, d1 = quant.quantize_k_frames(K, mu, a, F, F)
    c2, d2 = quant.quantize_k(K, mu, None, a)
    assert np.array_equal(c1, c2) and np.array_equal(d1, d2)
    v1, e1 = quant.quantize_v_fp8_frames(V, F, F)
    v2, e2, _ = quant.quantize_v_fp8(V)
    assert np.array_equal(v1, v2) and np.array_equal(e1, e2)


def test_partly_written_frames_equal_contiguous_quantization_with_kv_len():
    """A frame cache holding kv_len[b] tokens quantizes like the contiguous
    path with the same kv_len: tokens past it are padding (zero codes, outside
    every amax), also inside the frame that holds the boundary."""
    rng = np.random.default_rng(43)
    F = 2 * BK
    K = _rnd16(rng.standard_normal((2, 3, 5 * F, 16)) + rng.standard_normal((1, 3, 1, 16)))
    V = _rnd16(rng.standard_normal((2, 3, 5 * F, 16)))
    kv = [300, 411]  # inside frames 2 and 3
    mu = quant.k_mean(K)
    a = rng.integers(-2, 3, (2, 3, 16))
    c1, d1 = quant.quantize_k_frames(K, mu, a, F, F, kv_len=kv)
    c2, d2 = quant.quantize_k(K, mu, kv, a)
    assert np.array_equal(c1, c2) and np.array_equal(d1, d2)
    assert not c1[0, :, 300:].any() and not c1[1, :, 411:].any()
    v1, e1 = quant.quantize_v_fp8_frames(V, F, F, kv_len=kv)
    v2, e2, _ = quant.quantize_v_fp8(V, kv)
    assert np.array_equal(v1, v2) and np.array_equal(e1, e2)
    # the stale tokens past kv_len change nothing
    K2, V2 = K.copy(), V.copy()
    K2[0, :, 300:] *= 40
    V2[1, :, 411:] *= 40
    assert np.array_equal(quant.quantize_k_frames(K2, mu, a, F, F, kv_len=kv)[0], c1)
    assert np.array_equal(quant.quantize_v_fp8_frames(V2, F, F, kv_len=kv)[1], e1)


def test_frame_cache_padding_and_append_once():
    """With padding (F = 200 tokens at a stride of 256 slots) the padding slots
    hold 0, and quantizing frames one at a time into the cache gives the same
    codes and scales as quantizing them all at once (no block is shared)."""
    rng = np.random.default_rng(43)
    F, FS, nf = 200, 256, 4
    K = _rnd16(rng.standard_normal((1, 2, nf * F, 32)) * 2)
    V = _rnd16(rng.standard_normal((1, 2, nf * F, 32)))
    mu = quant.k_mean(K)
    a = np.zeros((1, 2, 32), np.int64)
    ca, da = quant.quantize_k_frames(K, mu, a, F, FS)
    va, ea = quant.quantize_v_fp8_frames(V, F, FS)
    pad = (np.arange(nf * FS) % FS) >= F
    assert not ca[:, :, pad].any() and not va[:, :, pad].any()
    for f in range(nf):
        cf, df = quant.quantize_k_frames(K[:, :, f * F:(f + 1) * F], mu, a, F, FS)
        vf, ef = quant.quantize_v_fp8_frames(V[:, :, f * F:(f + 1) * F], F, FS)
        assert np.array_equal(ca[:, :, f * FS:(f + 1) * FS], cf)
        assert np.array_equal(da[:, :, f * FS // BK:(f + 1) * FS // BK], df)
        assert np.array_equal(va[:, :, f * FS:(f + 1) * FS], vf)
        assert np.array_equal(ea[:, :, f * FS // 32:(f + 1) * FS // 32], ef)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_cache_emulation_without_padding_equals_token_emulation(pv_mode):
    rng = np.random.default_rng(44)
    F, nf, d = BK * 2, 5, 32
    Q = _rnd16(rng.standard_normal((1, 2, F, d)))
    K = _rnd16(rng.standard_normal((1, 2, nf * F, d)) + 1.5)
    V = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    kw = dict(frame_len=F, kv_len=[nf * F], q_pos0=[(nf - 1) * F], mu=mu, shift=a)
    tok, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", **kw)
    cache, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", frame_stride=F, **kw)
    assert np.array_equal(tok, cache)


@pytest.mark.parametrize("pv_mode", [PV_16, PV_FP8])
def test_cache_emulation_q_zero_is_mean_over_window(pv_mode):
    """Q = 0: every visible p is equal, so each row is the mean of V^ over the
    visible tokens of the sink and window frames (padding never counted)."""
    rng = np.random.default_rng(45)
    F, FS, nf, S, W, d = 100, 128, 7, 1, 2, 16
    Q = np.zeros((1, 2, 2 * F, d), np.float32)
    K = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    V = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    mu = quant.k_mean(K)
    a = np.zeros((1, 2, d), np.int64)
    q0 = (nf - 2) * F
    o64, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", frame_len=F, kv_len=[nf * F],
                                         q_pos0=[q0], mu=mu, shift=a, frame_stride=FS,
                                         sink_frames=S, window_frames=W)
    if pv_mode == PV_FP8:
        vc, ve = quant.quantize_v_fp8_frames(V, F, FS)
        Vt = quant.dequant_v_fp8(vc, ve)[:, :, quant.frame_slot(np.arange(nf * F), F, FS)]
    else:
        Vt = V.astype(np.float64)
    for i in range(2 * F):
        fq = (q0 + i) // F
        frames = sorted(set(range(S)) | set(range(fq - W, fq + 1)))
        idx = np.concatenate([np.arange(f * F, f * F + F) for f in frames])
        np.testing.assert_allclose(o64[0, :, i], Vt[0][:, idx].mean(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("pv_mode,eps", [(PV_16, 2.0 ** -8), (PV_FP8, 2.0 ** -4)])
def test_cache_emulation_equals_attention_on_dequantized_operands(pv_mode, eps):
    """Textbook windowed attention on the dequantized cache operands differs
    from the emulation only by P's rounding (bound as in the dense case)."""
    rng = np.random.default_rng(46)
    F, FS, nf, S, W, d = 150, 192, 6, 1, 3, 32
    Q = _rnd16(rng.standard_normal((1, 2, F, d)))
    K = _rnd16(rng.standard_normal((1, 2, nf * F, d)) + rng.standard_normal((1, 2, 1, d)))
    V = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    q0 = (nf - 1) * F
    o64, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, "bf16", 0.3, frame_len=F, kv_len=[nf * F],
                                         q_pos0=[q0], mu=mu, shift=a, frame_stride=FS,
                                         sink_frames=S, window_frames=W)
    qc, dq = quant.quantize_q(Q, a)
    kc, dk = quant.quantize_k_frames(K, mu, a, F, FS)
    tok = quant.frame_slot(np.arange(nf * F), F, FS)
    Kd = (kc * np.repeat(dk, BK, axis=2)[..., None])[:, :, tok]
    Qd = qc * np.repeat(dq, 128, axis=2)[:, :, :F, None]
    if pv_mode == PV_FP8:
        vc, ve = quant.quantize_v_fp8_frames(V, F, FS)
        Vh = quant.dequant_v_fp8(vc, ve)[:, :, tok]
    else:
        Vh = V.astype(np.float64)
    ref = attention.attention_fp64(Qd, Kd, Vh, 0.3, frame_len=F, kv_len=[nf * F], q_pos0=[q0],
                                   sink_frames=S, window_frames=W)
    assert np.abs(o64 - ref).max() <= 2 * eps * np.abs(Vh).max() * 1.01


@pytest.mark.parametrize("F,FS,S,W,q0,Nq,kv,nsplit", [
    (200, 256, 1, 3, 1400, 200, 1600, 1), (200, 256, 1, 3, 1250, 350, 1600, 3),
    (100, 128, 2, 2, 300, 300, 600, 4), (64, 64, 4, 1, 64, 128, 192, 2),
    (150, 192, 2, 1, 1200, 150, 1350, 2), (200, 256, 0, 0, 1000, 200, 1200, 3),
    (2040, 2048, 1, 16, 40 * 2040, 2040, 41 * 2040, 3), (2040, 2048, 1, 16, 40 * 2040, 2040, 41 * 2040, 16),
    (2040, 2048, 1, 4, 8 * 2040 + 1740, 600, 9 * 2040 + 340, 5), (150, 192, 3, 2, 0, 450, 450, 3)])
def test_cache_splits_cover_exactly_the_visible_chunks(F, FS, S, W, q0, Nq, kv, nsplit):
    """Brute force over slots, for the batch's whole query range: the split
    ranges are disjoint and ascending, they cover every chunk holding a slot
    that some query row sees, every chunk they cover that no row sees lies in
    the gap between the sink frames and the window, and there are
    min(nsplit, list length) of them."""
    nslots = -(-kv // F) * FS
    rows = np.arange(Nq)
    vis = emulate.visible_slots(rows, nslots, kv, q0, F, FS, S, W)
    vis_chunk = vis.reshape(len(rows), -1, BK).any(axis=(0, 2))
    a0, b1, end = emulate.cache_list(Nq, q0, kv, F, FS, S, W)
    listed = np.zeros(vis_chunk.size, bool)
    listed[:a0] = True
    listed[b1:end] = True
    assert np.array_equal(listed, vis_chunk)      # the list is exactly the visible chunks
    sp = emulate.cache_splits(Nq, q0, kv, F, FS, S, W, nsplit)
    if nsplit == 1:
        assert sp is None
        return
    covered = np.zeros(vis_chunk.size, bool)
    prev_hi = 0
    for lo, hi in sp:
        assert prev_hi <= lo < hi
        covered[lo:hi] = True
        prev_hi = hi
    assert not (vis_chunk & ~covered).any()
    extra = np.nonzero(covered & ~vis_chunk)[0]
    assert np.all((extra >= a0) & (extra < b1))
    assert len(sp) == min(nsplit, int(vis_chunk.sum()))


def test_cache_emulation_splits_merge_to_the_unsplit_result():
    """Each split work item keeps its own running max, so P is rounded against
    another reference than in one pass: the merged result differs from the
    unsplit one only within P's rounding (2^-8 relative in 16-bit mode, on
    each side of textbook attention on the same operands)."""
    rng = np.random.default_rng(47)
    F, FS, nf, S, W, d = 150, 192, 6, 1, 3, 32
    Q = _rnd16(rng.standard_normal((1, 2, 2 * F, d)))
    K = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    V = _rnd16(rng.standard_normal((1, 2, nf * F, d)))
    mu = quant.k_mean(K)
    a = quant.channel_shift(Q, K, mu)
    args = (Q, K, V, PV_16, "bf16", F, FS, S, W, [nf * F], [(nf - 2) * F], mu, a)
    o1 = emulate.emulate_frame_cache(*args, 1)[0]
    o3 = emulate.emulate_frame_cache(*args, 3, rows=np.arange(0, 2 * F, 7))[0]
    assert np.abs(o3 - o1[:, :, ::7]).max() <= 2 * 2 * 2.0 ** -8 * np.abs(V).max()
    assert not np.array_equal(o3, o1[:, :, ::7])  # the split ranges were really taken
