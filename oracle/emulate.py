"""Quantized attention, emulated on the CPU step by step.

Test infrastructure: only tests/, the smoke check and the bench's CPU
baseline use this module; the library never does.

The pages describe SageAttention only as low-bit quantized attention that
keeps the output of the FlashAttention it replaces ("37:54 One line of code,
twice the speed"; "02:48 There were clearly faster compute units on the
hardware").  This module is the library's own stated algorithm, written out
step by step in the precision the scheme fixes:

Given the INT8 codes and scales of ``quant`` (and V^, the P.V operand:
V itself in 16-bit mode, or its dequantized FP8 codes), for every query row i
of head (b,h), with state m = -inf, l = 0, acc = 0, the keys are taken in
chunks of BK = 64 (chunk t = keys [64t, 64t+64)), in ascending order:

  1. S[i,j]   = sum_c qcode[i,c] * kcode[j,c]            (exact integers)
  2. sigma    = fp32(sm_scale * log2 e);  qs = fp32(dq[i // 128] * sigma)
     c_t      = fp32(qs * dk[t])             (log2-domain scale of chunk t)
  3. tm       = max over visible j of fp32(S[i,j] * c_t)  (-inf if none)
  4. lazy running max: if tm > fp32(m + TAU) the row adopts m' = tm and
     rescales its state by alpha = fp32(2^fp32(m - m')) (0 when m = -inf);
     otherwise m, l and acc are kept as they are.
  5. x[i,j]   = fp32(S[i,j] * c_t - mref), rounded once from the exact value
              (|S| < 2^24, so S is a float32 and this is a fused multiply-add),
     with mref = fp32(m - s) (s = 4 in FP8 mode, 0 in 16-bit mode);
     p = fp32(2^x), 0 if not visible.
  6. p~       = p rounded to the P.V operand type: e4m3fn in FP8 mode (where
     p already carries the 2^s pre-scale), else the input's fp16/bf16
  7. l       += sum_j p~                     (the rounded operand itself)
  8. acc     += sum_j p~[i,j] * V^[j,:]
Finally O[i] = acc / l; the 2^s pre-scale cancels in that ratio.  Under
PV_AUTO every (b,h) runs these steps in the mode quant.pv_modes_auto gives it.  The output
is rounded (RNE) to the input dtype.  Because l sums exactly the weights that
multiply V^, every output row is a convex combination of the visible V^ rows
(a constant V^ column comes out unchanged).

Because m only moves when a chunk maximum exceeds it by more than TAU, the
exponent argument is at most TAU + s = 8, so p~ never exceeds 2^8 -- inside
both e4m3fn (448) and the 16-bit types.

Split-KV: each batch's key chunks form one ordered list (``split_ranges``,
``cache_splits``); split s takes entries [s*n/S, (s+1)*n/S) of it, runs steps
1-8 from a fresh state, and the partial results are merged exactly (float64):
M = max_s m_s, O = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  Where
the cut falls changes which keys share a running max, hence how P rounds; the
list depends only on the batch (its key range, frames and window), not on how
query rows are grouped into work.

Accumulations (l, acc) are float64 here.

Sensitivity bound.  An implementation that evaluates step 5 with extra
rounding (its exponent argument within dx of x) and 2^x with a relative error
up to rel_exp can round some p differently in step 6, because p~ is a
rounding of p: such a flip moves p~ by one step of the P.V operand type.  With
``slack`` given, the emulation also carries, per row, the interval of every
p~ reachable that way -- W_j = round(p_hi) - round(p_lo), rounding being
monotone -- and returns the bound that follows from
O' - O = sum_j (p~'_j - p~_j)(V^_j - O) / l':
    |O' - O| <= (sum_j W_j |V^_j| + |O| sum_j W_j) / (l - sum_j W_j),
both sums taken with the same rescalings and split weights as acc and l.
"""

import numpy as np

from .constants import BQ, BK, TAU, PSHIFT_FP8, PSHIFT_16, LOG2E, PV_16, PV_FP8, PV_AUTO
from . import codecs
from .fp32 import fma_f32
from .attention import row_end, default_q_pos0

_F32 = np.float32


def log2_scale(sm_scale, d):
    """sigma = fp32(float64(sm_scale) * log2 e); sm_scale 0/None -> 1/sqrt(d)."""
    if not sm_scale:
        sm_scale = float(_F32(1.0 / np.sqrt(d)))
    return _F32(np.float64(_F32(sm_scale)) * LOG2E)


def exponent_arg(S, c_t, mref):
    """Step 5: x = fp32(S c_t - mref), one rounding (rows of S pair with
    entries of c_t and mref; S integer scores, |S| < 2^24)."""
    S = np.asarray(S, dtype=np.float64)
    if np.any(np.abs(S) >= 2.0 ** 24):
        raise ValueError("score outside float32's exact integers")
    R, n = S.shape
    c = np.broadcast_to(np.asarray(c_t, _F32)[:, None], (R, n))
    k = np.broadcast_to((-np.asarray(mref, _F32))[:, None], (R, n))
    return fma_f32(S.astype(_F32), c, k)


class Slack:
    """How far an implementation may deviate from steps 4-5 (see the module
    docstring): dx(c_t, mref, x) -> per-element bound on |x' - x| (arrays of
    shape [R, n] from c_t, mref [R] and x [R, n]); rel_exp: relative error of
    its 2^x (and of alpha and the split weights); flush: results below 2^-126
    may be flushed to zero."""

    def __init__(self, dx, rel_exp, flush=True):
        self.dx = dx
        self.rel_exp = float(rel_exp)
        self.flush = flush


class _State:
    """Running state of a set of rows: m, l, acc, and with ``aux`` the sums
    that bound an implementation's deviation: a = sum p~ |V^| (rows x d),
    wl = sum W, wa = sum W |V^|, and the visible-key count."""

    def __init__(self, R, d, aux):
        self.m = np.full(R, -np.inf, dtype=_F32)
        self.l = np.zeros(R, dtype=np.float64)
        self.acc = np.zeros((R, d), dtype=np.float64)
        self.aux = aux
        if aux:
            self.a = np.zeros((R, d))
            self.wl = np.zeros(R)
            self.wa = np.zeros((R, d))
            self.nvis = np.zeros(R, dtype=np.int64)
            self.nres = np.zeros(R, dtype=np.int64)

    def scale(self, alpha):
        self.l = self.l * alpha
        self.acc = self.acc * alpha[:, None]
        if self.aux:
            self.a = self.a * alpha[:, None]
            self.wl = self.wl * alpha
            self.wa = self.wa * alpha[:, None]


def _round_p(p, pv_mode, p_dtype):
    """Step 6 on float64 values (monotone in p)."""
    if pv_mode == PV_FP8:
        return codecs.round_e4m3(p)
    return codecs.round_to(p.astype(_F32), p_dtype).astype(np.float64)


def _run_rows(S_full, c_row, dk_bh, vis_end, Vhat_bh, chunk_lo, chunk_hi,
              pv_mode, p_dtype, trace=None, slack=None, perturb=None):
    """Steps 1-8 over chunks [chunk_lo, chunk_hi) for a set of rows.

    vis_end: per row, the exclusive end of its visible key prefix; or a
    boolean [R, keys] visibility matrix.
    trace: optional list; receives the running max m after every chunk.
    slack: optional ``Slack``; the state then carries the deviation sums.
    perturb: test hook, f(x, c_t, mref) -> x' standing in for an
    implementation's step 5 (its result is then rounded by exp2 as usual).
    Returns the final ``_State``.
    """
    vis_end = np.asarray(vis_end)
    R = S_full.shape[0]
    d = Vhat_bh.shape[1]
    st = _State(R, d, slack is not None)
    for t in range(chunk_lo, chunk_hi):
        j0 = t * BK
        j1 = min(j0 + BK, S_full.shape[1])
        if j0 >= j1:
            break
        j = np.arange(j0, j1)
        vis = vis_end[:, j0:j1] if vis_end.ndim == 2 else j[None, :] < vis_end[:, None]
        if not vis.any():
            continue
        c_t = (c_row * _F32(dk_bh[t])).astype(_F32)          # [R] fp32
        _chunk_step(S_full[:, j0:j1], c_t, vis, st, Vhat_bh[j0:j1], pv_mode, p_dtype, slack, perturb)
        if trace is not None:
            trace.append(st.m.copy())
    return st


def _chunk_step(S, c_t, vis, st, Vc, pv_mode, p_dtype, slack=None, perturb=None):
    """Steps 3-8 for one chunk; c_t is per row (rows may span Q blocks)."""
    shift = PSHIFT_FP8 if pv_mode == PV_FP8 else PSHIFT_16
    m = st.m
    logit = (S * c_t.astype(np.float64)[:, None]).astype(_F32)       # exact product, one rounding
    tm = np.where(vis, logit, -np.inf).max(axis=1).astype(_F32)
    upd = tm > (m + _F32(TAU)).astype(_F32)
    with np.errstate(invalid="ignore"):
        diff = (m - tm).astype(_F32)
    alpha = np.where(np.isneginf(m), _F32(0.0),
                     np.exp2(np.where(upd, diff, _F32(0)).astype(np.float64)).astype(_F32))
    alpha = np.where(upd, alpha, _F32(1.0)).astype(np.float64)
    st.m = m = np.where(upd, tm, m).astype(_F32)
    st.scale(alpha)
    # a row still at m = -inf has no visible key in this chunk; its p is 0
    mref = np.where(np.isneginf(m), _F32(0.0), (m - _F32(shift)).astype(_F32)).astype(_F32)
    x = exponent_arg(S, c_t, mref)
    if perturb is not None:
        x = np.asarray(perturb(x, c_t, mref), dtype=_F32)
    p = np.exp2(x.astype(np.float64)).astype(_F32)
    p = np.where(vis, p, _F32(0.0))
    pt = _round_p(p.astype(np.float64), pv_mode, p_dtype)
    st.l = st.l + pt.sum(axis=1)
    st.acc = st.acc + pt @ Vc
    if st.aux:
        x64 = x.astype(np.float64)
        dx = np.asarray(slack.dx(c_t, mref, x), dtype=np.float64)
        r = slack.rel_exp
        # masked keys take no part (their exponent argument is unbounded)
        lo = np.where(vis, np.exp2(x64 - dx) * (1 - r), 0.0)
        hi = np.where(vis, np.exp2(x64 + dx) * (1 + r), 0.0)
        if slack.flush:
            lo = np.where(lo < 2.0 ** -126, 0.0, lo)
        W = _round_p(hi, pv_mode, p_dtype) - _round_p(lo, pv_mode, p_dtype)
        aV = np.abs(Vc)
        st.a = st.a + pt @ aV
        st.wl = st.wl + W.sum(axis=1)
        st.wa = st.wa + W @ aV
        st.nvis = st.nvis + vis.sum(axis=1)
        st.nres = st.nres + upd


def split_ranges(kv_len_b, nsplit):
    """Chunk ranges of the KV splits over contiguous keys: the batch's chunks
    [0, ceil(kv_len/64)) cut into nsplit equal parts (split s takes
    [s*n/nsplit, (s+1)*n/nsplit)); None for one split."""
    n = -(-int(kv_len_b) // BK)
    if nsplit <= 1:
        return None
    return [(s * n // nsplit, (s + 1) * n // nsplit) for s in range(nsplit)]


def visible_slots(rows, n_slots, kv_len_b, q_pos0_b, frame_len, frame_stride,
                  sink_frames=0, window_frames=0):
    """Visibility [R, n_slots] of cache slots (frames of frame_len tokens at a
    stride of frame_stride slots) under the mask of ``attention.visible``;
    padding slots are never visible."""
    from .attention import frame_visible
    slot = np.arange(n_slots, dtype=np.int64)
    fk, r = slot // frame_stride, slot % frame_stride
    valid = (r < frame_len) & (fk * frame_len + r < int(kv_len_b))
    fq = (int(q_pos0_b) + np.asarray(rows, dtype=np.int64)) // frame_len
    return valid[None, :] & frame_visible(fk[None, :], fq[:, None], sink_frames, window_frames)


def sage_attention_emulated(qcodes, dq, kcodes, dk, Vhat, pv_mode, dtype,
                            sm_scale=None, frame_len=0, kv_len=None,
                            q_pos0=None, rows=None, splits=None,
                            frame_stride=0, sink_frames=0, window_frames=0,
                            block_mask=None, slack=None, perturb=None):
    """Emulate the quantized attention for the selected query rows.

    qcodes int8 [B,H,Nq,d], dq float32 [B,H,ceil(Nq/128)];
    kcodes int8 [B,H,Nkv,d], dk float32 [B,H,ceil(Nkv/64)];
    Vhat: the P.V right operand as exact values [B,H,Nkv,d] -- V (16-bit
    mode) or dequant_v_fp8(...) (FP8 mode);  dtype: 'bf16' | 'f16' (input and
    output type, and P's type in 16-bit mode).
    pv_mode: PV_16, PV_FP8, or an int array [B,H] giving each head's mode
    (Vhat[b,h] must then be that head's operand).
    splits: optional list of (chunk_lo, chunk_hi) ranges covering the keys,
    or a list of such lists, one per batch (see ``split_ranges`` and
    ``cache_splits``).
    frame_stride > 0: K/V operands are a frame cache (``quant.quantize_k_frames``
    layout: frame f's tokens at slots f*frame_stride + [0, frame_len)); kv_len and
    q_pos0 stay in tokens; sink_frames / window_frames restrict the visible
    frames as in ``attention.visible``.
    block_mask: optional [B,H,ceil(Nq/128),ceil(Nkv/64)] (contiguous keys);
    chunks of dropped tiles are skipped -- they change neither m, l nor acc,
    exactly as if they were absent -- and a row with no visible key gives 0.
    slack, perturb: see ``Slack`` and ``_run_rows``.
    Returns (O64 float64 [B,H,R,d], O rounded to dtype as float32); with
    slack, a third item: a dict of float64 arrays [B,H,R(,d)] -- 'a' =
    sum p~ |V^| / l, 'flip' = the sensitivity bound of the module docstring,
    'nvis' = visible keys of the row, 'nres' = rescales of its running max.
    """
    qcodes = np.asarray(qcodes)
    kcodes = np.asarray(kcodes)
    B, H, Nq, d = qcodes.shape
    Nkv = kcodes.shape[2]
    sigma = log2_scale(sm_scale, d)
    kv = np.full(B, Nkv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    qp = default_q_pos0(Nq, kv, frame_len) if q_pos0 is None else np.asarray(q_pos0, np.int64)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    nchunks = -(-Nkv // BK)
    pvm = np.broadcast_to(np.asarray(pv_mode, dtype=np.int64), (B, H))
    if splits is not None and len(splits) and isinstance(splits[0], tuple):
        splits = [splits] * B
    out = np.empty((B, H, len(rows), d), dtype=np.float64)
    if slack is not None:
        aux = {k: np.zeros((B, H, len(rows), d)) for k in ("a", "flip")}
        aux.update({k: np.zeros((B, H, len(rows)), np.int64) for k in ("nvis", "nres")})
    if window_frames and not frame_stride:
        raise ValueError("sink/window frames need the frame cache layout")
    if block_mask is not None and frame_stride:
        raise ValueError("a block mask needs contiguous keys")
    for b in range(B):
        if frame_stride:
            vis_end = visible_slots(rows, Nkv, kv[b], qp[b], frame_len, frame_stride,
                                    sink_frames, window_frames)
            last = np.nonzero(vis_end.any(axis=0))[0]
            jmax = int(last.max()) + 1 if last.size else 0
            vis_end = vis_end[:, :jmax]
        else:
            vis_end = row_end(rows, kv[b], qp[b], frame_len)
            jmax = int(vis_end.max())
        parts_b = [(0, nchunks)] if splits is None or splits[b] is None else splits[b]
        for h in range(H):
            vis_h = vis_end
            if block_mask is not None:
                from .attention import block_visible
                vis_h = block_visible(np.arange(jmax)[None, :] < vis_end[:, None], rows, block_mask[b, h])
            qs = (dq[b, h, rows // BQ].astype(_F32) * sigma).astype(_F32)   # [R]
            S_full = qcodes[b, h, rows, :].astype(np.float64) @ \
                kcodes[b, h, :jmax, :].astype(np.float64).T                # exact
            Vh = np.asarray(Vhat[b, h, :jmax, :], dtype=np.float64)
            parts = [_run_rows(S_full, qs, dk[b, h], vis_h, Vh, lo, hi, int(pvm[b, h]), dtype,
                               slack=slack, perturb=perturb)
                     for (lo, hi) in parts_b]
            ms = np.stack([p.m for p in parts]).astype(np.float64)         # [P, R]
            M = np.max(ms, axis=0)
            with np.errstate(invalid="ignore"):   # rows with no key at all: M = -inf
                w = np.where(np.isneginf(ms), 0.0, np.exp2(ms - M[None, :]))

            def merged(get, vec):
                tot = sum((w[i][:, None] if vec else w[i]) * get(p) for i, p in enumerate(parts))
                return tot

            L = merged(lambda p: p.l, False)
            num = merged(lambda p: p.acc, True)
            has = L > 0
            Ls = np.where(has, L, 1.0)
            O = np.where(has[:, None], num / Ls[:, None], 0.0)
            out[b, h] = O
            if slack is not None:
                WL = merged(lambda p: p.wl, False)
                aux["a"][b, h] = np.where(has[:, None], merged(lambda p: p.a, True) / Ls[:, None], 0.0)
                lo = np.maximum(L - WL, 0.0)
                flip = (merged(lambda p: p.wa, True) + np.abs(O) * WL[:, None])
                with np.errstate(divide="ignore", invalid="ignore"):
                    flip = np.where(flip > 0, flip / np.where(lo > 0, lo, 0.0)[:, None], 0.0)
                aux["flip"][b, h] = np.where(has[:, None], flip, 0.0)
                aux["nvis"][b, h] = sum(p.nvis for p in parts)
                aux["nres"][b, h] = sum(p.nres for p in parts)
    rounded = codecs.round_to(out.astype(_F32), dtype)
    if slack is not None:
        return out, rounded, aux
    return out, rounded


def scores_int(qcodes, kcodes):
    """Exact integer scores S = qcodes . kcodes^T for one (b,h): int64 [Nq,Nkv].

    Computed as a float64 matrix product of integer-valued operands, which is
    exact because |S| <= 127^2 * d < 2^53.
    """
    q = np.asarray(qcodes, dtype=np.float64)
    k = np.asarray(kcodes, dtype=np.float64)
    return (q @ k.T).astype(np.int64)


def emulate_from_inputs(Q, K, V, pv_mode, dtype, sm_scale=None, frame_len=0,
                        kv_len=None, q_pos0=None, rows=None, splits=None,
                        mu=None, shift=None, frame_stride=0, sink_frames=0,
                        window_frames=0, block_mask=None, slack=None, perturb=None):
    """Quantize the 16-bit inputs with ``quant`` and run the emulation.

    frame_stride > 0: K and V (tokens of whole frames from frame 0) go into a
    frame cache, each frame quantized once against the given (frozen) mu and
    shift (both required then).
    pv_mode PV_AUTO (contiguous keys only): each (b,h) in the mode
    quant.pv_modes_auto gives it; with slack, aux['pv_modes'] holds them."""
    from . import quant
    Qf = np.asarray(Q, dtype=np.float32)
    Kf = np.asarray(K, dtype=np.float32)
    Vf = np.asarray(V, dtype=np.float32)
    if frame_stride and pv_mode == PV_AUTO:
        raise ValueError("PV_AUTO needs contiguous keys")
    if frame_stride:
        qc, dq = quant.quantize_q(Qf, shift)
        kc, dk = quant.quantize_k_frames(Kf, mu, shift, frame_len, frame_stride, kv_len=kv_len)
        if pv_mode == PV_FP8:
            vc, ve = quant.quantize_v_fp8_frames(Vf, frame_len, frame_stride, kv_len=kv_len)
            Vhat = quant.dequant_v_fp8(vc, ve)
        else:
            Vhat = quant.to_frame_slots(Vf, frame_len, frame_stride).astype(np.float64)
        return sage_attention_emulated(qc, dq, kc, dk, Vhat, pv_mode, dtype, sm_scale,
                                       frame_len, kv_len, q_pos0, rows, splits,
                                       frame_stride, sink_frames, window_frames,
                                       slack=slack, perturb=perturb)
    if mu is None:
        mu = quant.k_mean(Kf, kv_len)
    a = quant.channel_shift(Qf, Kf, mu, kv_len) if shift is None else shift
    qc, dq = quant.quantize_q(Qf, a)
    kc, dk = quant.quantize_k(Kf, mu, kv_len, a)
    modes = quant.pv_modes_auto(a) if pv_mode == PV_AUTO else pv_mode
    Vhat = Vf.astype(np.float64)
    if np.any(np.asarray(modes) == PV_FP8):
        vc, ve, _ = quant.quantize_v_fp8(Vf, kv_len)
        V8 = quant.dequant_v_fp8(vc, ve)
        Vhat = V8 if pv_mode == PV_FP8 else np.where((modes == PV_FP8)[:, :, None, None], V8, Vhat)
    res = sage_attention_emulated(qc, dq, kc, dk, Vhat, modes, dtype, sm_scale,
                                  frame_len, kv_len, q_pos0, rows, splits,
                                  block_mask=block_mask, slack=slack, perturb=perturb)
    if slack is not None:
        res[2]["pv_modes"] = np.broadcast_to(np.asarray(modes, dtype=np.int64), qc.shape[:2])
    return res


def cache_list(Nq, q_pos0_b, kv_len_b, frame_len, frame_stride, sink_frames, window_frames):
    """The ordered key-chunk list of one batch over a frame cache: every chunk
    that some query row of the batch can see, ascending -- the chunks of the
    sink frames, then those of the window frames from the first row's window
    start through the last row's frame (up to its last valid token); with no
    window, every chunk up to there.  Returns (a0, b1, end): entry v is chunk
    v for v < a0, else chunk b1 + (v - a0); n = a0 + end - b1 entries.
    (Window reading: Vidu S1 blog, section "Infra".)"""
    cpf = frame_stride // BK
    fq_lo = q_pos0_b // frame_len
    fq_hi = (q_pos0_b + Nq - 1) // frame_len
    end = (fq_hi * frame_stride + min(frame_len, kv_len_b - fq_hi * frame_len) + BK - 1) // BK
    a0 = b1 = 0
    if window_frames > 0:
        a0 = min(min(sink_frames, fq_hi + 1) * cpf, end)
        b1 = max(min(max(sink_frames, fq_lo - window_frames) * cpf, end), a0)
    return a0, b1, end


def cache_splits(Nq, q_pos0_b, kv_len_b, frame_len, frame_stride, sink_frames, window_frames,
                 nsplit):
    """Chunk ranges of the KV splits of one batch over a frame cache: split s
    takes entries [s*n/nsplit, (s+1)*n/nsplit) of ``cache_list``, returned as
    the physical chunk range that spans them (chunks of the gap between the
    sinks and the window are invisible to every row, so they change nothing
    in the emulation); None for one split."""
    if nsplit <= 1:
        return None
    a0, b1, end = cache_list(Nq, q_pos0_b, kv_len_b, frame_len, frame_stride, sink_frames,
                             window_frames)
    n = a0 + (end - b1)

    def phys(v):
        return v if v < a0 else b1 + (v - a0)

    out = []
    for s in range(nsplit):
        lo, hi = s * n // nsplit, (s + 1) * n // nsplit
        if hi > lo:
            out.append((phys(lo), phys(hi - 1) + 1))
    return out


def emulate_frame_cache(Q, K, V, pv_mode, dtype, frame_len, frame_stride, sink_frames,
                        window_frames, kv_len, q_pos0, mu, shift, nsplit, rows=None, slack=None):
    """``emulate_from_inputs`` over a frame cache with each batch's KV splits
    (``cache_splits``).  Q [B,H,Nq,d]; K, V [B,H,tokens,d] of whole frames
    from frame 0; mu, shift: the frozen mean and exponents.  Returns what
    ``sage_attention_emulated`` returns."""
    Nq = np.shape(Q)[2]
    sp = [cache_splits(Nq, int(q_pos0[b]), int(kv_len[b]), frame_len, frame_stride, sink_frames,
                       window_frames, nsplit) for b in range(np.shape(Q)[0])]
    return emulate_from_inputs(Q, K, V, pv_mode, dtype, None, frame_len, kv_len, q_pos0, rows, sp,
                               mu, shift, frame_stride, sink_frames, window_frames, slack=slack)


def emulate_block_sparse(Q, K, V, pv_mode, dtype, block_mask, nsplit, frame_len=0, kv_len=None,
                         q_pos0=None, rows=None, mu=None, shift=None, slack=None):
    """``emulate_from_inputs`` with a block mask and nsplit KV splits: split s
    covers the batch's chunks [s*n/nsplit, (s+1)*n/nsplit) (n =
    ceil(kv_len/64), as without a mask) and, inside them, each query tile's
    kept chunks.  Returns what ``sage_attention_emulated`` returns."""
    B, _, _, _ = np.shape(Q)
    Nkv = np.shape(K)[2]
    kv = np.full(B, Nkv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    sp = [split_ranges(kv[b], nsplit) for b in range(B)]
    return emulate_from_inputs(Q, K, V, pv_mode, dtype, None, frame_len, kv, q_pos0, rows, sp,
                               mu, shift, block_mask=block_mask, slack=slack)
