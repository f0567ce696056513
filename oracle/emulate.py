"""Quantized attention, emulated on the CPU step by step.

The pages describe SageAttention only as low-bit quantized attention that
keeps the output of the FlashAttention it replaces ("37:54 One line of code,
twice the speed"; "02:48 There were clearly faster compute units on the
hardware").  This module is the library's own stated algorithm, written out so
that each rounding the GPU performs happens here in the same precision:

Given the INT8 codes and scales of ``quant`` (and V^, the P.V operand:
V itself in 16-bit mode, or its dequantized FP8 codes), for every query row i
of head (b,h), with state m = -inf, l = 0, acc = 0, the keys are taken in
chunks of BK = 64 (chunk t = keys [64t, 64t+64)), in ascending order:

  1. S[i,j]   = sum_c qcode[i,c] * kcode[j,c]            (exact integers)
  2. sigma    = fp32(sm_scale * log2 e);  qs = fp32(dq[i // 128] * sigma)
     c_t      = fp32(qs * dk[t])             (log2-domain scale of chunk t)
  3. tm       = max over visible j of fp32(S[i,j] * c_t)  (-inf if none)
  4. lazy running max: if tm > fp32(m + TAU) the row adopts m' = tm and
     rescales its state by alpha = exp2(fp32(m - m')) (0 when m = -inf);
     otherwise m, l and acc are kept as they are.
  5. x[i,j]   = S[i,j] * c_t - mref, mref = fp32(m - s) (s = 4 in FP8 mode,
     0 in 16-bit mode), evaluated on the score as the float32
     F = F0 + S * 2^-26, where F0 is the float32 with bits 0x3E22F983 (the
     constant 1/(2 pi)); F is exact (its bits are those of F0 plus S) for
     |S| < 2292099.  With c2 = c_t * 2^26 (exact):
        K = fp32(-F0 * c2 - mref)   (one FMA, per row and chunk)
        x = fp32(F * c2 + K)        (one FMA)
     so x is S c_t - mref up to K's rounding (half an ulp of
     |K| <= 1.07e7 c_t + |mref|: about 0.64 c_t, under one integer step of
     S, when the first term dominates) and x's own;  p = fp32(2^x), 0 if not
     visible.
  6. p~       = p rounded to the P.V operand type: e4m3fn in FP8 mode (where
     p already carries the 2^s pre-scale), else the input's fp16/bf16
  7. l       += sum_j p~                     (the rounded operand itself)
  8. acc     += sum_j p~[i,j] * V^[j,:]
Finally O[i] = acc / l; the 2^s pre-scale cancels in that ratio.  The output
is rounded (RNE) to the input dtype.  Because l sums exactly the weights that
multiply V^, every output row is a convex combination of the visible V^ rows
(a constant V^ column comes out unchanged).

Because m only moves when a chunk maximum exceeds it by more than TAU, the
exponent argument is at most TAU + s = 8, so p~ never exceeds 2^8 -- inside
both e4m3fn (448) and the 16-bit types.

Split-KV: when ``splits`` lists chunk ranges, each range runs steps 1-8 from a
fresh state and the partial results are merged exactly (float64):
M = max_s m_s, O = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).

Accumulations (l, acc) are float64 here; the GPU keeps them in float32.  That,
the GPU's hardware exp2 (within ~1 ulp) and the final division are the only
places where the two may differ, all far below the acceptance tolerance.
"""

import numpy as np

from .constants import BQ, BK, TAU, PSHIFT_FP8, PSHIFT_16, LOG2E, PV_16, PV_FP8, CACHE_TILE
from . import codecs
from .fp32 import fma_f32
from .attention import row_end, default_q_pos0

_F32 = np.float32


def log2_scale(sm_scale, d):
    """sigma = fp32(float64(sm_scale) * log2 e); sm_scale 0/None -> 1/sqrt(d)."""
    if not sm_scale:
        sm_scale = float(_F32(1.0 / np.sqrt(d)))
    return _F32(np.float64(_F32(sm_scale)) * LOG2E)


def _run_rows(S_full, c_row, dk_bh, vis_end, Vhat_bh, chunk_lo, chunk_hi,
              pv_mode, p_dtype, trace=None):
    """Steps 1-8 over chunks [chunk_lo, chunk_hi) for a set of rows.

    vis_end: per row, the exclusive end of its visible key prefix; or a
    boolean [R, keys] visibility matrix.
    trace: optional list; receives the running max m after every chunk.
    """
    vis_end = np.asarray(vis_end)
    R = S_full.shape[0]
    d = Vhat_bh.shape[1]
    m = np.full(R, -np.inf, dtype=_F32)
    l = np.zeros(R, dtype=np.float64)
    acc = np.zeros((R, d), dtype=np.float64)
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
        S = S_full[:, j0:j1]
        m, l, acc = _chunk_step(S, c_t, vis, m, l, acc, Vhat_bh[j0:j1], pv_mode, p_dtype)
        if trace is not None:
            trace.append(m.copy())
    return m, l, acc


F0 = np.array(0x3E22F983, dtype=np.uint32).view(np.float32)  # 1/(2 pi) as float32
S_BIAS_LIMIT = 2292099   # |S| below this keeps F0 + S 2^-26 in F0's binade


def score_as_float(S):
    """The float32 F0 + S 2^-26 (exact: bits(F) = bits(F0) + S) for integer
    scores |S| < 2292099."""
    S = np.asarray(S, dtype=np.float64)
    if np.any(np.abs(S) >= S_BIAS_LIMIT):
        raise ValueError("score outside the biased-float range")
    return (np.float64(F0) + S * 2.0 ** -26).astype(_F32)


def scaled_logit(S, c_t, mref):
    """Step 5: x = S c_t - mref as two float32 FMAs on F = F0 + S 2^-26 (rows of
    S pair with entries of c_t and mref)."""
    F = score_as_float(S)
    c2 = (np.asarray(c_t, _F32) * _F32(2.0 ** 26)).astype(_F32)      # exact
    K = fma_f32(np.broadcast_to(-F0, c2.shape), c2, -np.asarray(mref, _F32))
    return fma_f32(F, np.broadcast_to(c2[:, None], F.shape), np.broadcast_to(K[:, None], F.shape))


def _chunk_step(S, c_t, vis, m, l, acc, Vc, pv_mode, p_dtype):
    """Steps 3-8 for one chunk; c_t is per row (rows may span Q blocks)."""
    shift = PSHIFT_FP8 if pv_mode == PV_FP8 else PSHIFT_16
    c64 = c_t.astype(np.float64)[:, None]
    logit = (S * c64).astype(_F32)
    tm = np.where(vis, logit, -np.inf).max(axis=1).astype(_F32)
    upd = tm > (m + _F32(TAU)).astype(_F32)
    with np.errstate(invalid="ignore"):
        diff = (m - tm).astype(_F32)
    alpha = np.where(np.isneginf(m), _F32(0.0),
                     np.exp2(np.where(upd, diff, _F32(0)).astype(np.float64)).astype(_F32))
    alpha = np.where(upd, alpha, _F32(1.0)).astype(np.float64)
    m = np.where(upd, tm, m).astype(_F32)
    l = l * alpha
    acc = acc * alpha[:, None]
    # a row still at m = -inf has no visible key in this chunk; its p is 0
    mref = np.where(np.isneginf(m), _F32(0.0), (m - _F32(shift)).astype(_F32)).astype(_F32)
    x = scaled_logit(S, c_t, mref)
    p = np.exp2(x.astype(np.float64)).astype(_F32)
    p = np.where(vis, p, _F32(0.0))
    if pv_mode == PV_FP8:
        pt = codecs.round_e4m3(p.astype(np.float64))
    else:
        pt = codecs.round_to(p, p_dtype).astype(np.float64)
    l = l + pt.sum(axis=1)
    acc = acc + pt @ Vc
    return m, l, acc


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
                            block_mask=None):
    """Emulate the quantized attention for the selected query rows.

    qcodes int8 [B,H,Nq,d], dq float32 [B,H,ceil(Nq/128)];
    kcodes int8 [B,H,Nkv,d], dk float32 [B,H,ceil(Nkv/64)];
    Vhat: the P.V right operand as exact values [B,H,Nkv,d] -- V (16-bit
    mode) or dequant_v_fp8(...) (FP8 mode);  dtype: 'bf16' | 'f16' (input and
    output type, and P's type in 16-bit mode).
    splits: optional list of (chunk_lo, chunk_hi) ranges covering the keys.
    frame_stride > 0: K/V operands are a frame cache (``quant.quantize_k_frames``
    layout: frame f's tokens at slots f*frame_stride + [0, frame_len)); kv_len and
    q_pos0 stay in tokens; sink_frames / window_frames restrict the visible
    frames as in ``attention.visible``.
    block_mask: optional [B,H,ceil(Nq/128),ceil(Nkv/64)] (contiguous keys);
    chunks of dropped tiles are skipped -- they change neither m, l nor acc,
    exactly as if they were absent -- and a row with no visible key gives 0.
    splits then index the tile's list of kept chunks (see
    ``sparse_tile_splits``).
    Returns (O64 float64 [B,H,R,d], O rounded to dtype as float32).
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
    if splits is None:
        splits = [(0, nchunks)]
    out = np.empty((B, H, len(rows), d), dtype=np.float64)
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
        for h in range(H):
            vis_h = vis_end
            if block_mask is not None:
                from .attention import block_visible
                vis_h = block_visible(np.arange(jmax)[None, :] < vis_end[:, None], rows, block_mask[b, h])
            qs = (dq[b, h, rows // BQ].astype(_F32) * sigma).astype(_F32)   # [R]
            S_full = qcodes[b, h, rows, :].astype(np.float64) @ \
                kcodes[b, h, :jmax, :].astype(np.float64).T                # exact
            Vh = np.asarray(Vhat[b, h, :jmax, :], dtype=np.float64)
            parts = [_run_rows(S_full, qs, dk[b, h], vis_h, Vh, lo, hi, pv_mode, dtype)
                     for (lo, hi) in splits]
            ms = np.stack([p[0] for p in parts]).astype(np.float64)        # [P, R]
            ls = np.stack([p[1] for p in parts])
            accs = np.stack([p[2] for p in parts])
            M = np.max(ms, axis=0)
            with np.errstate(invalid="ignore"):   # rows with no key at all: M = -inf
                w = np.where(np.isneginf(ms), 0.0, np.exp2(ms - M[None, :]))
            L = np.sum(w * ls, axis=0)
            num = np.sum(w[:, :, None] * accs, axis=0)
            out[b, h] = np.where(L[:, None] > 0, num / np.where(L > 0, L, 1.0)[:, None], 0.0)
    rounded = codecs.round_to(out.astype(_F32), dtype)
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
                        window_frames=0, block_mask=None):
    """Quantize the 16-bit inputs with ``quant`` and run the emulation.

    frame_stride > 0: K and V (tokens of whole frames from frame 0) go into a
    frame cache, each frame quantized once against the given (frozen) mu and
    shift (both required then)."""
    from . import quant
    Qf = np.asarray(Q, dtype=np.float32)
    Kf = np.asarray(K, dtype=np.float32)
    Vf = np.asarray(V, dtype=np.float32)
    if frame_stride:
        qc, dq = quant.quantize_q(Qf, shift)
        kc, dk = quant.quantize_k_frames(Kf, mu, shift, frame_len, frame_stride)
        if pv_mode == PV_FP8:
            vc, ve = quant.quantize_v_fp8_frames(Vf, frame_len, frame_stride)
            Vhat = quant.dequant_v_fp8(vc, ve)
        else:
            Vhat = quant.to_frame_slots(Vf, frame_len, frame_stride).astype(np.float64)
        return sage_attention_emulated(qc, dq, kc, dk, Vhat, pv_mode, dtype, sm_scale,
                                       frame_len, kv_len, q_pos0, rows, splits,
                                       frame_stride, sink_frames, window_frames)
    if mu is None:
        mu = quant.k_mean(Kf, kv_len)
    a = quant.channel_shift(Qf, Kf, mu, kv_len) if shift is None else shift
    qc, dq = quant.quantize_q(Qf, a)
    kc, dk = quant.quantize_k(Kf, mu, kv_len, a)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(Vf, kv_len)
        Vhat = quant.dequant_v_fp8(vc, ve)
    else:
        Vhat = Vf.astype(np.float64)
    return sage_attention_emulated(qc, dq, kc, dk, Vhat, pv_mode, dtype, sm_scale,
                                   frame_len, kv_len, q_pos0, rows, splits,
                                   block_mask=block_mask)


def cache_tile_splits(first, last, q_pos0_b, kv_len_b, frame_len, frame_stride,
                      sink_frames, window_frames, nsplit):
    """Chunk ranges of the split work items of one query tile (rows
    first..last, CACHE_TILE of them) over a frame cache.

    The tile's key chunks, in order, are those of the sink frames, then those
    of the window frames up to the last row's frame (through its last valid
    token); with no window, every chunk up to there.  Split s takes entries
    [s*n/nsplit, (s+1)*n/nsplit) of that list.  Each entry range is returned
    as the physical chunk range that spans it: chunks of the gap between the
    sinks and the window are invisible to every row of the tile, so they
    change nothing in the emulation.  (Window reading: Vidu S1 blog, section
    "Infra".)"""
    cpf = frame_stride // BK
    fq_lo = (q_pos0_b + first) // frame_len
    fq_hi = (q_pos0_b + last) // frame_len
    end = (fq_hi * frame_stride + min(frame_len, kv_len_b - fq_hi * frame_len) + BK - 1) // BK
    a0 = b1 = 0
    if window_frames > 0:
        a0 = min(min(sink_frames, fq_hi + 1) * cpf, end)
        b1 = max(min(max(sink_frames, fq_lo - window_frames) * cpf, end), a0)
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
                        window_frames, kv_len, q_pos0, mu, shift, nsplit, rows=None):
    """``emulate_from_inputs`` over a frame cache, tile by tile of CACHE_TILE
    query rows, each tile with the chunk ranges of its split work items
    (``cache_tile_splits``).  Q [B,H,Nq,d]; K, V [B,H,tokens,d] of whole
    frames from frame 0; mu, shift: the frozen mean and exponents.
    Returns float64 O [B,H,R,d] for the selected rows (all when None)."""
    from . import quant
    Qf = np.asarray(Q, dtype=np.float32)
    B, H, Nq, d = Qf.shape
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    qc, dq = quant.quantize_q(Qf, shift)
    kc, dk = quant.quantize_k_frames(np.asarray(K, dtype=np.float32), mu, shift, frame_len, frame_stride,
                                     kv_len=kv_len)
    Vf = np.asarray(V, dtype=np.float32)
    if pv_mode == PV_FP8:
        vc, ve = quant.quantize_v_fp8_frames(Vf, frame_len, frame_stride, kv_len=kv_len)
        Vhat = quant.dequant_v_fp8(vc, ve)
    else:
        Vhat = quant.to_frame_slots(Vf, frame_len, frame_stride).astype(np.float64)
    out = np.empty((B, H, len(rows), d))
    for b in range(B):
        for t in np.unique(rows // CACHE_TILE):
            sel = np.nonzero(rows // CACHE_TILE == t)[0]
            first, last = t * CACHE_TILE, min(t * CACHE_TILE + CACHE_TILE, Nq) - 1
            sp = cache_tile_splits(first, last, int(q_pos0[b]), int(kv_len[b]), frame_len,
                                   frame_stride, sink_frames, window_frames, nsplit)
            o64, _ = sage_attention_emulated(qc[b:b + 1], dq[b:b + 1], kc[b:b + 1], dk[b:b + 1],
                                             Vhat[b:b + 1], pv_mode, dtype, None, frame_len,
                                             [kv_len[b]], [q_pos0[b]], rows[sel],
                                             sp if nsplit > 1 else None, frame_stride,
                                             sink_frames, window_frames)
            out[b, :, sel] = o64[0].transpose(1, 0, 2)
    return out


def sparse_tile_splits(mask_row, n_chunks, nsplit):
    """Chunk ranges of the split work items of one 128-query tile under a
    block mask: the tile's list is its kept chunks among [0, n_chunks) (the
    chunks its last row can see), in ascending order; split s takes entries
    [s*n/nsplit, (s+1)*n/nsplit) of it, returned as the physical chunk range
    that spans them (the dropped chunks inside are invisible to the tile)."""
    kept = np.nonzero(np.asarray(mask_row)[:n_chunks] != 0)[0]
    n = kept.size
    out = []
    for s in range(nsplit):
        lo, hi = s * n // nsplit, (s + 1) * n // nsplit
        if hi > lo:
            out.append((int(kept[lo]), int(kept[hi - 1]) + 1))
    return out


def emulate_block_sparse(Q, K, V, pv_mode, dtype, block_mask, nsplit, frame_len=0, kv_len=None,
                         q_pos0=None, rows=None, mu=None, shift=None):
    """``emulate_from_inputs`` with a block mask, tile by tile of 128 query
    rows, each tile with the chunk ranges of its split work items
    (``sparse_tile_splits``).  Returns float64 O [B,H,R,d]."""
    from . import quant
    from .attention import row_end
    Qf = np.asarray(Q, dtype=np.float32)
    Kf = np.asarray(K, dtype=np.float32)
    Vf = np.asarray(V, dtype=np.float32)
    B, H, Nq, d = Qf.shape
    Nkv = Kf.shape[2]
    kv = np.full(B, Nkv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    qp = default_q_pos0(Nq, kv, frame_len) if q_pos0 is None else np.asarray(q_pos0, np.int64)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    if mu is None:
        mu = quant.k_mean(Kf, kv)
    a = quant.channel_shift(Qf, Kf, mu, kv) if shift is None else shift
    qc, dq = quant.quantize_q(Qf, a)
    kc, dk = quant.quantize_k(Kf, mu, kv, a)
    if pv_mode == PV_FP8:
        vc, ve, _ = quant.quantize_v_fp8(Vf, kv)
        Vhat = quant.dequant_v_fp8(vc, ve)
    else:
        Vhat = Vf.astype(np.float64)
    out = np.empty((B, H, len(rows), d))
    for b in range(B):
        for t in np.unique(rows // BQ):
            sel = np.nonzero(rows // BQ == t)[0]
            last = min(t * BQ + BQ, Nq) - 1
            nch = -(-int(row_end([last], kv[b], qp[b], frame_len)[0]) // BK)
            for h in range(H):
                sp = sparse_tile_splits(block_mask[b, h, t], nch, nsplit)
                if not sp:
                    out[b, h, sel] = 0.0
                    continue
                o64, _ = sage_attention_emulated(qc[b:b + 1, h:h + 1], dq[b:b + 1, h:h + 1], kc[b:b + 1, h:h + 1],
                                                 dk[b:b + 1, h:h + 1], Vhat[b:b + 1, h:h + 1], pv_mode, dtype,
                                                 None, frame_len, [kv[b]], [qp[b]], rows[sel],
                                                 sp if nsplit > 1 else None,
                                                 block_mask=block_mask[b:b + 1, h:h + 1])
                out[b, h, sel] = o64[0, 0]
    return out
