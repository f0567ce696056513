"""Exact attention in float64: the result the quantized path approximates.

SageAttention is used as a drop-in replacement for FlashAttention (podcast
notes, section "37:54 One line of code, twice the speed"), and FlashAttention
computes exact softmax attention.  So the reference is the plain definition

    O = softmax(Q K^T * sm_scale + M) V,   M[i,j] = 0 if visible else -inf,

evaluated entirely in float64 with no quantization.

Mask.  Streaming generation produces a video frame by frame under a causal
attention mask, each frame attending to the condition and to earlier frames
through a KV cache (Vidu S1 blog, sections "模型架构" and "训练方法"; podcast
notes on the KV cache of streaming diffusion).  The reading taken here is the
frame-block-causal mask: with frame length F > 0, query token i (absolute
position q_pos0[b] + i) sees key j iff j < kv_len[b] and
floor(j / F) <= floor((q_pos0[b] + i) / F) -- every earlier frame and all of
its own frame.  F = 0 means full (non-causal) attention over kv_len[b] keys.

Sliding window with sinks.  Streaming decoding keeps attention to a window of
fixed length: a persistent reference context computed once (the analogue of
sink tokens / sink frames), the history frames cached inside the window, and
the frame being denoised (Vidu S1 blog, section "Infra").  Reading taken
here, with S sink frames and W window frames: key frame fk is visible from
query frame fq iff fk <= fq and (W == 0 or fk < S or fk >= fq - W), i.e. the
first S frames, the W most recent history frames and the current frame;
W == 0 keeps every earlier frame (the plain frame-block-causal mask).

Block-sparse attention.  Sparse attention kernels (SpargeAttention, and the
sparse branch of Sparse-Linear Attention, which can be built on top of
SageAttention: Vidu S1 blog, section "Infra"; TurboDiffusion digests) skip
whole (query block, key block) tiles that a predictor marks as negligible.
The pages give neither the predictor nor a sparsity level, so the mask is an
input here: block_mask[b, h, i // 128, j // 64] != 0 keeps the tile, and key
j is visible from row i only if its tile is kept and the mask above allows
it.  A row left with no visible key outputs 0 (the softmax of an empty set is
undefined; the kernel's accumulators stay zero).
"""

import numpy as np

from .constants import BQ, BK


def row_end(i_rows, kv_len_b, q_pos0_b, frame_len):
    """Exclusive end of the visible key range of each query row.

    The frame-block-causal mask makes every row's visible set a prefix
    [0, end) of the keys: end = min(kv_len, (floor((q_pos0+i)/F) + 1) * F).
    """
    i = np.asarray(i_rows, dtype=np.int64)
    if frame_len == 0:
        return np.full(i.shape, int(kv_len_b), dtype=np.int64)
    f = (int(q_pos0_b) + i) // int(frame_len)
    return np.minimum(int(kv_len_b), (f + 1) * int(frame_len))


def frame_visible(fk, fq, sink_frames=0, window_frames=0):
    """Key frame fk visible from query frame fq (broadcasting arrays)."""
    fk = np.asarray(fk, dtype=np.int64)
    fq = np.asarray(fq, dtype=np.int64)
    ok = fk <= fq
    if window_frames:
        ok = ok & ((fk < int(sink_frames)) | (fk >= fq - int(window_frames)))
    return ok


def visible(i_rows, Nkv, kv_len_b, q_pos0_b, frame_len, sink_frames=0, window_frames=0):
    """Boolean [len(i_rows), Nkv]: the mask (frame-block-causal, optionally
    restricted to sink + window frames)."""
    i = np.asarray(i_rows, dtype=np.int64)
    j = np.arange(Nkv, dtype=np.int64)
    vis = np.broadcast_to(j[None, :] < int(kv_len_b), (i.shape[0], Nkv)).copy()
    if frame_len:
        fq = (int(q_pos0_b) + i) // int(frame_len)
        vis = vis & frame_visible(j[None, :] // int(frame_len), fq[:, None], sink_frames, window_frames)
    elif window_frames:
        raise ValueError("a window needs frames")
    return vis


def block_visible(vis, rows, block_mask_bh):
    """vis [R, n] restricted to the kept (query block, key block) tiles of one
    (b, h): block_mask_bh [ceil(Nq/128), ceil(Nkv/64)]."""
    rows = np.asarray(rows, dtype=np.int64)
    kb = np.arange(vis.shape[1], dtype=np.int64) // BK
    keep = np.asarray(block_mask_bh)[(rows // BQ)[:, None], kb[None, :]] != 0
    return vis & keep


def default_q_pos0(Nq, kv_len, frame_len):
    """Absent an explicit q_pos0, the query chunk is the tail of the keys."""
    kv = np.asarray(kv_len, dtype=np.int64)
    if frame_len == 0:
        return np.zeros_like(kv)
    return kv - int(Nq)


def attention_fp64(Q, K, V, sm_scale=None, frame_len=0, kv_len=None,
                   q_pos0=None, rows=None, sink_frames=0, window_frames=0,
                   block_mask=None):
    """softmax(Q K^T * sm_scale + M) V in float64 for the selected rows.

    Q [B,H,Nq,d], K and V [B,H,Nkv,d] (any float dtype; widened exactly),
    tokens contiguous.  rows: indices of the query rows to compute (all when
    None).  block_mask: optional [B,H,ceil(Nq/128),ceil(Nkv/64)], nonzero =
    tile kept; rows with no visible key give 0.
    Returns float64 [B,H,len(rows),d].
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Nq, d = Q.shape
    Nkv = K.shape[2]
    scale = 1.0 / np.sqrt(d) if sm_scale is None else float(sm_scale)
    kv = np.full(B, Nkv, np.int64) if kv_len is None else np.asarray(kv_len, np.int64)
    qp = default_q_pos0(Nq, kv, frame_len) if q_pos0 is None else np.asarray(q_pos0, np.int64)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, H, len(rows), d), dtype=np.float64)
    for b in range(B):
        vis_b = visible(rows, Nkv, kv[b], qp[b], frame_len, sink_frames, window_frames)
        for h in range(H):
            vis = vis_b if block_mask is None else block_visible(vis_b, rows, block_mask[b, h])
            s = (Q[b, h, rows, :] @ K[b, h].T) * scale
            s = np.where(vis, s, -np.inf)
            mx = np.max(s, axis=1, keepdims=True)
            w = np.exp(s - np.where(np.isneginf(mx), 0.0, mx))
            den = np.sum(w, axis=1, keepdims=True)
            out[b, h] = np.where(den > 0, w @ V[b, h] / np.where(den > 0, den, 1.0), 0.0)
    return out
