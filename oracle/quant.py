"""Quantization of Q, K and V, step by step in the scheme's own order.

The pages call SageAttention "low-bit quantized attention" and say it had to
overcome the precision loss of low-bit compute (podcast notes, section "02:48
There were clearly faster compute units on the hardware"; the TurboDiffusion
digests on the reportify page).  They give no scheme.  The scheme here is the
library's stated design:

1. K smoothing: one mean vector mu[b,h,:] over the valid keys of each
   (batch, head).  Subtracting a vector shared by every key a query sees
   adds the same constant to each of that query's logits, so the softmax is
   unchanged while the per-channel offset (the source of K outliers) leaves
   the quantization range.
2. Channel balance: for each (b,h,c) a power-of-two exponent a_c moves range
   between Q and K~ -- Q'[.,c] = Q[.,c] * 2^a_c and K'[.,c] = K~[.,c] * 2^-a_c
   -- which leaves every product q.k exactly unchanged (scaling by a power of
   two is exact in binary floating point).  a_c is the integer nearest to
   half of log2(amax_c(K~) / amax_c(Q)), so that one outlier channel of K
   (the large config scales 1% of channels x8) no longer sets the scale of
   its whole K block.
3. Symmetric per-block INT8 for Q (blocks of BQ = 128 tokens) and for the
   smoothed K (blocks of BK = 64 tokens): delta = amax / 127, codes
   rint(x * (127 / amax)) in [-127, 127].
4. FP8 P.V mode only: V in OCP e4m3fn with one power-of-two (E8M0) scale per
   (32-key block, channel), the smallest that keeps the block within 448.
5. Per-head P.V mode (PV_AUTO): FP8 for a (b,h) whose channel-balance
   exponents are all 0, the input's 16-bit type for one where some a_c != 0
   (``pv_modes_auto``).

Shapes: Q [B,H,Nq,d]; K, V [B,H,Nkv,d]; kv_len [B] with 1 <= kv_len[b] <= Nkv.
Keys at positions >= kv_len[b] are padding: they take no part in the mean or
any amax, and their codes are 0.
"""

import numpy as np

from .constants import BQ, BK, VB, QMAX, KMEAN_CHUNK, PV_16, PV_FP8
from . import codecs


def _kv_len(B, Nkv, kv_len, least=0):
    """Valid tokens per batch (all when None); the block quantizers accept a
    batch with none (every block empty: scale 0, codes 0), the mean needs one."""
    if kv_len is None:
        return np.full(B, Nkv, dtype=np.int64)
    kv = np.asarray(kv_len, dtype=np.int64)
    assert kv.shape == (B,) and np.all(kv >= least) and np.all(kv <= Nkv)
    return kv


def k_mean(K, kv_len=None):
    """mu[b,h,c] = mean of K[b,h,:kv_len[b],c], as float32.

    Fixed order: for each run of KMEAN_CHUNK = 128 tokens, a float64 sum in
    ascending token order; then the run sums added in ascending run order in
    float64; then float64 division by the token count, rounded to float32.
    """
    K = np.asarray(K, dtype=np.float32)
    B, H, Nkv, d = K.shape
    kv = _kv_len(B, Nkv, kv_len, least=1)
    mu = np.empty((B, H, d), dtype=np.float32)
    for b in range(B):
        n = int(kv[b])
        total = np.zeros((H, d), dtype=np.float64)
        for start in range(0, n, KMEAN_CHUNK):
            stop = min(start + KMEAN_CHUNK, n)
            run = np.zeros((H, d), dtype=np.float64)
            for j in range(start, stop):           # ascending, sequential
                run += K[b, :, j, :].astype(np.float64)
            total += run
        mu[b] = (total / np.float64(n)).astype(np.float32)
    return mu


def quant_int8_blocks(X, block, n_valid=None):
    """Per-block symmetric INT8 quantization along the token axis.

    X: float32 [B,H,N,d] (already smoothed for K).  n_valid: [B] count of
    valid tokens (all N when None).  For block t of (b,h): the valid tokens
    are [t*block, min((t+1)*block, n_valid[b])).
      amax  = max |x| over the block's valid elements
      delta = fp32(amax / 127),  inv = fp32(127 / amax)   (IEEE division)
      code  = clamp(rint(fp32(x * inv)), -127, 127)        (ties to even)
    A block with amax == 0 (or no valid token) has delta = 0 and all codes 0.
    Returns codes int8 [B,H,N,d] and delta float32 [B,H,ceil(N/block)].
    """
    X = np.asarray(X, dtype=np.float32)
    B, H, N, d = X.shape
    nv = _kv_len(B, N, n_valid)
    nblk = -(-N // block)
    codes = np.zeros((B, H, N, d), dtype=np.int8)
    delta = np.zeros((B, H, nblk), dtype=np.float32)
    q127 = np.float32(QMAX)
    for b in range(B):
        for t in range(nblk):
            lo = t * block
            hi = min(lo + block, int(nv[b]))
            if hi <= lo:
                continue
            blk = X[b, :, lo:hi, :]                       # [H, n, d]
            amax = np.max(np.abs(blk), axis=(1, 2))       # [H] float32
            nz = amax > 0
            safe = np.where(nz, amax, np.float32(1.0)).astype(np.float32)
            dlt = np.where(nz, (safe / q127).astype(np.float32), np.float32(0))
            inv = (q127 / safe).astype(np.float32)
            y = (blk * inv[:, None, None]).astype(np.float32)
            c = np.clip(np.rint(y), -QMAX, QMAX)
            c = np.where(nz[:, None, None], c, 0)
            codes[b, :, lo:hi, :] = c.astype(np.int8)
            delta[b, :, t] = dlt
    return codes, delta


def channel_shift(Q, K, mu, kv_len=None):
    """Channel-balance exponents a [B,H,d] (int64).

    With A = amax over all query tokens of |Q[b,h,:,c]| and
    B = amax over valid keys of |K~[b,h,:,c]| (both float32):
    a = 0 when A == 0 or B == 0; otherwise, with k = floor(log2(B / A)),
    a = floor((k + 1) / 2), i.e. the integer a with 2^(2a-1) <= B/A < 2^(2a+1)
    -- the integer nearest to log2(B/A) / 2, halves rounded up.  k comes from
    the binary exponents alone: B = mB 2^eB, A = mA 2^eA with m in [0.5, 1)
    give k = eB - eA - (1 if mB < mA else 0).
    """
    Qf = np.asarray(Q, dtype=np.float32)
    Ks = smooth_k(K, mu, kv_len)
    A = np.max(np.abs(Qf), axis=2).astype(np.float64)      # [B,H,d]
    Bm = np.max(np.abs(Ks), axis=2).astype(np.float64)
    mA, eA = np.frexp(A)
    mB, eB = np.frexp(Bm)
    k = eB - eA - (mB < mA).astype(np.int64)
    a = np.floor_divide(k + 1, 2)
    return np.where((A == 0) | (Bm == 0), 0, a).astype(np.int64)


def pv_modes_auto(shift):
    """P.V mode of every (b,h) under PV_AUTO, from its channel-balance
    exponents a [B,H,d]: PV_FP8 where every a_c is 0, PV_16 where some a_c is
    not.  (int64 [B,H].)

    The library's reading, not the pages' (they fix no bit widths).  a_c != 0
    means the range of K~ and Q in channel c differ by a factor of 2 or more
    -- an outlier channel, as in the large workload's x8 channels -- and such
    a head's INT8 scores already spend much of the output's error budget
    (cosine 0.999 against exact attention); the 3-bit mantissas of e4m3 P and
    V would add about as much again.  A head with no such channel keeps the
    FP8 P.V, which runs at the INT8 matrix rate.
    """
    a = np.asarray(shift)
    return np.where(np.all(a == 0, axis=-1), PV_FP8, PV_16).astype(np.int64)


def quantize_q(Q, shift=None):
    """Q codes and per-128-token scales of Q' = Q * 2^a (all tokens valid)."""
    Qf = np.asarray(Q, dtype=np.float32)
    if shift is not None:
        Qf = np.ldexp(Qf, np.asarray(shift)[:, :, None, :]).astype(np.float32)
    return quant_int8_blocks(Qf, BQ)


def smooth_k(K, mu, kv_len=None):
    """K~ = fp32(K) - mu (float32 subtraction, RNE); padding keys set to 0."""
    K = np.asarray(K, dtype=np.float32)
    B, H, Nkv, d = K.shape
    kv = _kv_len(B, Nkv, kv_len)
    Ks = (K - np.asarray(mu, dtype=np.float32)[:, :, None, :]).astype(np.float32)
    for b in range(B):
        Ks[b, :, int(kv[b]):, :] = 0
    return Ks


def quantize_k(K, mu, kv_len=None, shift=None):
    """K codes and per-64-token scales of K' = (fp32(K) - mu) * 2^-a."""
    B, _, Nkv, _ = np.shape(K)
    kv = _kv_len(B, Nkv, kv_len)
    Ks = smooth_k(K, mu, kv)
    if shift is not None:
        Ks = np.ldexp(Ks, -np.asarray(shift)[:, :, None, :]).astype(np.float32)
    return quant_int8_blocks(Ks, BK, kv)


def quantize_v_fp8(V, kv_len=None):
    """FP8 e4m3fn codes of V with one E8M0 scale per (32-key block, channel).

    For block t (keys [32t, 32t+32) of (b,h), valid ones only) and channel c:
      e    = smallest integer with amax * 2^-e <= 448 (0 if amax == 0)
      code = e4m3_RNE(v * 2^-e)   (the scaling by 2^-e is exact)
    Returns codes uint8 [B,H,Nkv,d] (padding keys 0), exponents int64
    [B,H,ceil(Nkv/32),d] and the stored E8M0 bytes (e + 127) as uint8.
    """
    V = np.asarray(V, dtype=np.float32)
    B, H, Nkv, d = V.shape
    kv = _kv_len(B, Nkv, kv_len)
    nblk = -(-Nkv // VB)
    codes = np.zeros((B, H, Nkv, d), dtype=np.uint8)
    exps = np.zeros((B, H, nblk, d), dtype=np.int64)
    for b in range(B):
        for t in range(nblk):
            lo = t * VB
            hi = min(lo + VB, int(kv[b]))
            if hi <= lo:
                continue
            blk = V[b, :, lo:hi, :].astype(np.float64)        # [H, n, d]
            amax = np.max(np.abs(blk), axis=1)                # [H, d]
            e = codecs.e8m0_exponent(amax)
            codes[b, :, lo:hi, :] = codecs.e4m3_encode(np.ldexp(blk, -e[:, None, :]))
            exps[b, :, t, :] = e
    e8m0 = (exps + 127).astype(np.uint8)
    return codes, exps, e8m0


def dequant_v_fp8(codes, exps):
    """V^[b,h,j,c] = decode(code) * 2^e[block(j), c], as float64 (exact)."""
    codes = np.asarray(codes)
    B, H, Nkv, d = codes.shape
    e = np.repeat(np.asarray(exps), VB, axis=2)[:, :, :Nkv, :]
    return np.ldexp(codecs.e4m3_decode(codes), e)


# ---------------------------------------------------------------------------
# KV cache of whole frames.  Streaming decoding caches the history frames and
# reuses them step after step (Vidu S1 blog, section "Infra"), so each frame is
# quantized once, when it enters the cache, against a frozen K mean and
# channel shift.  Frame f's F tokens occupy slots [f*FS, f*FS + F) of the
# cache, FS >= F a multiple of BK; slots [f*FS + F, (f+1)*FS) are padding
# (codes 0, never visible).  Every K block (BK slots) and V block (VB slots)
# therefore lies inside one frame, and quantizing a frame never touches
# another frame's codes.

def frame_slot(t, frame_len, frame_stride):
    """Cache slot of token t."""
    t = np.asarray(t, dtype=np.int64)
    return (t // frame_len) * frame_stride + t % frame_len


def _frames_of(X, frame_len):
    n = np.shape(X)[2]
    return [(f, f * frame_len, min((f + 1) * frame_len, n)) for f in range(-(-n // frame_len))]


def _frame_valid(kv_len, lo, hi):
    """Valid tokens of the frame [lo, hi) per batch: those below kv_len[b]
    (tokens past it are padding, as in quantize_k), or all when None."""
    return None if kv_len is None else np.clip(np.asarray(kv_len) - lo, 0, hi - lo)


def quantize_k_frames(K, mu, shift, frame_len, frame_stride, n_slots=None, kv_len=None):
    """K [B,H,Ntok,d] (tokens of consecutive frames from frame 0) -> codes int8
    [B,H,n_slots,d] and scales float32 [B,H,n_slots/BK], each frame quantized
    as its own sequence (quantize_k with the given frozen mu and shift).
    kv_len [B]: tokens written so far per batch; a partly written frame
    quantizes its valid tokens only (codes 0 past kv_len)."""
    B, H, n, d = np.shape(K)
    if frame_stride % BK or frame_stride < frame_len:
        raise ValueError("frame stride must be a multiple of BK and >= the frame length")
    n_slots = n_slots or -(-n // frame_len) * frame_stride
    codes = np.zeros((B, H, n_slots, d), dtype=np.int8)
    dk = np.zeros((B, H, n_slots // BK), dtype=np.float32)
    for f, lo, hi in _frames_of(K, frame_len):
        c, dl = quantize_k(np.asarray(K)[:, :, lo:hi], mu, _frame_valid(kv_len, lo, hi), shift)
        s0 = f * frame_stride
        codes[:, :, s0:s0 + hi - lo] = c
        dk[:, :, s0 // BK:s0 // BK + dl.shape[2]] = dl
    return codes, dk


def quantize_v_fp8_frames(V, frame_len, frame_stride, n_slots=None, kv_len=None):
    """quantize_v_fp8 per frame into cache slots: codes uint8 [B,H,n_slots,d],
    exponents int64 [B,H,n_slots/VB,d]; kv_len as in quantize_k_frames."""
    B, H, n, d = np.shape(V)
    n_slots = n_slots or -(-n // frame_len) * frame_stride
    codes = np.zeros((B, H, n_slots, d), dtype=np.uint8)
    exps = np.zeros((B, H, n_slots // VB, d), dtype=np.int64)
    for f, lo, hi in _frames_of(V, frame_len):
        c, e, _ = quantize_v_fp8(np.asarray(V)[:, :, lo:hi], _frame_valid(kv_len, lo, hi))
        s0 = f * frame_stride
        codes[:, :, s0:s0 + hi - lo] = c
        exps[:, :, s0 // VB:s0 // VB + e.shape[2]] = e
    return codes, exps


def to_frame_slots(X, frame_len, frame_stride, n_slots=None):
    """Place tokens [B,H,Ntok,...] into cache slots (padding zero)."""
    X = np.asarray(X)
    B, H, n = X.shape[:3]
    n_slots = n_slots or -(-n // frame_len) * frame_stride
    out = np.zeros((B, H, n_slots) + X.shape[3:], dtype=X.dtype)
    out[:, :, frame_slot(np.arange(n), frame_len, frame_stride)] = X
    return out
