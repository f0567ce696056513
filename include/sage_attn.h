/*
 * sage_attn.h -- C ABI of a low-bit (SageAttention-style) quantized attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Quantized softmax attention meant as a drop-in for exact
 * attention: the podcast notes "Faster! Even faster! ..." (section "37:54 One
 * line of code, twice the speed") describe replacing FlashAttention with
 * SageAttention by changing one line, and (section "02:48 There were clearly
 * faster compute units on the hardware") motivate it by the low-precision
 * matrix units that exact attention leaves idle while video-generation
 * attention is compute-bound.  The pages give no quantization scheme; the
 * scheme of this library is:
 *   - K mean-smoothing: mu[b,h,:] = mean of the valid keys, subtracted from K;
 *   - channel balance: per (b,h,channel) power-of-two exponent a moving range
 *     between Q (x 2^a) and K (x 2^-a), exact in binary floating point;
 *   - symmetric INT8 per block: Q in blocks of 128 tokens, K in blocks of 64,
 *     scale = amax/127, code = rint(x * (127/amax));
 *   - S = Q K^T on INT8 matrix cores with int32 accumulation, dequantized in
 *     fp32, online softmax in fp32 over 64-key chunks with a lazy running max;
 *   - P V on 16-bit matrix cores (P rounded to the input type) or, in FP8
 *     mode, on scaled FP8 matrix cores: P as OCP e4m3fn (pre-scaled by 2^4),
 *     V as e4m3fn with one E8M0 scale per (32-key block, channel);
 *   - per-head mode (SAGE_PV_AUTO, contiguous keys only): FP8 P V for a
 *     (b,h) whose channel-balance exponents are all 0, 16-bit P V for one
 *     with an outlier channel (some a != 0), whose INT8 scores already take
 *     much of the output's error budget.
 * Frame-block-causal mask for streaming against a KV cache (the Vidu S1 blog,
 * sections "模型架构", "训练方法" and "Infra": frame-by-frame causal
 * generation over cached history): with frame length F > 0, query i
 * (absolute position q_pos0[b] + i) sees key j iff j < kv_len[b] and
 * floor(j/F) <= floor((q_pos0[b]+i)/F).  F = 0: every key j < kv_len[b].
 *
 * Frame cache and sliding window (frame_stride > 0).  Streaming decoding
 * attends within a fixed window -- a persistent reference context computed
 * once (like sink frames), the history cached inside the window and the
 * current frame -- over cached history (Vidu S1 blog, section "Infra").  K and
 * V are then held as a cache of whole frames quantized once: frame f's F
 * tokens occupy slots [f*FS, f*FS + F) of the quantized K/V operands (FS =
 * frame_stride, a multiple of 64, >= F; the other slots are padding, never
 * visible), so no scale block spans two frames and appending a frame
 * (sage_attn_quantize_frames) touches no other frame's codes.  With S =
 * sink_frames and W = window_frames > 0, query frame fq sees key frame fk iff
 * fk <= fq and (fk < S or fk >= fq - W); W = 0 keeps every earlier frame.
 * kv_len and q_pos0 stay in tokens; Nkv counts cache slots.
 *
 * Block-sparse attention (block_mask != NULL, contiguous keys only).  Sparse
 * attention built on top of SageAttention skips whole tiles (SpargeAttention
 * and Sparse-Linear Attention in the Vidu S1 blog, section "Infra", and the
 * TurboDiffusion digests); the pages give no predictor, so the caller passes
 * the tile mask: byte block_mask[((b*H + h)*ceil(Nq/128) + i/128)*
 * ceil(Nkv/64) + j/64] != 0 keeps the tile of query i and key j, which is
 * then visible iff the mask above also allows it.  Dropped tiles cost no
 * work.  A query row with no visible key gets an output of 0.  At most
 * SAGE_MAX_MASK_CHUNKS key blocks (SAGE_E_UNSUPPORTED otherwise).  KV splits
 * chosen by the library assume a dense mask (the mask is device memory and
 * is not read on the host); kv_splits overrides.
 *
 * Tensors.  Q [B,H,Nq,d], K and V [B,H,Nkv,d], O [B,H,Nq,d], all of one
 * 16-bit type (fp16 or bf16), device memory, channel dimension contiguous,
 * strides of the b, h and n dimensions given in ELEMENTS.  d is 64 or 128.
 * One head's staged K/V must stay below 2 GiB: ceil(Nkv/128)*128 * d * 2 <
 * 2^31, i.e. Nkv <= 8,388,480 for d = 128 and 16,776,960 for d = 64
 * (SAGE_E_SHAPE otherwise).
 *
 * Ownership.  The caller allocates every device buffer (inputs, output,
 * workspace); the library never allocates, frees or synchronizes (except
 * under SAGE_FLAG_DEBUG_SYNC).  Host arrays (kv_len, q_pos0) are read during
 * the call only.  Buffers must stay alive until the enqueued work completes.
 * O must not alias Q, K, V or the workspace.
 *
 * Errors.  Every entry point returns a sage_status.  Arguments are validated
 * on the host before anything is enqueued; on an error nothing is enqueued
 * and sage_attn_last_error() (thread-local) describes it.  SAGE_OK means
 * "enqueued"; a fault inside a kernel surfaces at the caller's next
 * synchronization.  No C++ exception crosses this boundary.
 *
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Calls are
 * thread-safe and contain no allocation or synchronization, so they can be
 * captured into a hipGraph.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ATTN_ABI_VERSION 4

typedef enum {
  SAGE_OK = 0,
  SAGE_E_NULL = 1,        /* a required pointer is NULL                      */
  SAGE_E_SHAPE = 2,       /* a size is out of range                          */
  SAGE_E_DTYPE = 3,       /* unknown dtype or pv_mode                        */
  SAGE_E_STRIDE = 4,      /* a stride is not a multiple of 8 elements        */
  SAGE_E_ALIGN = 5,       /* a device pointer is not 16-byte aligned         */
  SAGE_E_MASK = 6,        /* kv_len / q_pos0 / frame_len inconsistent        */
  SAGE_E_UNSUPPORTED = 7, /* d not in {64,128}, B > SAGE_MAX_BATCH, ...      */
  SAGE_E_WORKSPACE = 8,   /* workspace missing or too small                  */
  SAGE_E_VERSION = 9,     /* desc->abi_version != SAGE_ATTN_ABI_VERSION      */
  SAGE_E_HIP = 10         /* a kernel launch failed (see last_error)         */
} sage_status;

enum { SAGE_F16 = 0, SAGE_BF16 = 1 };       /* sage_attn_desc.dtype          */
enum { SAGE_PV_16 = 0, SAGE_PV_FP8 = 1,     /* sage_attn_desc.pv_mode        */
       SAGE_PV_AUTO = 2 };                  /* per (b,h), from chan_shift    */

#define SAGE_FLAG_DEBUG_SYNC 0x1u  /* synchronize the stream after each launch */
#define SAGE_MAX_BATCH 128
#define SAGE_MAX_SPLITS 16
#define SAGE_MAX_MASK_CHUNKS 4096  /* key blocks of 64 a block mask may cover */

typedef struct sage_attn_desc {
  int32_t abi_version;  /* must be SAGE_ATTN_ABI_VERSION                      */
  int32_t dtype;        /* SAGE_F16 | SAGE_BF16: Q, K, V and O share it       */
  int32_t pv_mode;      /* SAGE_PV_16 | SAGE_PV_FP8 | SAGE_PV_AUTO (the last
                           with frame_stride 0 only: SAGE_E_UNSUPPORTED)     */
  int32_t B, H, Nq, Nkv, d; /* Nkv = allocated key length (>= every kv_len) */
  int32_t frame_len;    /* 0: no mask; > 0: frame-block-causal, F tokens      */
  int32_t kv_splits;    /* 0: chosen by the library; 1..SAGE_MAX_SPLITS       */
  float sm_scale;       /* softmax scale; 0 -> 1/sqrt(d)                      */
  uint32_t flags;       /* SAGE_FLAG_*                                        */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3]; /* b, h, n     */
  const int32_t *kv_len; /* host [B] valid keys per batch, or NULL: all Nkv
                            (frame cache: Nkv/frame_stride full frames)       */
  const int32_t *q_pos0; /* host [B] absolute position of query 0, or NULL:
                            kv_len[b] - Nq when frame_len > 0                 */
  const float *k_mean_in; /* device [B,H,d] fixed mean to use, or NULL      */
  int32_t frame_stride;   /* 0: K/V tokens contiguous (Nkv = key count);
                             > 0: frame cache of FS slots per frame (see top):
                             multiple of 64, >= frame_len (> 0), < 131072, and
                             Nkv = cache slots, a multiple of it               */
  int32_t sink_frames;    /* S: leading frames always visible (window only)   */
  int32_t window_frames;  /* W: history frames visible besides the sinks and
                             the current frame; 0 = all (needs frame_stride)  */
  int32_t reserved;       /* must be 0                                         */
  const int8_t *chan_shift_in; /* device [B,H,d] fixed channel-balance exponents
                             (in [-64, 64]) to use, or NULL: computed          */
  const uint8_t *block_mask; /* device [B][H][ceil(Nq/128)][ceil(Nkv/64)] bytes,
                             or NULL: block-sparse attention (see top); read
                             by the attention calls only                      */
} sage_attn_desc;

/* Quantized operands, in caller-owned device memory (normally carved out of
 * the workspace by sage_attn_quant_layout).  Nq_pad = ceil(Nq/128)*128 and
 * Nkv_pad = ceil(Nkv/128)*128; padding positions hold code 0 and scale 0. */
typedef struct sage_quant_bufs {
  int8_t *q_codes;     /* [B,H,Nq_pad,d] row-major                            */
  float *q_scale;      /* [B,H,Nq_pad/128]                                    */
  int8_t *k_codes;     /* [B,H,Nkv_pad,d] row-major                           */
  float *k_scale;      /* [B,H,Nkv_pad/64]                                    */
  float *k_mean;       /* [B,H,d]                                             */
  int8_t *chan_shift;  /* [B,H,d] channel-balance exponents a                 */
  void *v_t;           /* [B,H,Nkv_pad/64,d,64]: per 64-key chunk, V transposed
                          (channel-major); 16-bit values in SAGE_PV_16 mode,
                          e4m3fn codes in SAGE_PV_FP8 mode.  SAGE_PV_AUTO:
                          Nkv_pad*d*2 bytes per (b,h), holding that head's
                          16-bit values, or its e4m3fn codes in the first
                          Nkv_pad*d bytes                                    */
  uint8_t *v_e8m0;     /* FP8 and AUTO modes: E8M0 scale bytes,
                          [B,H,Nkv_pad/64,64,4]: per 64-key chunk, byte
                          [32k + r][cb] scales channel 32cb + r of keys
                          [32k, 32k+32) (AUTO: written for the FP8 heads
                          only); else NULL                                   */
  void *stats;         /* internal: partial statistics of the quantize pass;
                          SAGE_PV_AUTO also keeps each mode's head list here,
                          so the attention calls need it in that mode        */
  void *partial;       /* internal: split-KV partial results                  */
  int32_t partial_splits; /* KV splits `partial` holds room for (set by
                          sage_attn_quant_layout): a call whose split count
                          exceeds it fails with SAGE_E_WORKSPACE            */
  int32_t pv_layout;   /* pv_mode the buffers were carved for (set by
                          sage_attn_quant_layout): a SAGE_PV_AUTO call needs
                          SAGE_PV_AUTO here (its V slots and head lists are
                          larger), else SAGE_E_WORKSPACE                     */
} sage_quant_bufs;

/* Version of the library's ABI (SAGE_ATTN_ABI_VERSION it was built with). */
int sage_attn_abi_version(void);

/* Static description of a status code. */
const char *sage_attn_status_string(sage_status status);

/* Thread-local text of the last failure reported by this thread: the
 * validation message, or for SAGE_E_HIP the HIP runtime's error string. */
const char *sage_attn_last_error(void);

/* Value of a named scheme constant ("BQ", "BK", "VB", "QMAX", "TAU",
 * "PSHIFT_FP8", "PSHIFT_16", "KMEAN_CHUNK"), for cross-checks.
 * Returns SAGE_E_UNSUPPORTED for an unknown name. */
sage_status sage_attn_constant(const char *name, double *value);

/* Number of KV splits the library will use for *desc (kv_splits, or its own
 * choice when kv_splits == 0).  Each batch's key chunks form one ordered
 * list, the same for every query tile of the batch, and split s takes
 * entries [s*n/S, (s+1)*n/S) of it (n entries; a tile visits the entries of
 * its part that its rows can see).  Contiguous keys, with or without a
 * block mask: the 64-key chunks [0, ceil(kv_len[b]/64)).  Frame cache: the
 * cache chunks that some query row of the batch sees -- those of the sink
 * frames, then those of the window frames from the first query's window
 * start through the last query's frame (up to its last token).  Partial
 * results are merged exactly as the online softmax would. */
sage_status sage_attn_kv_splits(const sage_attn_desc *desc, int32_t *splits);

/* Bytes of workspace sage_attn_fwd needs for *desc (validated first).  The
 * split-KV region has room for the larger of the split count for *desc and
 * the one for the same desc with every batch at its full key length, so a
 * frame cache carved once keeps working while kv_len grows. */
sage_status sage_attn_workspace_bytes(const sage_attn_desc *desc, size_t *bytes);

/* Carve the quantized-operand buffers out of a workspace of ws_bytes bytes
 * (256-byte aligned sub-buffers) and record the split capacity in
 * out->partial_splits.  Host-only: enqueues nothing. */
sage_status sage_attn_quant_layout(const sage_attn_desc *desc, void *ws, size_t ws_bytes,
                                   sage_quant_bufs *out);

/* Quantize: K mean (unless k_mean_in), channel balance (unless
 * chan_shift_in), INT8 Q and K codes and scales, V prepared for P.V
 * (transposed; FP8 codes and E8M0 scales in FP8 mode).  q, k, v: device
 * inputs as described by desc (with a frame cache, k and v hold the kv_len
 * tokens contiguously; they are written into the cache slots). */
sage_status sage_attn_quantize(const sage_attn_desc *desc, const void *q, const void *k,
                               const void *v, const sage_quant_bufs *bufs, void *stream);

/* Frame cache only (frame_stride > 0): quantize once, against the K mean and
 * channel-balance exponents already in bufs (left there by sage_attn_quantize
 * or written by the caller), the nframes frames [frame0, frame0 + nframes) of
 * new keys and values -- k, v: [B,H,nframes*frame_len,d] with desc's k/v
 * strides -- into their cache slots, for every batch; and, when q is not NULL,
 * the queries q (as described by desc) with the same exponents.  Codes and
 * scales of all other frames are left untouched.  Errors: SAGE_E_UNSUPPORTED
 * without a frame cache; SAGE_E_SHAPE if the frames do not fit in Nkv slots. */
sage_status sage_attn_quantize_frames(const sage_attn_desc *desc, const void *q, const void *k,
                                      const void *v, int32_t frame0, int32_t nframes,
                                      const sage_quant_bufs *bufs, void *stream);

/* As sage_attn_quantize_frames, with each batch appending at its own place:
 * batch b's nframes new frames (rows [0, nframes*frame_len) of its k, v) go to
 * frames [frame0[b], frame0[b] + nframes) of its cache -- the step of B
 * independent streaming sessions, each with a cache of its own length (the
 * streaming setting of the Vidu S1 blog, section "Infra").  frame0: host
 * array [B], read during the call.  Errors as sage_attn_quantize_frames;
 * SAGE_E_NULL if frame0 is NULL; SAGE_E_SHAPE if some batch's frames do not
 * fit in Nkv slots. */
sage_status sage_attn_quantize_frames_batched(const sage_attn_desc *desc, const void *q,
                                              const void *k, const void *v, const int32_t *frame0,
                                              int32_t nframes, const sage_quant_bufs *bufs,
                                              void *stream);

/* Fused attention on already-quantized operands: writes O [B,H,Nq,d].
 * SAGE_PV_AUTO: the heads are split by their exponents in bufs->chan_shift
 * on the device (lists in bufs->stats) and each mode runs as its own launch
 * over its own heads.  Errors: SAGE_E_WORKSPACE if the call needs more KV
 * splits than bufs->partial_splits (a workspace carved for another desc);
 * SAGE_E_NULL for SAGE_PV_AUTO without bufs->stats. */
sage_status sage_attn_fwd_quantized(const sage_attn_desc *desc, const sage_quant_bufs *bufs,
                                    void *o, void *stream);

/* For callers that cannot allocate device memory (code under hipGraph
 * capture, tight serving loops, harnesses that forbid allocation): as
 * sage_attn_fwd_quantized, except that the split-KV partial results go to a
 * device scratch array inside the library (128 MiB, one per GPU, held until
 * the process ends) instead of bufs->partial, which may be NULL.  The call
 * allocates and frees nothing.  Its split count (kv_splits or the library's
 * choice) needs splits * B * H * ceil(Nq/128)*128 * (d + 2) * 4 bytes of
 * that scratch when splits > 1: more fails with SAGE_E_WORKSPACE, before
 * anything is enqueued.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (concurrent streams, threads) race; the
 * kernels write every partial they read, so nothing needs clearing between
 * calls.  The stream must belong to the current device
 * (SAGE_E_UNSUPPORTED otherwise). */
sage_status sage_attn_fwd_quantized_noalloc(const sage_attn_desc *desc, const sage_quant_bufs *bufs,
                                            void *o, void *stream);

/* Drop-in call: quantize into the workspace, then attend.  Equivalent to
 * sage_attn_quant_layout + sage_attn_quantize + sage_attn_fwd_quantized. */
sage_status sage_attn_fwd(const sage_attn_desc *desc, const void *q, const void *k,
                          const void *v, void *o, void *ws, size_t ws_bytes, void *stream);

/* Test support: exact int32 scores S = qcodes . kcodes^T of ntiles tiles of
 * 32 queries x 64 keys, computed by the same matrix-core routine as the fused
 * kernel.  tiles: host [ntiles][3] = {b*H + h, q0 (multiple of 32),
 * k0 (multiple of 64)} within the padded sizes; out: device [ntiles][32][64]
 * int32, row = query q0+r, column = key k0+c. */
sage_status sage_attn_debug_scores_i32(const sage_attn_desc *desc, const sage_quant_bufs *bufs,
                                      const int32_t *tiles, int32_t ntiles, int32_t *out,
                                      void *stream);

/* Test support: apply to n float32 values the kernels' own conversion
 * routines.  kind 0: e4m3fn bytes (as P is converted in FP8 mode);
 * 1: bf16 bits; 2: fp16 bits (uint16); 3: float32 2^x by the same hardware
 * exponential the softmax uses.  Inputs for kind 0 must satisfy
 * |x| <= 448. */
sage_status sage_attn_debug_convert(int kind, const float *in, void *out, int64_t n,
                                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
