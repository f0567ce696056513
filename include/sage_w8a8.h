/*
 * sage_w8a8.h -- C ABI of the per-block W8A8 INT8 linear layer of the same
 * library (libsage_attn.so), for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Y = X W^T + bias with X [M,K] (activations) and W [N,K]
 * (weights) quantized to INT8 per block and multiplied on the INT8 matrix
 * cores.  The Vidu S1 blog (section "Infra") gives the reason: per-tensor and
 * per-channel scales let outliers widen the quantization range and lose
 * precision, so its video model's linear layers use a per-block W8A8
 * quantized GEMM; the TurboDiffusion digests add that weights and
 * activations are quantized block-wise to 8 bits for the INT8 units.  The
 * block shapes are this library's reading:
 *   - X: one scale per (row, group of 128 channels);
 *   - W: one scale per 128 x 128 tile (128 output features x 128 channels);
 *   - each block: delta = amax / 127, code = rint(x * (127 / amax)) in
 *     [-127, 127] (fp32, ties to even; an all-zero block has delta 0);
 *   - Y[m,n] = bias[n] + sum over K blocks kb of fp32(dx[m,kb] * dw[n/128,kb])
 *     * S_kb[m,n], where S_kb is the exact int32 product of the codes over
 *     the block's 128 channels, accumulated in float32 and rounded (RNE) to
 *     the 16-bit output type.
 *
 * Ownership and errors as in sage_attn.h: the caller allocates every device
 * buffer; nothing is allocated or synchronized (except under
 * SAGE_FLAG_DEBUG_SYNC); arguments are validated on the host before anything
 * is enqueued, errors are sage_status codes with sage_attn_last_error().
 * Calls are asynchronous on `stream` (a hipStream_t, NULL = default).
 */
#ifndef SAGE_W8A8_H
#define SAGE_W8A8_H

#include "sage_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_W8A8_GROUP 128

typedef struct sage_w8a8_desc {
  int32_t abi_version;  /* must be SAGE_ATTN_ABI_VERSION                      */
  int32_t dtype;        /* SAGE_F16 | SAGE_BF16: X, W, bias and Y share it    */
  int32_t M, N, K;      /* M >= 1 rows; N and K multiples of 128; M_pad * K
                           and N * K below 2^31 (M_pad = ceil(M/128)*128)     */
  int32_t reserved;     /* must be 0                                           */
  int64_t x_stride;     /* row stride of X in elements (>= K, multiple of 8)  */
  int64_t w_stride;     /* row stride of W in elements (>= K, multiple of 8)  */
  int64_t y_stride;     /* row stride of Y in elements (>= N, multiple of 8)  */
  uint32_t flags;       /* SAGE_FLAG_DEBUG_SYNC                                */
} sage_w8a8_desc;

/* Bytes of the quantized activations: xq [M_pad][K] int8 (rows >= M zero)
 * and x_scale [K/128][M_pad] float32 (block-major: one row per channel
 * group), and of the quantized weights: wq [N][K] int8 and w_scale
 * [N/128][K/128] float32.  Any pointer may be NULL. */
sage_status sage_w8a8_sizes(const sage_w8a8_desc *desc, size_t *xq_bytes, size_t *x_scale_bytes,
                    size_t *wq_bytes, size_t *w_scale_bytes);

/* Quantize the weights W [N,K] (device, 16-bit, row stride w_stride) into wq
 * and w_scale (device).  Done once per layer. */
sage_status sage_w8a8_quantize_weight(const sage_w8a8_desc *desc, const void *w, int8_t *wq,
                              float *w_scale, void *stream);

/* Quantize the activations X [M,K] (device, 16-bit, row stride x_stride) into
 * xq and x_scale (device). */
sage_status sage_w8a8_quantize_act(const sage_w8a8_desc *desc, const void *x, int8_t *xq,
                           float *x_scale, void *stream);

/* Y [M,N] (device, 16-bit, row stride y_stride) = dequantized xq wq^T + bias.
 * bias: device [N] 16-bit, or NULL.  xq, wq, y and bias 16-byte aligned. */
sage_status sage_w8a8_gemm(const sage_w8a8_desc *desc, const int8_t *xq, const float *x_scale,
                   const int8_t *wq, const float *w_scale, const void *bias, void *y,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_W8A8_H */
