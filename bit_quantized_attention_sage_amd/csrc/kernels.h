// Host-side launch descriptions shared by the C ABI (api.cpp) and the kernel
// translation units.  Plain structs; no allocation anywhere.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sage_attn.h"
#include "common.h"

namespace sage {

constexpr int MAXB_ARGS = 128;  // batches passed by value in kernel arguments

// Per-batch mask data, copied into the kernel arguments of every launch.
struct BatchInfo {
  int kv_len[MAXB_ARGS];
  int q_pos0[MAXB_ARGS];
  int frame0[MAXB_ARGS];  // per-batch frame appends: the first frame of batch b's new frames
};

struct QuantLaunch {
  int dtype, pv_mode, d;
  int B, H, Nq, Nkv, Nq_pad, Nkv_pad;
  const void *q, *k, *v;
  int64_t qs[3], ks[3], vs[3];
  const float* k_mean_in;
  const int8_t* chan_shift_in;
  int frame_len, frame_stride;  // frame cache when frame_stride > 0
  int frames_only;              // 1: quantize frames [frame0, frame0 + nframes) (q optional)
  int frame0, nframes;          // frame0 < 0: each batch from its own bi.frame0[b]
  BatchInfo bi;
  sage_quant_bufs bufs;
  // views into bufs.stats
  double* stat_ksum;
  float *stat_kmax, *stat_kmin, *stat_qamax;
};

struct AttnLaunch {
  int dtype, pv_mode, d;
  int B, H, Nq, Nkv, Nq_pad, Nkv_pad;
  int frame_len, splits;
  int frame_stride, sink_frames, window_frames;  // frame cache and window
  uint32_t cpf_magic;  // ceil(2^32 / (frame_stride / 64)): chunk -> frame by __umulhi
  const uint8_t* block_mask;  // [B,H,Nq_pad/128,mask_nkc] or null
  int mask_nkc;               // ceil(Nkv / 64)
  float sigma;  // fp32(sm_scale * log2 e)
  BatchInfo bi;
  int order[MAXB_ARGS];  // batches by decreasing kv_len (longest first)
  sage_quant_bufs bufs;
  void* o;
  int64_t os[3];
  int64_t vt_hb;  // bytes of one (b,h)'s V^T operand in bufs.v_t
  int* pick;      // SAGE_PV_AUTO: [1 + B*H] 16-bit heads then [1 + B*H] FP8
                  // heads (count, then b*H + h in batch order); else null
};

// Per-block W8A8 linear layer (w8a8.hip).
struct W8A8Launch {
  int dtype;
  int M, M_pad, N, K;  // M_pad = ceil(M/128)*128
  int64_t xs, ws, ys;  // row strides (elements) of X, W and Y
};

hipError_t launch_w8a8_quant_act(const W8A8Launch& L, const void* x, int8_t* xq, float* xscale, hipStream_t st);
hipError_t launch_w8a8_quant_weight(const W8A8Launch& L, const void* w, int8_t* wq, float* wscale, hipStream_t st);
hipError_t launch_w8a8_gemm(const W8A8Launch& L, const int8_t* xq, const float* xscale, const int8_t* wq,
                            const float* wscale, const void* bias, void* y, hipStream_t st);

// Device scratch of the allocation-free entry point (attn.hip): its size, and
// its address on the current device (fetched once per device).
constexpr size_t SCRATCH_BYTES = size_t{128} << 20;
constexpr int MAX_DEVICES = 64;
hipError_t scratch_address(void** ptr);

hipError_t launch_quantize(const QuantLaunch& L, hipStream_t st);
hipError_t launch_attention(const AttnLaunch& L, hipStream_t st);
hipError_t launch_debug_scores(const AttnLaunch& L, const int32_t* tiles, int ntiles,
                               int32_t* out, hipStream_t st);
hipError_t launch_convert(int kind, const float* in, void* out, int64_t n, hipStream_t st);

}  // namespace sage
