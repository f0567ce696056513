// Per-block W8A8 INT8 linear layer for gfx950: Y = X W^T (+ bias) with X
// quantized per (row, 128-channel group) and W per 128 x 128 tile, the
// products taken on the INT8 matrix cores.
//
// Why: per-tensor and per-channel scales let outliers widen the quantization
// range, so the linear layers of the pages' video models use a per-block
// W8A8 GEMM (Vidu S1 blog, section "Infra"), on the INT8 units (TurboDiffusion
// digests).  The block shapes are this library's reading: a channel outlier
// of an activation only widens its own 128-channel group of its own token.
//
//   Y[m, n] = bias[n] + sum_kb dx[kb][m] * dw[n / 128][kb] * S_kb[m, n]
//   S_kb[m, n] = sum over the 128 channels k of block kb of xq[m, k] * wq[n, k]
//
// S_kb is exact in int32 (|S| <= 127^2 * 128).  Each K block's int32 result is
// converted and added to a float32 running sum with one FMA by its scale
// dx * dw (rounded to float32 once).
//
// GEMM decomposition.  One workgroup = 8 waves = a tile of 128 rows (tokens)
// x 256 output features; wave w takes rows 64*(w&1) + [0,64) and features
// 64*(w>>1) + [0,64) (half a weight block of N).  Per K block of 128
// channels the X tile (128 x 128 bytes) and the W tile (256 x 128 bytes) are
// staged from HBM straight into LDS (buffer loads with an LDS destination,
// double-buffered), and each wave runs 2 x 2 x 4 = 16 MFMAs i32 32x32x32:
// for each 32-token group t, S^T(t) = W X_t^T as in the fused attention
// kernel's score tile (W rows in the A operand, permuted by a_row_key, X
// rows as the B operand), so lane l ends with token 32t + l%32 and 16
// consecutive features of each 32-feature subtile.
//
// Ping-pong.  Waves w and w+4 share a SIMD.  Each K block is two phases
// split by a barrier, the MFMAs (at raised wave priority) and the
// dequantization into the float32 sums, and waves 4-7 run one phase behind
// waves 0-3, so on every SIMD one wave's MFMAs overlap the other's VALU work
// (one wave alone issues FP32 VALU ops only every ~5 cycles, and its own
// MFMAs hide little of it).
//
// Staging.  Three buffers per tile: while the MFMAs of block kb read buffer
// kb % 3, every wave stages its share of block kb + 2 (6 DMA instructions,
// one behind each of its first MFMAs) into buffer (kb + 2) % 3, which both
// groups finished reading in block kb - 1.  A wave waits for its DMA of
// block kb + 1 at the barrier that ends its own MFMA phase of block kb, which
// is before either group's first read of block kb + 1; the DMA of block
// kb + 2 stays in flight.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sage {

namespace {

constexpr int WG = 128;      // K channels per block; N rows per weight block
constexpr int TM = 128;      // tokens per workgroup tile
constexpr int TN = 256;      // output features per workgroup tile
constexpr int XB = TM * WG;  // bytes of a staged X tile
constexpr int WB = TN * WG;  // bytes of a staged W tile

// X tile granule swizzle: granule g of row r at slot g ^ ((r >> 1) & 7).  A
// ds_read_b128 B-operand read has 16 lanes read 16 consecutive rows at one
// granule; rows are 128 bytes, so the 16 slots 8*(r&1) + (g ^ ((r>>1)&7)) are
// distinct.
__device__ __forceinline__ int x_swz(int r) { return (r >> 1) & 7; }

}  // namespace

// Activations: one 16-lane group per (row, 128-channel group), 8 channels per
// lane.  Rows in [M, M_pad) get zero codes and scales.
template <typename T>
__global__ __launch_bounds__(256) void w8a8_quant_act_kernel(const T* __restrict__ x, int64_t xs, int M, int M_pad,
                                                             int K, int8_t* __restrict__ xq,
                                                             float* __restrict__ xscale) {
  const int ngrp = K / WG;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (gid >= static_cast<int64_t>(M_pad) * ngrp) return;  // whole 16-lane groups leave together
  const int m = static_cast<int>(gid / ngrp), g = static_cast<int>(gid % ngrp);
  float v[8];
  if (m < M) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + m * xs + g * WG + 8 * sub);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = to_f32(T{static_cast<uint16_t>((w4[c / 2] >> (16 * (c % 2))) & 0xFFFFu)});
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(v[c]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  const float q127 = static_cast<float>(QMAX);
  const float delta = amax > 0.f ? amax / q127 : 0.f;
  const float inv = amax > 0.f ? q127 / amax : 0.f;
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float y = v[c] * inv;
    const int code = static_cast<int>(fminf(fmaxf(__builtin_rintf(y), -q127), q127));
    packed[c / 4] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (c % 4));
  }
  *reinterpret_cast<uint2*>(xq + static_cast<int64_t>(m) * K + g * WG + 8 * sub) = make_uint2(packed[0], packed[1]);
  if (sub == 0) xscale[static_cast<int64_t>(g) * M_pad + m] = delta;
}

// Weights: one workgroup per 128 x 128 tile; thread t takes 8 channels of
// rows t/16 + 16 j (j < 8).
template <typename T>
__global__ __launch_bounds__(256) void w8a8_quant_weight_kernel(const T* __restrict__ w, int64_t ws, int K,
                                                                int8_t* __restrict__ wq,
                                                                float* __restrict__ wscale) {
  __shared__ float red[4];
  const int kb = blockIdx.x, nb = blockIdx.y;
  const int t = threadIdx.x, c8 = (t & 15) * 8, r0 = t >> 4;
  float v[8][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = nb * WG + r0 + 16 * j;
    const uint4 raw = *reinterpret_cast<const uint4*>(w + n * ws + kb * WG + c8);
    const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[j][c] = to_f32(T{static_cast<uint16_t>((w4[c / 2] >> (16 * (c % 2))) & 0xFFFFu)});
      amax = fmaxf(amax, fabsf(v[j][c]));
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float q127 = static_cast<float>(QMAX);
  const float delta = amax > 0.f ? amax / q127 : 0.f;
  const float inv = amax > 0.f ? q127 / amax : 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float y = v[j][c] * inv;
      const int code = static_cast<int>(fminf(fmaxf(__builtin_rintf(y), -q127), q127));
      packed[c / 4] |= (static_cast<uint32_t>(code) & 0xFFu) << (8 * (c % 4));
    }
    const int n = nb * WG + r0 + 16 * j;
    *reinterpret_cast<uint2*>(wq + static_cast<int64_t>(n) * K + kb * WG + c8) = make_uint2(packed[0], packed[1]);
  }
  if (t == 0) wscale[static_cast<int64_t>(nb) * (K / WG) + kb] = delta;
}

struct GemmArgs {
  const int8_t* xq;      // [M_pad][K]
  const float* xscale;   // [K/128][M_pad]
  const int8_t* wq;      // [N][K]
  const float* wscale;   // [N/128][K/128]
  const void* bias;      // [N] 16-bit, or null
  void* y;               // [M][N] 16-bit, row stride ys
  int64_t ys;
  int M, M_pad, N, K;
  int mt, nt;            // tiles along M and N
};

template <int DT>
__global__ __launch_bounds__(512, 1) void w8a8_gemm_kernel(GemmArgs A) {
  // (separate objects, so that the compiler can tell the buffer being filled
  // by DMA from the ones being read)
  __shared__ __attribute__((aligned(16))) int8_t xL0[XB];
  __shared__ __attribute__((aligned(16))) int8_t xL1[XB];
  __shared__ __attribute__((aligned(16))) int8_t xL2[XB];
  __shared__ __attribute__((aligned(16))) int8_t wL0[WB];
  __shared__ __attribute__((aligned(16))) int8_t wL1[WB];
  __shared__ __attribute__((aligned(16))) int8_t wL2[WB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, r32 = lane & 31;

  // Tile order: groups of 8 row tiles sweep the feature tiles together, so
  // the 32 workgroups an XCD runs at once share X and W slices in its L2.
  const int total = A.mt * A.nt;
  const int L = xcd_remap(blockIdx.x, total);
  constexpr int GM = 8;
  const int grp = L / (GM * A.nt), first = grp * GM;
  const int gsz = min(GM, A.mt - first);
  const int rem = L - grp * GM * A.nt;
  const int mtile = first + rem % gsz, ntile = rem / gsz;
  const int m0 = mtile * TM, n0 = ntile * TN;
  const int mw = m0 + 64 * (w & 1);   // this wave's rows
  const int nw = n0 + 64 * (w >> 1);  // this wave's 64 features (half a weight block)
  const int nkb = A.K / WG;

  // Staging (all 8 waves): DMA instruction i of wave w fills LDS granule
  // (8i + w)*64 + lane of a tile; its global source is chosen so that the
  // tile ends up swizzled.
  // Rows past M (X) read zero codes from the padding rows; rows past N (W)
  // are outside the buffer and read as zero.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(A.xq), 0, static_cast<int>(static_cast<int64_t>(A.M_pad) * A.K), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(A.wq), 0, static_cast<int>(static_cast<int64_t>(A.N) * A.K), 0x00020000);
  constexpr int XI = XB / 8192, WI = WB / 8192;  // 1 KB DMA instructions per wave and block
  constexpr int NDMA = XI + WI;
  const int wgrp = w >> 2;
  int xoff[XI], woff[WI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int s = (8 * i + w) * 64 + lane, r = s / 8, gp = s % 8;
    xoff[i] = (m0 + r) * A.K + ((gp ^ x_swz(r)) << 4);
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int s = (8 * i + w) * 64 + lane, r = s / 8, gp = s % 8;  // r: row of the 256-row tile
    const int key = r & 63;
    // a row past N points at the buffer's end, which reads as zero
    woff[i] = n0 + r < A.N ? (n0 + r) * A.K + ((gp ^ k_swz<128>(key)) << 4) : A.N * A.K;
  }
  auto dma = [&](int8_t* xd, int8_t* wd, int kb) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int off = xoff[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, xd + (8 * i + w) * 1024, 16, off, kb * WG, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      const int off = woff[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, wd + (8 * i + w) * 1024, 16, off, kb * WG, 0, 0);
    }
  };

  const int wr_base = 64 * (w >> 1);

  constexpr int NU = 1;  // 64-feature groups per wave
  v16f y[NU][2][2];  // [feature group u][token group t][subtile s]
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s) y[u][t][s] = v16f{0.f};

  // Scales of K block kb: this lane's two tokens x the wave's weight block.
  // They are loaded one block ahead, at the start of a dequantization phase,
  // so that the next step's wait for its DMA covers them.
  const float* dxp = A.xscale + mw + r32;
  // (a wave whose features lie past N computes on zero weights and stores
  // nothing; it reads the last weight block's scales)
  const float* dwp = A.wscale + static_cast<int64_t>(min(nw, A.N - WG) / WG) * nkb;
  float dx0, dx1, dwv;
  auto load_scales = [&](int kb) {
    const int k = min(kb, nkb - 1);
    dx0 = dxp[static_cast<int64_t>(k) * A.M_pad];
    dx1 = dxp[static_cast<int64_t>(k) * A.M_pad + 32];
    dwv = dwp[k];
  };

  load_scales(0);
  dma(xL0, wL0, 0);
  if (nkb > 1) dma(xL1, wL1, 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  v16i s[2][2];  // [t][subtile]: int32 products of the current K block
  // ln: the lane.  This lane's rows in the X tile (B operand: token r32 of
  // group t, bytes [32 ks + 16 h2, +16)) and rows in the W tile (A operand,
  // two 64-row halves).
  auto mma = [&](const int8_t* xl, const int8_t* wl, int ln) {
    const int r32l = ln & 31, h2l = ln >> 5;
    const int xr0 = 64 * (w & 1) + r32l, xr1 = xr0 + 32;
    const int key0 = a_row_key(r32l, 0), key1 = a_row_key(r32l, 1);
    const int sw0 = k_swz<128>(key0), sw1 = k_swz<128>(key1);
    v4i xb[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int g = 2 * ks + h2l;
      xb[0][ks] = *reinterpret_cast<const v4i*>(xl + xr0 * WG + ((g ^ x_swz(xr0)) << 4));
      xb[1][ks] = *reinterpret_cast<const v4i*>(xl + xr1 * WG + ((g ^ x_swz(xr1)) << 4));
    }
    const int8_t* wt = wl + wr_base * WG;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int g = 2 * ks + h2l;
      const v4i a0 = *reinterpret_cast<const v4i*>(wt + key0 * WG + ((g ^ sw0) << 4));
      const v4i a1 = *reinterpret_cast<const v4i*>(wt + key1 * WG + ((g ^ sw1) << 4));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (ks == 0) {
          s[t][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, xb[t][0], v16i{0}, 0, 0, 0);
          s[t][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, xb[t][0], v16i{0}, 0, 0, 0);
        } else {
          s[t][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, xb[t][ks], s[t][0], 0, 0, 0);
          s[t][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, xb[t][ks], s[t][1], 0, 0, 0);
        }
      }
    }
  };
  auto deq = [&](float c0, float c1) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float c = t ? c1 : c0;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          y[0][t][sub][i] = __builtin_fmaf(static_cast<float>(s[t][sub][i]), c, y[0][t][sub][i]);
    }
  };
  // One K block: the MFMA phase (with this wave's DMA of block kb + 2), the
  // wait for its DMA of block kb + 1, a barrier, the dequantization phase and
  // a barrier.  Group 1 runs one phase behind group 0.  B: the buffer of
  // block kb (kb % 3).
  auto step = [&](auto bc, auto sc, int kb) {
    constexpr int B = decltype(bc)::value;
    constexpr bool stage = decltype(sc)::value;  // kb + 2 < nkb
    const int8_t* xl = B == 0 ? xL0 : B == 1 ? xL1 : xL2;
    const int8_t* wl = B == 0 ? wL0 : B == 1 ? wL1 : wL2;
    int8_t* xn = B == 0 ? xL2 : B == 1 ? xL0 : xL1;  // buffer (kb + 2) % 3
    int8_t* wn = B == 0 ? wL2 : B == 1 ? wL0 : wL1;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    if constexpr (stage) {
      dma(xn, wn, kb + 2);
      mma(xl, wl, lane);
      // the X operand reads and the first two k-steps' W reads, then the
      // other W reads and this wave's DMA one behind each MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // one MFMA
        if (g < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA
        if (g < 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // a W operand read
      }
    } else {
      mma(xl, wl, lane);
    }
    asm volatile("" : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // this wave's DMA of block kb + 1 (and the scales) landed; that of block
    // kb + 2 (the NDMA loads issued last) may still be in flight
    if constexpr (stage)
      __builtin_amdgcn_s_waitcnt(0x0F70 | NDMA);  // vmcnt(NDMA)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // block kb's scales (loaded one step ahead, waited for with the DMA);
    // then the next block's, which the next step's DMA wait covers
    const float c0 = dx0 * dwv, c1 = dx1 * dwv;  // fp32(dx dw), rounded once
    load_scales(kb + 1);
    deq(c0, c1);
    // the sums are final here: without this the compiler sinks the
    // dequantization into the next block and keeps several blocks' int32
    // tiles alive
    asm volatile("" : "+v"(y[0][0][0]), "+v"(y[0][0][1]), "+v"(y[0][1][0]), "+v"(y[0][1][1]));
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;

  using Stage = std::integral_constant<bool, true>;
  using Last = std::integral_constant<bool, false>;

  // The blocks that stage block kb + 2 (all but the last two), then the last
  // two; each in its own copy of the step, so that no branch inside a step
  // leaves the compiler unsure which loads are still in flight.
  if (wgrp == 1) __builtin_amdgcn_s_barrier();  // one phase behind group 0
  const int nst = max(nkb - 2, 0);
  int kb = 0;
  for (; kb + 3 <= nst; kb += 3) {
    step(B0{}, Stage{}, kb);
    step(B1{}, Stage{}, kb + 1);
    step(B2{}, Stage{}, kb + 2);
  }
  if (kb < nst) step(B0{}, Stage{}, kb++);
  if (kb < nst) step(B1{}, Stage{}, kb++);
  // kb = nst here: at most two blocks left, starting in buffer kb % 3
  switch (kb % 3) {
    case 0:
      step(B0{}, Last{}, kb);
      if (kb + 1 < nkb) step(B1{}, Last{}, kb + 1);
      break;
    case 1:
      step(B1{}, Last{}, kb);
      if (kb + 1 < nkb) step(B2{}, Last{}, kb + 1);
      break;
    default:
      step(B2{}, Last{}, kb);
      if (kb + 1 < nkb) step(B0{}, Last{}, kb + 1);
      break;
  }
  if (wgrp == 0) __builtin_amdgcn_s_barrier();  // as many barriers as group 1

  // ---- epilogue: + bias, round, store (lane: token 32t + r32, features
  // nw + 64u + 32 sub + 16 h2 + [0, 16))
  if (nw >= A.N) return;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int nf = nw + 64 * u + 32 * sub + 16 * h2;
      float bv[16];
      if (A.bias) {
        const uint4* bp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(A.bias) + nf);
        const uint4 b0 = bp[0], b1 = bp[1];
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          bv[2 * i] = Pack16<DT>::lo(bw[i]);
          bv[2 * i + 1] = Pack16<DT>::hi(bw[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) bv[i] = 0.f;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int m = mw + 32 * t + r32;
        if (m >= A.M) continue;
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pk[i] = Pack16<DT>::pack(y[u][t][sub][2 * i] + bv[2 * i], y[u][t][sub][2 * i + 1] + bv[2 * i + 1]);
        uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(A.y) + m * A.ys + nf);
        dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      }
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_w8a8_quant_act(const W8A8Launch& L, const void* x, int8_t* xq, float* xscale, hipStream_t st) {
  const int64_t groups = static_cast<int64_t>(L.M_pad) * (L.K / WG);
  const dim3 grid(static_cast<unsigned>((groups + 15) / 16));
  if (L.dtype == DT_BF16)
    hipLaunchKernelGGL(w8a8_quant_act_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(x),
                       L.xs, L.M, L.M_pad, L.K, xq, xscale);
  else
    hipLaunchKernelGGL(w8a8_quant_act_kernel<f16_t>, grid, dim3(256), 0, st, static_cast<const f16_t*>(x),
                       L.xs, L.M, L.M_pad, L.K, xq, xscale);
  return hipGetLastError();
}

hipError_t launch_w8a8_quant_weight(const W8A8Launch& L, const void* w, int8_t* wq, float* wscale, hipStream_t st) {
  const dim3 grid(L.K / WG, L.N / WG);
  if (L.dtype == DT_BF16)
    hipLaunchKernelGGL(w8a8_quant_weight_kernel<bf16_t>, grid, dim3(256), 0, st, static_cast<const bf16_t*>(w),
                       L.ws, L.K, wq, wscale);
  else
    hipLaunchKernelGGL(w8a8_quant_weight_kernel<f16_t>, grid, dim3(256), 0, st, static_cast<const f16_t*>(w),
                       L.ws, L.K, wq, wscale);
  return hipGetLastError();
}

hipError_t launch_w8a8_gemm(const W8A8Launch& L, const int8_t* xq, const float* xscale, const int8_t* wq,
                            const float* wscale, const void* bias, void* y, hipStream_t st) {
  GemmArgs A{};
  A.xq = xq;
  A.xscale = xscale;
  A.wq = wq;
  A.wscale = wscale;
  A.bias = bias;
  A.y = y;
  A.ys = L.ys;
  A.M = L.M;
  A.M_pad = L.M_pad;
  A.N = L.N;
  A.K = L.K;
  A.mt = L.M_pad / TM;
  A.nt = (L.N + TN - 1) / TN;
  const dim3 grid(static_cast<unsigned>(A.mt * A.nt));
  if (L.dtype == DT_BF16)
    hipLaunchKernelGGL(w8a8_gemm_kernel<DT_BF16>, grid, dim3(512), 0, st, A);
  else
    hipLaunchKernelGGL(w8a8_gemm_kernel<DT_F16>, grid, dim3(512), 0, st, A);
  return hipGetLastError();
}

}  // namespace sage
