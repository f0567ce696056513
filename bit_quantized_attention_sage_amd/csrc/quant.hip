// Quantize pass: K mean-smoothing, channel balance, per-block INT8 codes for Q
// and K, and V laid out (and, in FP8 mode, encoded) for the P.V matrix cores.
//
// The pages ask SageAttention to beat the precision loss of low-bit compute
// (podcast notes, section "02:48 There were clearly faster compute units on
// the hardware") but give no scheme; this is the library's stated one.  Every
// step is HBM-bound: each kernel streams its tensor once with 16-byte loads.
// This translation unit is compiled with floating-point contraction off so
// each operation rounds exactly as written.
#include "common.h"
#include "kernels.h"

namespace sage {

// ---------------------------------------------------------------- statistics
// One thread per (128-token chunk, group of 8 channels).  K: float64 sums in
// ascending token order, plus max and min; Q: max |x|.  Tokens at or beyond
// n_valid take no part.  A thread loads SP_BATCH rows before using any (a
// mid-size tensor gives about two waves per SIMD, so the loads in flight per
// thread set the bandwidth), then adds them in token order.
constexpr int SP_BATCH = 16;
template <typename T, int D, bool IS_K>
__global__ __launch_bounds__(256) void stats_partial_kernel(
    const T* __restrict__ x, int64_t sb, int64_t sh, int64_t sn, int H, int nchunk,
    BatchInfo bi, int n_all, double* __restrict__ psum, float* __restrict__ pmax,
    float* __restrict__ pmin) {
  constexpr int G = D / 8;
  constexpr int CPB = 256 / G;
  const int b = blockIdx.z, h = blockIdx.y;
  const int chunk = blockIdx.x * CPB + threadIdx.x / G;
  const int g = threadIdx.x % G;
  if (chunk >= nchunk) return;
  const int n_valid = IS_K ? bi.kv_len[b] : n_all;
  const int j0 = chunk * KMEAN_CHUNK;
  const int j1 = min(j0 + KMEAN_CHUNK, n_valid);
  const T* base = x + b * sb + h * sh + 8 * g;
  double s[8];
  float mx[8], mn[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s[c] = 0.0;
    mx[c] = -__builtin_inff();
    mn[c] = __builtin_inff();
  }
  for (int jb = j0; jb < j1; jb += SP_BATCH) {
    // rows past j1 repeat row j1 - 1 (in bounds) and are not used
    uint4 raw[SP_BATCH];
#pragma unroll
    for (int k = 0; k < SP_BATCH; ++k)
      raw[k] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(min(jb + k, j1 - 1)) * sn);
#pragma unroll
    for (int k = 0; k < SP_BATCH; ++k) {
      const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
      const bool use = jb + k < j1;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t bits = (w[c / 2] >> (16 * (c % 2))) & 0xFFFFu;
        const float v = to_f32(T{static_cast<uint16_t>(bits)});
        if (IS_K) {
          // (a repeated row changes no maximum or minimum; it is not summed)
          if (use) s[c] += static_cast<double>(v);
          mx[c] = fmaxf(mx[c], v);
          mn[c] = fminf(mn[c], v);
        } else {
          mx[c] = fmaxf(mx[c], fabsf(v));
        }
      }
    }
  }
  const int64_t o = ((static_cast<int64_t>(b) * H + h) * nchunk + chunk) * D + 8 * g;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (IS_K) {
      psum[o + c] = s[c];
      pmin[o + c] = mn[c];
    }
    pmax[o + c] = mx[c];
  }
}

// One workgroup of SF_THREADS per (b, h): the mean and the channel-balance
// exponent of every channel.  The partials are staged through LDS in tiles
// of SF_TILE runs, loaded by the whole workgroup (consecutive threads take
// consecutive channels: coalesced, many loads in flight), and thread c adds
// channel c's sums from LDS in ascending run order: the fp64 sum keeps its
// sequential order (runs past the end are not added).  Maxima and minima,
// which no order changes, are reduced while staging and merged at the end.
constexpr int SF_THREADS = 512;
constexpr int SF_TILE = 64;  // runs per LDS tile: 64 x 128 channels x 8 B = 64 KB
template <int D>
__global__ __launch_bounds__(SF_THREADS) void stats_final_kernel(int H, int nchunk_k, int nchunk_q,
                                                                 BatchInfo bi, const double* __restrict__ ksum,
                                                                 const float* __restrict__ kmax,
                                                                 const float* __restrict__ kmin,
                                                                 const float* __restrict__ qamax,
                                                                 const float* __restrict__ k_mean_in,
                                                                 const int8_t* __restrict__ shift_in,
                                                                 float* __restrict__ mu_out,
                                                                 int8_t* __restrict__ shift_out) {
  constexpr int PER = SF_TILE * D / SF_THREADS;  // elements of a tile per thread
  __shared__ double tile[SF_TILE * D];
  __shared__ float red[3][SF_THREADS];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / H;
  const int n = bi.kv_len[b];
  const int nch = (n + KMEAN_CHUNK - 1) / KMEAN_CHUNK;
  const int64_t base_k = static_cast<int64_t>(bh) * nchunk_k * D;
  float mx = -__builtin_inff(), mn = __builtin_inff(), qa = 0.f;
  double s = 0.0;
  for (int t0 = 0; t0 < nch; t0 += SF_TILE) {
    const int nt = min(SF_TILE, nch - t0);
    // all of this thread's loads of the tile first, then their use (element
    // e = run t0 + e / D, channel e % D = tid % D; elements past the last run
    // repeat that channel's last run, which changes no maximum and is never
    // summed)
    double v[PER];
    float x[PER], z[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int r = min((tid + k * SF_THREADS) / D, nt - 1);
      const int64_t g = base_k + static_cast<int64_t>(t0 + r) * D + tid % D;
      v[k] = ksum[g];
      x[k] = kmax[g];
      z[k] = kmin[g];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      tile[tid + k * SF_THREADS] = v[k];
      mx = fmaxf(mx, x[k]);
      mn = fminf(mn, z[k]);
    }
    __syncthreads();
    if (tid < D)
      for (int t = 0; t < nt; ++t) s += tile[t * D + tid];
    __syncthreads();
  }
  // Q's channel maxima: 16 loads in flight per thread (runs past the end
  // repeat the thread's channel in the last run)
  const float* qx = qamax + static_cast<int64_t>(bh) * nchunk_q * D + tid % D;
  constexpr int RPT = SF_THREADS / D;  // runs per pass of the workgroup
  for (int r0 = tid / D; r0 < nchunk_q; r0 += 16 * RPT) {
    float a[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = qx[static_cast<int64_t>(min(r0 + k * RPT, nchunk_q - 1)) * D];
#pragma unroll
    for (int k = 0; k < 16; ++k) qa = fmaxf(qa, a[k]);
  }
  // (SF_THREADS is a multiple of D, so thread tid only ever saw channel tid % D)
  red[0][tid] = mx;
  red[1][tid] = mn;
  red[2][tid] = qa;
  __syncthreads();
  if (tid >= D) return;
  const int c = tid;
  for (int j = c + D; j < SF_THREADS; j += D) {
    mx = fmaxf(mx, red[0][j]);
    mn = fminf(mn, red[1][j]);
    qa = fmaxf(qa, red[2][j]);
  }
  const float mu = k_mean_in ? k_mean_in[static_cast<int64_t>(bh) * D + c]
                             : static_cast<float>(s / static_cast<double>(n));
  // fp32 rounding of K - mu is monotone in K, so the extreme smoothed values
  // are those of the extreme raw values.
  const float ka = fmaxf(fabsf(mx - mu), fabsf(mn - mu));
  int a = 0;
  if (qa > 0.f && ka > 0.f) {
    int eq, ek;
    const float mq = frexpf(qa, &eq);
    const float mk = frexpf(ka, &ek);
    const int k = ek - eq - (mk < mq ? 1 : 0);   // floor(log2(ka / qa))
    a = (k + 1) >= 0 ? (k + 1) / 2 : -((-(k + 1) + 1) / 2);  // floor((k+1)/2)
  }
  if (shift_in) a = shift_in[static_cast<int64_t>(bh) * D + c];
  mu_out[static_cast<int64_t>(bh) * D + c] = mu;
  shift_out[static_cast<int64_t>(bh) * D + c] = static_cast<int8_t>(a);
}

// Input row of position j of the quantized operand, or -1 (zero).  Without a
// frame cache (FS == 0) position j is input row j.  With one, position j is
// cache slot j: frame f = j / FS holds tokens f*F .. f*F + F - 1 at its first
// F slots (the rest are padding); the input holds tokens from tok0 on, and
// n_valid of its rows are valid.
__device__ __forceinline__ int slot_row(int j, int F, int FS, int tok0, int n_valid) {
  if (FS == 0) return j < n_valid ? j : -1;
  const int f = j / FS, t = j - f * FS;
  if (t >= F) return -1;
  const int r = f * F + t - tok0;
  return (r >= 0 && r < n_valid) ? r : -1;
}

// ---------------------------------------------------------------- INT8 blocks
// One workgroup per block of ROWS positions of one (b, h) -- block blk0 +
// blockIdx.x; positions map to input rows through slot_row (n_in >= 0
// overrides the count of valid input rows).  Each thread holds 8 channels of
// ROWS*D/2048 rows in registers between the amax and the encode.
template <typename T, int D, int ROWS, bool IS_K>
__global__ __launch_bounds__(256) void quant_i8_kernel(
    const T* __restrict__ x, int64_t sb, int64_t sh, int64_t sn, int H, int n_all,
    int n_pad, BatchInfo bi, const float* __restrict__ mu, const int8_t* __restrict__ shift,
    int8_t* __restrict__ codes, float* __restrict__ scale, int F, int FS, int tok0, int n_in, int blk0) {
  constexpr int G = D / 8;
  constexpr int RPP = 256 / G;       // rows per pass
  constexpr int PASSES = ROWS / RPP;
  static_assert(ROWS % RPP == 0, "block shape");
  const int b = blockIdx.z, h = blockIdx.y;
  if (blk0 < 0) {  // per-batch frame appends: batch b's new frames start at frame bi.frame0[b]
    tok0 = bi.frame0[b] * F;
    blk0 = bi.frame0[b] * (FS / ROWS);
  }
  const int blk = blk0 + blockIdx.x;
  const int bh = b * H + h;
  const int g = threadIdx.x % G, r0 = threadIdx.x / G;
  const int n_valid = n_in >= 0 ? n_in : (IS_K ? bi.kv_len[b] : n_all);
  float sh_mul[8], m8[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int a = shift[static_cast<int64_t>(bh) * D + 8 * g + c];
    sh_mul[c] = ldexpf(1.0f, IS_K ? -a : a);   // exact power of two
    m8[c] = IS_K ? mu[static_cast<int64_t>(bh) * D + 8 * g + c] : 0.f;
  }
  float v[PASSES][8];
  float amax = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int j = blk * ROWS + p * RPP + r0;
    const int row = slot_row(j, F, FS, tok0, n_valid);
    if (row >= 0) {
      const uint4 raw = *reinterpret_cast<const uint4*>(x + b * sb + h * sh + row * sn + 8 * g);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float f = to_f32(T{static_cast<uint16_t>((w[c / 2] >> (16 * (c % 2))) & 0xFFFFu)});
        if (IS_K) f = f - m8[c];
        f = f * sh_mul[c];
        v[p][c] = f;
        amax = fmaxf(amax, fabsf(f));
      }
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) v[p][c] = 0.f;
    }
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float delta = amax > 0.f ? amax / 127.0f : 0.f;
  const float inv = amax > 0.f ? 127.0f / amax : 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int j = blk * ROWS + p * RPP + r0;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float q = rintf(v[p][c] * inv);
      q = fminf(fmaxf(q, -127.f), 127.f);
      const uint32_t byte = static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu;
      if (c < 4) lo |= byte << (8 * c);
      else hi |= byte << (8 * (c - 4));
    }
    *reinterpret_cast<uint2*>(codes + (static_cast<int64_t>(bh) * n_pad + j) * D + 8 * g) =
        make_uint2(lo, hi);
  }
  if (threadIdx.x == 0) scale[static_cast<int64_t>(bh) * (n_pad / ROWS) + blk] = delta;
}

// ---------------------------------------------------------------- V layout
// One workgroup per 64-key chunk of one (b, h); 2*D threads.  Writes the chunk
// channel-major ([D][64]) so that each lane of the P.V matrix-core operand
// reads its keys contiguously.  FP8 mode: one E8M0 scale per (32-key block,
// channel) -- the smallest power of two 2^e >= 2^-127 with amax * 2^-e <= 448 -- and
// e4m3fn codes of v * 2^-e; the scales of a chunk are stored as 64 lanes x 4
// bytes (lane 32*k + r holds channels r, r+32, r+64, r+96 of key block k).
//
// VM: PV16, PVFP8, or PVAUTO -- each (b,h) in FP8 when its channel-balance
// exponents (shift) are all 0, else in 16 bits; every head then has a 16-bit
// sized slot, an FP8 head's codes filling its first half.
template <typename T, int D, int VM>
__global__ __launch_bounds__(2 * D) void prep_v_kernel(
    const T* __restrict__ x, int64_t sb, int64_t sh, int64_t sn, int H, int n_pad,
    BatchInfo bi, void* __restrict__ vt, uint8_t* __restrict__ e8m0, const int8_t* __restrict__ shift, int F,
    int FS, int tok0, int n_in, int ch0) {
  __shared__ uint16_t tile[64][D + 2];
  const int b = blockIdx.z, h = blockIdx.y;
  if (ch0 < 0) {  // per-batch frame appends (as in quant_i8_kernel)
    tok0 = bi.frame0[b] * F;
    ch0 = bi.frame0[b] * (FS / 64);
  }
  const int ch = ch0 + blockIdx.x;
  const int bh = b * H + h;
  const int n_valid = n_in >= 0 ? n_in : bi.kv_len[b];
  constexpr int GR = D / 8;  // 16-byte granules per key row
  for (int gi = threadIdx.x; gi < 64 * GR; gi += 2 * D) {
    const int r = gi / GR, g = gi % GR;
    const int row = slot_row(ch * 64 + r, F, FS, tok0, n_valid);
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (row >= 0) raw = *reinterpret_cast<const uint4*>(x + b * sb + h * sh + row * sn + 8 * g);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) tile[r][8 * g + c] = static_cast<uint16_t>((w[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
  }
  __syncthreads();
  bool fp8 = VM == PVFP8;
  if constexpr (VM == PVAUTO) {
    bool moved = false;
    if (threadIdx.x < D) moved = shift[static_cast<int64_t>(bh) * D + threadIdx.x] != 0;
    fp8 = !__syncthreads_or(moved);
  }
  const int c = threadIdx.x >> 1, kh = threadIdx.x & 1;
  const int64_t head_bytes = static_cast<int64_t>(n_pad) * D * (VM == PVFP8 ? 1 : 2);
  uint8_t* const vhead = static_cast<uint8_t*>(vt) + static_cast<int64_t>(bh) * head_bytes;
  const int64_t chunk_base = static_cast<int64_t>(ch) * D * 64;  // elements into the head
  if (!fp8) {
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      w[k] = static_cast<uint32_t>(tile[32 * kh + 2 * k][c]) |
             (static_cast<uint32_t>(tile[32 * kh + 2 * k + 1][c]) << 16);
    uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(vhead) + chunk_base + c * 64 + 32 * kh);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
  } else {
    float f[32];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      f[k] = to_f32(T{tile[32 * kh + k][c]});
      amax = fmaxf(amax, fabsf(f[k]));
    }
    int e = 0;
    if (amax > 0.f) {
      int k2;
      const float m = frexpf(amax, &k2);
      // floored at the smallest E8M0 scale 2^-127 (byte 0): a block below
      // 448 * 2^-127 keeps it, and its values round to e4m3 at that scale
      e = max((m <= 0.875f) ? k2 - 9 : k2 - 8, -127);
    }
    const float sc = ldexpf(1.0f, -e);
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      w[k] = pack_e4m3x4(f[4 * k] * sc, f[4 * k + 1] * sc, f[4 * k + 2] * sc, f[4 * k + 3] * sc);
    uint4* dst = reinterpret_cast<uint4*>(vhead + chunk_base + c * 64 + 32 * kh);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    // E8M0 layout per chunk: [lane = 32*kh + c%32][byte = c/32], four bytes per
    // lane, so each lane of the P.V MFMA loads its scales as one dword.
    uint8_t* eb = e8m0 + (static_cast<int64_t>(bh) * (n_pad / 64) + ch) * 256 + (32 * kh + c % 32) * 4;
    eb[c / 32] = static_cast<uint8_t>(e + 127);
    if (D == 64) eb[c / 32 + 2] = 127;  // unused byte positions hold the scale 1
  }
}

// ---------------------------------------------------------------- conversions
template <int KIND>
__global__ void convert_kernel(const float* __restrict__ in, void* __restrict__ out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t k = 4 * i;
  if (k >= n) return;
  float f[4];
  for (int t = 0; t < 4; ++t) f[t] = (k + t < n) ? in[k + t] : 0.f;
  if (KIND == 3) {  // 2^x as the softmax evaluates it (the hardware exponential)
    for (int t = 0; t < 4 && k + t < n; ++t) static_cast<float*>(out)[k + t] = __builtin_amdgcn_exp2f(f[t]);
  } else if (KIND == 0) {
    const uint32_t w = pack_e4m3x4(f[0], f[1], f[2], f[3]);
    for (int t = 0; t < 4 && k + t < n; ++t) static_cast<uint8_t*>(out)[k + t] = (w >> (8 * t)) & 0xFF;
  } else {
    const uint32_t w0 = KIND == 1 ? pack_bf16x2(f[0], f[1]) : pack_f16x2(f[0], f[1]);
    const uint32_t w1 = KIND == 1 ? pack_bf16x2(f[2], f[3]) : pack_f16x2(f[2], f[3]);
    const uint16_t hv[4] = {static_cast<uint16_t>(w0 & 0xFFFF), static_cast<uint16_t>(w0 >> 16),
                            static_cast<uint16_t>(w1 & 0xFFFF), static_cast<uint16_t>(w1 >> 16)};
    for (int t = 0; t < 4 && k + t < n; ++t) static_cast<uint16_t*>(out)[k + t] = hv[t];
  }
}

// ---------------------------------------------------------------- launchers
template <typename T, int D>
static hipError_t quantize_impl(const QuantLaunch& L, hipStream_t st) {
  const dim3 blk(256);
  constexpr int CPB = 256 / (D / 8);
  const int nck = (L.Nkv + KMEAN_CHUNK - 1) / KMEAN_CHUNK;
  const int ncq = (L.Nq + KMEAN_CHUNK - 1) / KMEAN_CHUNK;
  const int F = L.frame_len, FS = L.frame_stride;
  if (!L.frames_only) {
    hipLaunchKernelGGL((stats_partial_kernel<T, D, true>), dim3((nck + CPB - 1) / CPB, L.H, L.B), blk, 0, st,
                       static_cast<const T*>(L.k), L.ks[0], L.ks[1], L.ks[2], L.H, nck, L.bi, L.Nkv,
                       L.stat_ksum, L.stat_kmax, L.stat_kmin);
    hipLaunchKernelGGL((stats_partial_kernel<T, D, false>), dim3((ncq + CPB - 1) / CPB, L.H, L.B), blk, 0, st,
                       static_cast<const T*>(L.q), L.qs[0], L.qs[1], L.qs[2], L.H, ncq, L.bi, L.Nq,
                       nullptr, L.stat_qamax, nullptr);
    hipLaunchKernelGGL(stats_final_kernel<D>, dim3(L.B * L.H), dim3(SF_THREADS), 0, st, L.H, nck, ncq, L.bi,
                       L.stat_ksum, L.stat_kmax, L.stat_kmin, L.stat_qamax, L.k_mean_in, L.chan_shift_in,
                       L.bufs.k_mean, L.bufs.chan_shift);
  }
  if (L.q)
    hipLaunchKernelGGL((quant_i8_kernel<T, D, BQ, false>), dim3(L.Nq_pad / BQ, L.H, L.B), blk, 0, st,
                       static_cast<const T*>(L.q), L.qs[0], L.qs[1], L.qs[2], L.H, L.Nq, L.Nq_pad, L.bi,
                       L.bufs.k_mean, L.bufs.chan_shift, L.bufs.q_codes, L.bufs.q_scale, 0, 0, 0, -1, 0);
  // K and V: every position (blocks of the whole operand), or the slots of the
  // appended frames only (their tokens are the input's rows 0 ..); a negative
  // first chunk: each batch's own first frame, from bi.frame0
  const int c0 = L.frames_only ? (L.frame0 < 0 ? -1 : L.frame0 * FS / 64) : 0;
  const int nc = L.frames_only ? L.nframes * FS / 64 : L.Nkv_pad / 64;
  const int tok0 = L.frames_only && L.frame0 >= 0 ? L.frame0 * F : 0;
  const int n_in = L.frames_only ? L.nframes * F : -1;
  hipLaunchKernelGGL((quant_i8_kernel<T, D, BK, true>), dim3(nc, L.H, L.B), blk, 0, st,
                     static_cast<const T*>(L.k), L.ks[0], L.ks[1], L.ks[2], L.H, L.Nkv, L.Nkv_pad, L.bi,
                     L.bufs.k_mean, L.bufs.chan_shift, L.bufs.k_codes, L.bufs.k_scale, F, FS, tok0, n_in, c0);
  if (L.pv_mode == PVFP8)
    hipLaunchKernelGGL((prep_v_kernel<T, D, PVFP8>), dim3(nc, L.H, L.B), dim3(2 * D), 0, st,
                       static_cast<const T*>(L.v), L.vs[0], L.vs[1], L.vs[2], L.H, L.Nkv_pad, L.bi,
                       L.bufs.v_t, L.bufs.v_e8m0, L.bufs.chan_shift, F, FS, tok0, n_in, c0);
  else if (L.pv_mode == PVAUTO)
    hipLaunchKernelGGL((prep_v_kernel<T, D, PVAUTO>), dim3(nc, L.H, L.B), dim3(2 * D), 0, st,
                       static_cast<const T*>(L.v), L.vs[0], L.vs[1], L.vs[2], L.H, L.Nkv_pad, L.bi,
                       L.bufs.v_t, L.bufs.v_e8m0, L.bufs.chan_shift, F, FS, tok0, n_in, c0);
  else
    hipLaunchKernelGGL((prep_v_kernel<T, D, PV16>), dim3(nc, L.H, L.B), dim3(2 * D), 0, st,
                       static_cast<const T*>(L.v), L.vs[0], L.vs[1], L.vs[2], L.H, L.Nkv_pad, L.bi,
                       L.bufs.v_t, L.bufs.v_e8m0, L.bufs.chan_shift, F, FS, tok0, n_in, c0);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantLaunch& L, hipStream_t st) {
  if (L.dtype == DT_BF16)
    return L.d == 128 ? quantize_impl<bf16_t, 128>(L, st) : quantize_impl<bf16_t, 64>(L, st);
  return L.d == 128 ? quantize_impl<f16_t, 128>(L, st) : quantize_impl<f16_t, 64>(L, st);
}

hipError_t launch_convert(int kind, const float* in, void* out, int64_t n, hipStream_t st) {
  const int64_t threads = (n + 3) / 4;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (kind == 0) hipLaunchKernelGGL(convert_kernel<0>, grid, dim3(256), 0, st, in, out, n);
  else if (kind == 1) hipLaunchKernelGGL(convert_kernel<1>, grid, dim3(256), 0, st, in, out, n);
  else if (kind == 2) hipLaunchKernelGGL(convert_kernel<2>, grid, dim3(256), 0, st, in, out, n);
  else hipLaunchKernelGGL(convert_kernel<3>, grid, dim3(256), 0, st, in, out, n);
  return hipGetLastError();
}

}  // namespace sage
