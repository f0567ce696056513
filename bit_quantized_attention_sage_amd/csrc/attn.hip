// Fused quantized attention for gfx950: INT8 S^T = K Q^T on matrix cores with
// int32 accumulation, fp32 dequantization and online softmax, and O^T = V^T P^T
// on 16-bit or scaled-FP8 matrix cores.
//
// Why quantized: video-generation attention is compute-bound and low-precision
// matrix units sit idle under exact attention (podcast notes "Faster! Even
// faster! ...", section "02:48 There were clearly faster compute units on the
// hardware").  Why a frame-block-causal mask and a KV cache: streaming
// generation attends frame by frame to cached history (Vidu S1 blog, sections
// "模型架构", "训练方法" and "Infra").  The scheme itself is this library's own
// (the pages give none).
//
// Work decomposition.  Each wave owns 32 query rows.  Keys are streamed in
// 64-key chunks (one K scale each) through LDS; per chunk a wave runs 8 i8
// MFMAs 32x32x32 for S, the softmax on its 32x64 scores, and the P.V MFMAs.
// Two shapes of workgroup, for one (b, h) and optionally one of several KV
// splits:
//  * ping-pong (contiguous keys, frame cache): 8 waves = two 128-row query
//    blocks (two Q scales) sharing every staged K/V chunk.  Waves w and w+4
//    sit on the same SIMD; group 0 (waves 0-3) runs one phase ahead of group 1,
//    and each chunk step is two phases split by a barrier: the MFMAs, then the
//    softmax.  So on every SIMD one wave's matrix work meets the other's
//    vector work, which the hardware overlaps, instead of each wave
//    interleaving both (measured on gfx950: one wave issues plain FP32 VALU
//    ops every ~5 cycles, two every ~2.5; exp and the FP8 conversion take
//    ~8.4 cycles per wave instruction either way).
//  * 4 waves = one 128-row block (block-sparse tiles, whose kept chunks
//    differ from block to block); each wave interleaves its own MFMAs and
//    softmax.
//
// Register layouts (32x32 MFMA, lane l, h2 = l / 32, r32 = l % 32):
//  * S^T = K Q^T: the B operand is Q^T, so lane l holds query r32 and channel
//    bytes [32*ks + 16*h2, +16); the A operand row r (lane r32) loads key
//    32*u + 16*((r>>2)&1) + 4*(r>>3) + (r&3) of subtile u.  With that row
//    order, accumulator register i of lane l (row 8*(i/4) + 4*h2 + i%4) holds
//    key 32*u + 16*h2 + i: lane half h2 owns keys [16*h2, +16) and
//    [32 + 16*h2, +16) of the chunk for its query.
//  * The scaled FP8 MFMA 32x32x64 pairs byte e of lane half h2 with K index
//    16*h2 + e (e < 16) or 32 + 16*h2 + (e - 16), and takes the E8M0 scale of
//    K block b (indices [32b, 32b+32)) for row r from lane r + 32*b.  So P^T
//    is already in B-operand form for O^T = V^T P^T with K index == key
//    offset in the chunk, each E8M0 block is 32 consecutive keys, and V
//    stored per chunk channel-major makes the A operand two contiguous
//    16-byte reads.  The 16-bit P.V MFMAs (K = 16) take keys
//    32*(mu/2) + 16*h2 + 8*(mu%2) + [0, 8) in lane half h2 for step mu.
//  * O^T accumulator: lane l holds query r32 and channels
//    32*cb + 8*(i/4) + 4*h2 + i%4, so per-row factors (alpha, 1/l) are per lane.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace sage {

// Masked score: the bits of float -infinity.  As an int it lies far below
// every biased score (so it never wins the row maximum); as the float F it
// gives x = -inf and p = exp2(x) = 0 with no select.
constexpr int MASKED = static_cast<int>(0xFF800000u);

// Score bias.  The S MFMAs start their integer accumulation from the inline
// constant 1/(2 pi), whose float32 bits are SBIAS, so they return SBIAS + S.
// For |S| < 2292099 (|S| <= 127^2 d here) those bits are exactly the float32
// F0 + S 2^-26 (F0 = 1/(2 pi) rounded to float32), so the softmax reads the
// score as a float without a conversion and forms S c - mref as
// fma(F, c 2^26, fma(-F0, c 2^26, -mref)).
constexpr int SBIAS = 0x3E22F983;

// a_row_key and k_swz (common.h) give the A operand's row order and the
// chunk's LDS swizzle.

// First k-step of an S chain: A B + SBIAS, the bias as the MFMA's inline
// accumulator constant.  (Written out because the compiler, seeing the same
// constant start two chains, keeps it in sixteen registers and copies it
// into each accumulator every chunk instead.)  The compiler cannot see that
// this is an 8-pass matrix op, so it inserts none of the wait states its
// result needs: the block ends with 16 of them itself (an 8-pass XDL result
// needs 11 before any dependent read), which also keeps later writes to its
// source registers clear of its operand reads.
__device__ __forceinline__ v16i mfma_i8_biased(v4i a, v4i b) {
  v16i d;
  asm("v_mfma_i32_32x32x32_i8 %0, %1, %2, 0.15915494\n\ts_nop 7\n\ts_nop 7" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}

// S^T + SBIAS for one 64-key chunk held in LDS (row-major [64][D], swizzled):
// s0 = keys 16*h2 + [0,16), s1 = keys 32 + 16*h2 + [0,16), per the layout above.
template <int D>
__device__ __forceinline__ void qk_chunk(const int8_t* __restrict__ klds, const v4i* qv, int lane,
                                         v16i& s0, v16i& s1) {
  const int h2 = lane >> 5, r32 = lane & 31;
  const int key0 = a_row_key(r32, 0), key1 = a_row_key(r32, 1);
  const int sw0 = k_swz<D>(key0), sw1 = k_swz<D>(key1);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const int g = 2 * ks + h2;
    const v4i a0 = *reinterpret_cast<const v4i*>(klds + key0 * D + ((g ^ sw0) << 4));
    const v4i a1 = *reinterpret_cast<const v4i*>(klds + key1 * D + ((g ^ sw1) << 4));
    if (ks == 0) {
      s0 = mfma_i8_biased(a0, qv[0]);
      s1 = mfma_i8_biased(a1, qv[0]);
    } else {
      s0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qv[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qv[ks], s1, 0, 0, 0);
    }
  }
}

// Copy one 64-key K chunk (row-major, D bytes per key) into LDS, swizzled.
template <int D, int NT>
__device__ __forceinline__ void load_k_chunk(int8_t* __restrict__ klds, const int8_t* __restrict__ src,
                                             int tid) {
  constexpr int G = D / 16;
  constexpr int NG = 64 * G;
#pragma unroll
  for (int gi = tid; gi < NG; gi += NT) {
    const int key = gi / G, g = gi % G;
    const uint4 v = *reinterpret_cast<const uint4*>(src + gi * 16);
    *reinterpret_cast<uint4*>(klds + key * D + ((g ^ k_swz<D>(key)) << 4)) = v;
  }
}

// Load the 32 query rows' Q codes of a wave as B operands (16 bytes per k-step).
template <int D>
__device__ __forceinline__ void load_q(v4i* qv, const int8_t* __restrict__ qrow, int h2) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qv[ks] = *reinterpret_cast<const v4i*>(qrow + 32 * ks + 16 * h2);
}

struct AttnArgs {
  const int8_t* qc;
  const float* qscale;
  const int8_t* kc;
  const float* kscale;
  const void* vt;
  const uint8_t* ve;
  void* o;
  int64_t os_b, os_h, os_n;
  float* part_o;   // [splits][B*H][Nq_pad][D] fp32, when splits > 1
  float* part_ml;  // [splits][B*H][Nq_pad][2]  (m, l)
  int B, H, Nq, Nq_pad, Nkv_pad, nqt, splits, total;
  float sigma;
  int frame_len;
  int frame_stride, sink_frames, window_frames;  // frame cache and window (0: contiguous keys)
  uint32_t cpf_magic;                            // ceil(2^32 / (frame_stride / 64)), 0 if that is 1
  const uint8_t* block_mask;                     // [B*H][nqt][mask_nkc], nonzero = tile kept
  int mask_nkc;
  BatchInfo bi;
  int order[MAXB_ARGS];
};

// LDS layout of a staged chunk.  K: [64 keys][D] bytes with the granule
// swizzle above.  V^T: [D channels][64 keys], 64 B (FP8) or 128 B (16-bit)
// per channel row, granule g of row c stored at slot g ^ swz(c); a P.V
// operand read takes the same granule of consecutive channel rows.
template <int PV>
struct VRow {
  static constexpr int BYTES = (PV == PVFP8) ? 64 : 128;  // bytes per channel row
  static constexpr int GR = BYTES / 16;                    // granules per row
  // granule swizzle: the 16 channel rows c = 16t..16t+15 one read group
  // touches (and any 8 consecutive ones) fall on distinct bank slots
  static __device__ __forceinline__ int swz(int c) {
    const int b0 = c & 1, b1 = (c >> 1) & 1, b2 = (c >> 2) & 1, b3 = (c >> 3) & 1;
    if constexpr (PV == PVFP8) return (b1 ^ b3) | (b2 << 1);
    else return b1 | (b2 << 1) | ((b0 ^ b3) << 2);
  }
  static __device__ __forceinline__ int addr(int c, int g) { return c * BYTES + ((g ^ swz(c)) << 4); }
};

// P operand of the P.V MFMAs for one chunk: 32 e4m3 bytes (FP8 mode) or 16
// packed 16-bit pairs, in the key order described at the top of the file.
template <int PV>
struct PTile;
template <>
struct PTile<PVFP8> {
  v8i b;
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(b)); }
};
template <>
struct PTile<PV16> {
  uint32_t w[16];
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int i = 0; i < 16; i += 4) asm volatile("" : "+v"(w[i]), "+v"(w[i + 1]), "+v"(w[i + 2]), "+v"(w[i + 3]));
  }
};

// Per-wave online-softmax state and the math of one chunk.
// Constant A operand of the row-sum MFMAs (16x16, K = 128 e4m3 or 32 16-bit
// values).  A 16x16 MFMA pairs lane m + 16g of A with lane n + 16g of B (same
// K indices) and returns D[4*(l/16) + j][l%16] to lane l.  The P tile, read
// as such a B operand, has query row n + 16*(g&1) in lane group g.  Row m of
// A is all ones where m%4 == 0 and (m/4)&1 == g&1, zero elsewhere, so D[4k][n]
// sums row n + 16*(k&1) over both lane halves: register 0 of lane l ends up
// with the P sum of its own query row l%32.
__device__ __forceinline__ int lsum_select(int lane, int one4) {
  const int m = lane & 15, g = lane >> 4;
  return ((m & 3) == 0 && ((m >> 2) & 1) == (g & 1)) ? one4 : 0;
}

template <int D, int PV, int DT>
struct WaveState {
  static constexpr int NCB = D / 32;
  static constexpr int SHIFT = (PV == PVFP8) ? PSHIFT_FP8 : PSHIFT_16;
  v16f o[NCB];
  v4f ls;  // row sums of P as the P.V MFMAs see it (register 0; see lsum_select)
  float m;

  // Masking of a boundary chunk: keys at or beyond `lim` (counted from this
  // lane half's first key, 16*h2) get the MASKED score.
  __device__ __forceinline__ void mask(v16i& s0, v16i& s1, int lim) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = (i < lim) ? s0[i] : MASKED;
      s1[i] = (32 + i < lim) ? s1[i] : MASKED;
    }
  }

  // Softmax step of one chunk on its integer scores: the row maximum (the
  // two lane halves hold the same query), the lazy running-max update (the
  // row adopts the chunk maximum only when it exceeds m by more than TAU),
  // p = 2^(S c - (m - s)) and P rounded to the P.V operand type.  Returns
  // alpha (1 for rows that kept m); the caller rescales O and the row sums
  // by it when any row of the wave moved.  The row sums of the rounded P are
  // taken on the matrix cores in pv().
  // `has`: this row has a visible key in the chunk (rows without one keep m).
  __device__ __forceinline__ float softmax(const v16i& s0, const v16i& s1, float c, bool has, PTile<PV>& P) {
    // two v_max3 chains of 8 over the lane's 32 scores
    int ma = max3_i32(s0[0], s0[1], s0[2]), mb = max3_i32(s1[0], s1[1], s1[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) {
      ma = max3_i32(ma, s0[i], s0[i + 1]);
      mb = max3_i32(mb, s1[i], s1[i + 1]);
    }
    int mx = max3_i32(max(ma, s0[15]), mb, s1[15]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
      mx = max(static_cast<int>(sw[0]), static_cast<int>(sw[1]));
    }
    const float tm = static_cast<float>(mx - SBIAS) * c;
    const bool upd = has && (tm > m + TAU);
    const float alpha = upd ? __builtin_amdgcn_exp2f(m - tm) : 1.0f;
    m = upd ? tm : m;
    const float nmref = -(m - static_cast<float>(SHIFT));
    // c 2^26, exact; a zero scale (all-zero Q or K block: every score 0)
    // becomes the smallest normal float so that MASKED keys still give -inf
    const float c2 = fmaxf(c, 1.17549435e-38f) * 67108864.0f;
    const float kx = __builtin_fmaf(-__builtin_bit_cast(float, SBIAS), c2, nmref);
    float p0[16], p1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // (copy the element out first: a bit cast of a vector subscript reads element 0)
      const int b0 = s0[i], b1 = s1[i];
      p0[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_bit_cast(float, b0), c2, kx));
      p1[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_bit_cast(float, b1), c2, kx));
    }
    if constexpr (PV == PVFP8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        P.b[k] = static_cast<int>(pack_e4m3x4_into(p0[4 * k], p0[4 * k + 1], p0[4 * k + 2], p0[4 * k + 3]));
        P.b[4 + k] = static_cast<int>(pack_e4m3x4_into(p1[4 * k], p1[4 * k + 1], p1[4 * k + 2], p1[4 * k + 3]));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        P.w[k] = Pack16<DT>::pack(p0[2 * k], p0[2 * k + 1]);
        P.w[8 + k] = Pack16<DT>::pack(p1[2 * k], p1[2 * k + 1]);
      }
    }
    return alpha;
  }

  __device__ __forceinline__ void rescale(float alpha) {
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
      ls[0] *= alpha;
    }
  }

  // O += P V over the chunk, and the row sums of P; e8: this lane's four E8M0
  // bytes (FP8 mode; byte cb scales channel block cb of the lane's 32-key
  // block).
  __device__ __forceinline__ void pv(const PTile<PV>& P, const uint8_t* vlds, int e8, int lane) {
    const int h2 = lane >> 5, r32 = lane & 31;
    if constexpr (PV == PVFP8) {
      // channel block cb takes byte cb of the lane's scale register (op_sel)
      auto one = [&](auto cbc) {
        constexpr int cb = decltype(cbc)::value;
        const int c = 32 * cb + r32;
        const v4i lo = *reinterpret_cast<const v4i*>(vlds + VRow<PV>::addr(c, h2));
        const v4i hi = *reinterpret_cast<const v4i*>(vlds + VRow<PV>::addr(c, 2 + h2));
        const v8i va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, P.b, o[cb], 0, 0, cb, e8, 0, 127);
      };
      one(std::integral_constant<int, 0>{});
      one(std::integral_constant<int, 1>{});
      if constexpr (NCB > 2) {
        one(std::integral_constant<int, 2>{});
        one(std::integral_constant<int, 3>{});
      }
      const int s1 = lsum_select(lane, 0x38383838);  // e4m3 1.0 = 0x38
      const v8i sel = {s1, s1, s1, s1, s1, s1, s1, s1};
      ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, P.b, ls, 0, 0, 0, 127, 0, 127);
    } else {
      const int s1 = lsum_select(lane, DT == DT_BF16 ? 0x3F803F80 : 0x3C003C00);  // 1.0 pairs
      const v4i sel = {s1, s1, s1, s1};
#pragma unroll
      for (int mu = 0; mu < 4; ++mu) {
        const v4i pbv = {static_cast<int>(P.w[4 * mu]), static_cast<int>(P.w[4 * mu + 1]),
                         static_cast<int>(P.w[4 * mu + 2]), static_cast<int>(P.w[4 * mu + 3])};
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const v4i va = *reinterpret_cast<const v4i*>(
              vlds + VRow<PV>::addr(32 * cb + r32, 4 * (mu >> 1) + 2 * h2 + (mu & 1)));
          if (DT == DT_BF16)
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, va),
                                                            __builtin_bit_cast(v8bf, pbv), o[cb], 0, 0, 0);
          else
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, va),
                                                           __builtin_bit_cast(v8h, pbv), o[cb], 0, 0, 0);
        }
        if (DT == DT_BF16)
          ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, sel),
                                                       __builtin_bit_cast(v8bf, pbv), ls, 0, 0, 0);
        else
          ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, sel),
                                                      __builtin_bit_cast(v8h, pbv), ls, 0, 0, 0);
      }
    }
  }

};

// Key layouts / chunk lists of the fused kernel.
enum { KV_DENSE = 0,    // contiguous keys, every chunk up to the tile's range end
       KV_CACHE = 1,    // frame cache: the sink frames' chunks, then the window's
       KV_SPARSE = 2 }; // contiguous keys, only the chunks the block mask keeps
constexpr int MAX_LIST = 4096;  // kept-chunk list of a tile (LDS, 2 bytes each)

template <int D, int PV, int DT, int MODE, bool PP>
__global__ __launch_bounds__(PP ? 512 : 256, PP ? 1 : 2) void attn_fwd_kernel(AttnArgs A) {
  constexpr bool CACHE = MODE == KV_CACHE, SPARSE = MODE == KV_SPARSE;
  static_assert(!(PP && SPARSE), "the two query blocks of a ping-pong tile share one chunk list");
  constexpr int NWAVE = PP ? 8 : 4;
  constexpr int NCB = D / 32;                    // 32-channel blocks of O
  constexpr int VBYTES = (PV == PVFP8) ? 1 : 2;  // bytes per V element
  constexpr int KB = 64 * D;                     // bytes of a K chunk
  constexpr int VBC = 64 * D * VBYTES;           // bytes of a V^T chunk
  constexpr int KI = KB / 4096;                  // 1 KB DMA instructions per wave, K
  constexpr int VI = VBC / 4096;                 // ... and V
  static_assert(KI >= 1 && KI <= 2 && VI >= 1 && VI <= 4, "staging shape");
  // Two buffers each, as separate objects so that the compiler can tell the
  // buffer being filled by DMA from the one being read.
  __shared__ __attribute__((aligned(16))) int8_t kL0[KB];
  __shared__ __attribute__((aligned(16))) int8_t kL1[KB];
  __shared__ __attribute__((aligned(16))) uint8_t vL0[VBC];
  __shared__ __attribute__((aligned(16))) uint8_t vL1[VBC];
  __shared__ uint16_t slist[SPARSE ? MAX_LIST : 1];  // kept chunks of the tile, ascending
  __shared__ int scnt[8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5;

  // ---- work item: (batch by decreasing kv_len, head, split, query tile)
  const int ntile = PP ? (A.nqt + 1) / 2 : A.nqt;             // tiles of NWAVE * 32 rows
  const int L = xcd_group_remap(blockIdx.x, A.total, ntile);  // groups: the tiles of one (b, h, split)
  const int per_b = A.H * A.splits * ntile;
  const int b = A.order[L / per_b];
  int rem = L % per_b;
  const int h = rem / (A.splits * ntile);
  rem %= A.splits * ntile;
  const int split = rem / ntile;
  const int qt = rem % ntile;
  const int bh = b * A.H + h;
  // this wave's group, its place in the group and its 128-row Q block (the
  // second block of the last tile may lie past Nq: its rows load the last
  // real block and store nothing)
  const int grp = PP ? (w >> 2) : 0, w4 = w & 3;
  const int qb = PP ? 2 * qt + grp : qt;
  const int qbl = min(qb, A.nqt - 1);

  const int kv_len = A.bi.kv_len[b];
  const int q_pos0 = A.bi.q_pos0[b];
  const int F = A.frame_len, FS = CACHE ? A.frame_stride : 0;

  // ---- this lane's query row and the tile's first and last real rows
  const int qi = qb * BQ + w4 * 32 + (lane & 31);
  const int qi_valid = min(qi, A.Nq - 1);
  const int row_first = (PP ? 2 * qt : qt) * BQ, row_last = min(row_first + NWAVE * 32, A.Nq) - 1;

  // ---- the key chunks this work item visits: list entry v is chunk v for
  // v < a0, else chunk b1 + (v - a0); the split takes entries [v_lo, v_hi).
  //  * contiguous keys: the batch's chunks [0, ceil(kv_len/64)), split on that
  //    grid, cut at the end of the tile's last row; a row sees the prefix
  //    [0, re) of the keys;
  //  * frame cache: the chunks of the sink frames, then those of the window
  //    frames through the last row's frame (up to its last token); a row sees
  //    the valid slots of the frames of its window.
  int re = 0, fq = 0, fq_lo = 0, fq_hi = 0, a0 = 0, b1 = 0, v_lo, v_hi, full_end = 0, n_full = 0;
  if constexpr (!CACHE) {
    re = F > 0 ? min(kv_len, ((q_pos0 + qi_valid) / F + 1) * F) : kv_len;
    const int first_end = F > 0 ? min(kv_len, ((q_pos0 + row_first) / F + 1) * F) : kv_len;
    const int last_end = F > 0 ? min(kv_len, ((q_pos0 + row_last) / F + 1) * F) : kv_len;
    const int nch = (kv_len + 63) / 64;
    v_lo = split * nch / A.splits;
    v_hi = min((split + 1) * nch / A.splits, (last_end + 63) / 64);
    full_end = first_end;  // chunks ending at or before it are visible in full to every row
    if constexpr (SPARSE) {
      // The tile's list: the chunks among [0, ceil(last_end/64)) that the
      // mask keeps, compacted in order into LDS by the whole workgroup
      // (ballot + per-wave counts); `below` counts those visible in full to
      // every row.  The split takes entries [v_lo, v_hi) of the list.
      const int nbase = (last_end + 63) / 64, nfull = full_end / 64;
      const uint8_t* mrow = A.block_mask + (static_cast<int64_t>(bh) * A.nqt + qt) * A.mask_nkc;
      int total = 0, below = 0;
      for (int c0 = 0; c0 < nbase; c0 += 256) {
        const int c = c0 + tid;
        const bool keep = c < nbase && mrow[c] != 0;
        const uint64_t bk = __ballot(keep), bf = __ballot(keep && c < nfull);
        if (lane == 0) {
          scnt[w] = __popcll(bk);
          scnt[4 + w] = __popcll(bf);
        }
        __syncthreads();
        int off = total;
        for (int i = 0; i < w; ++i) off += scnt[i];
        const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bk >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bk), 0));
        if (keep) slist[off + rank] = static_cast<uint16_t>(c);
        total += scnt[0] + scnt[1] + scnt[2] + scnt[3];
        below += scnt[4] + scnt[5] + scnt[6] + scnt[7];
        __syncthreads();
      }
      v_lo = split * total / A.splits;
      v_hi = (split + 1) * total / A.splits;
      n_full = below;
    }
  } else {
    const int cpf = FS / 64;
    fq = (q_pos0 + qi_valid) / F;
    fq_lo = (q_pos0 + row_first) / F;
    fq_hi = (q_pos0 + row_last) / F;
    const int end_chunk = (fq_hi * FS + min(F, kv_len - fq_hi * F) + 63) / 64;
    int nv = end_chunk;
    if (A.window_frames > 0) {
      a0 = min(min(A.sink_frames, fq_hi + 1) * cpf, end_chunk);
      b1 = min(max(A.sink_frames, fq_lo - A.window_frames) * cpf, end_chunk);
      b1 = max(b1, a0);
      nv = a0 + (end_chunk - b1);
    }
    v_lo = split * nv / A.splits;
    v_hi = (split + 1) * nv / A.splits;
  }
  const int J = max(0, v_hi - v_lo);  // chunks of this work item
  // list entries below this one are visible in full to every row of the tile
  // (contiguous keys: up to the first row's end; frame cache: no shortcut)
  const int v_full = CACHE ? 0 : SPARSE ? n_full : full_end / 64;
  // physical chunk of list entry v; contiguous keys: v itself (the loads
  // clamp it to the head's last chunk); frame cache and block mask: clamped
  // to the item's range first
  auto chunk_of = [&](int v) -> int {
    if constexpr (MODE == KV_DENSE) {
      return v;
    } else if constexpr (SPARSE) {
      if (v_hi <= v_lo) return 0;
      v = max(min(v, v_hi - 1), v_lo);
      return __builtin_amdgcn_readfirstlane(static_cast<int>(slist[v]));
    } else {
      v = max(min(v, v_hi - 1), 0);
      return v < a0 ? v : b1 + (v - a0);
    }
  };

  // Visibility of chunk ch: every row sees all 64 keys (wave-uniform), or
  // this row sees its first row_lim keys.
  // frame of cache chunk ch: ch / (FS/64) by a multiply-high with the
  // host's rounded-up reciprocal (exact for ch < 2^20, FS/64 < 2^11); with
  // one chunk per frame the reciprocal (2^32) does not fit and f = ch
  auto frame_of = [&](int ch) -> int {
    return FS == 64 ? ch : static_cast<int>(__umulhi(static_cast<uint32_t>(ch), A.cpf_magic));
  };
  auto chunk_full = [&](int ch) -> bool {
    if constexpr (!CACHE) return (ch + 1) * 64 <= full_end;
    const int f = frame_of(ch);
    const int t0 = (ch - f * (FS / 64)) * 64;
    const int vc = min(min(F - t0, kv_len - (f * F + t0)), 64);
    const bool all = f <= fq_lo && (A.window_frames == 0 || f < A.sink_frames || f >= fq_hi - A.window_frames);
    return vc >= 64 && all;
  };
  auto row_lim = [&](int ch) -> int {
    if constexpr (!CACHE) return re - ch * 64;
    const int f = frame_of(ch);
    const int t0 = (ch - f * (FS / 64)) * 64;
    const int vc = min(min(F - t0, kv_len - (f * F + t0)), 64);
    const bool vis = f <= fq && (A.window_frames == 0 || f < A.sink_frames || f >= fq - A.window_frames);
    return vis ? vc : 0;
  };

  v4i qv[D / 32];
  load_q<D>(qv, A.qc + (static_cast<int64_t>(bh) * A.Nq_pad + qbl * BQ + w4 * 32 + (lane & 31)) * D, h2);
  const float qsc = A.qscale[static_cast<int64_t>(bh) * A.nqt + qbl] * A.sigma;

  WaveState<D, PV, DT> st;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) st.o[cb] = v16f{0.f};
  st.ls = v4f{0.f, 0.f, 0.f, 0.f};
  // The running max starts at the most negative finite float, not -inf: a
  // row can meet chunks with no visible key before its first visible one (a
  // split or a window that begins with keys of frames the row does not see),
  // and with m = -inf the softmax's -inf scores would give -inf + inf = NaN.
  // This way they give p = 2^-inf = 0, and the first visible chunk still
  // moves m (its alpha = 0 scales an O and l that are still 0).
  st.m = -3.40282347e38f;

  const int nkc = A.Nkv_pad / 64;
  const int8_t* kbase = A.kc + static_cast<int64_t>(bh) * A.Nkv_pad * D;
  const uint8_t* vbase = static_cast<const uint8_t*>(A.vt) + static_cast<int64_t>(bh) * nkc * VBC;
  const uint8_t* ebase = A.ve + static_cast<int64_t>(bh) * nkc * 256;
  const float* ksc = A.kscale + static_cast<int64_t>(bh) * nkc;

  // Staging: raw buffer loads that write straight into LDS (no registers),
  // issued one step ahead, by the four waves of group 0 (ping-pong) or of the
  // workgroup.  Lane l of DMA instruction i of wave w fills LDS
  // granule (4i + w)*64 + l of the buffer; its global source is chosen so that
  // the buffer ends up in the swizzled layouts above.  Every chunk index is
  // clamped to the head's last padded chunk, so all reads stay inside the
  // head's slice; the prefetches that the clamp redirects are never consumed.
  // The K scale and this lane's four E8M0 bytes of a chunk are plain loads
  // into registers.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(kbase), 0, nkc * KB, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(vbase), 0, nkc * VBC, 0x00020000);
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(ebase), 0, PV == PVFP8 ? nkc * 256 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ksc), 0, nkc * 4, 0x00020000);
  int koff[KI], voff[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    constexpr int G = D / 16;
    const int sidx = (4 * i + w) * 64 + lane, key = sidx / G, gp = sidx % G;
    koff[i] = key * D + ((gp ^ k_swz<D>(key)) << 4);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    constexpr int GR = VRow<PV>::GR;
    const int sidx = (4 * i + w) * 64 + lane, c = sidx / GR, gp = sidx % GR;
    voff[i] = c * VRow<PV>::BYTES + ((gp ^ VRow<PV>::swz(c)) << 4);
  }
  const int last = nkc - 1;  // chunk indices are clamped: prefetches past the end go unused
  auto dma_k = [&](int8_t* dst, int ch) {
    if (PP && grp != 0) return;  // group 0 stages every chunk
    ch = min(ch, last);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int off = koff[i];  // an array element as the builtin's argument drops the host stub
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, dst + (4 * i + w) * 1024, 16, off, ch * KB, 0, 0);
    }
  };
  auto dma_v = [&](uint8_t* dst, int ch) {
    if (PP && grp != 0) return;
    ch = min(ch, last);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int off = voff[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, dst + (4 * i + w) * 1024, 16, off, ch * VBC, 0, 0);
    }
  };
  auto load_ks = [&](int ch) -> float {
    ch = min(ch, last);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 0, ch * 4, 0));
  };
  auto load_e = [&](int ch) -> int {
    ch = min(ch, last);
    return PV == PVFP8 ? __builtin_amdgcn_raw_buffer_load_b32(ers, lane * 4, ch * 256, 0) : 0;
  };
  auto dma_wait = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };  // vmcnt(0): this wave's DMA landed

  // Masking of a chunk whose scores are in (s0, s1): a wave-uniform branch,
  // taken only at boundaries (the last chunks of a row's range, frame padding,
  // window edges).  Returns whether this row has a visible key in the chunk.
  auto mask_chunk = [&](int v, v16i& s0, v16i& s1) -> bool {
    const int ch = chunk_of(v);
    if (chunk_full(ch)) return true;
    asm volatile("");  // keep this a real branch
    const int lim = row_lim(ch);
    st.mask(s0, s1, lim - 16 * h2);
    return lim > 0;
  };

  // Software pipeline within each wave over three chunks: step j (list entry
  // n = v_lo + j) enters with S(n+1) and P(n) in registers, K(n+2) in K buffer
  // j&1 and V(n) in V buffer j&1.  One straight-line region issues the DMA of
  // K(n+3) and V(n+1), the S MFMAs of entry n+2, the P.V MFMAs of entry n and
  // the softmax of entry n+1, so the matrix cores and the vector ALUs work
  // side by side; then the (rare) rescale by entry n+1's alpha, the (rare)
  // masking of S(n+2), the wait for this step's DMA and the barrier.
  // Ping-pong: the region is two phases instead, the MFMAs (at raised wave
  // priority, with the operand reads 8 ahead) and, after a barrier, the
  // softmax; group 1 runs the same steps one phase behind group 0 (one extra
  // barrier before its first step, group 0 one after its last), so the
  // buffers a step fills are the ones both groups finished reading in the
  // step before.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  v16i sa0{}, sa1{}, sb0{}, sb1{};
  PTile<PV> pa, pb;
  bool ha = true, hb = true;  // the rows' visibility flags of the chunks in sa, sb
  int n = v_lo;
  int e_cur = load_e(chunk_of(n));
  float ksn1 = load_ks(chunk_of(n + 1)), ksn2 = load_ks(chunk_of(n + 2));  // K scales of n+1, n+2
  // Prologue: K(n) and V(n) in buffers 0, K(n+1) in K buffer 1; then S(n+1),
  // P(n) and K(n+2) in K buffer 0.
  {
    const float ks0 = load_ks(chunk_of(n));
    dma_k(kL0, chunk_of(n));
    dma_v(vL0, chunk_of(n));
    dma_k(kL1, chunk_of(n + 1));
    dma_wait();
    __syncthreads();
    if (J >= 1) {
      qk_chunk<D>(kL0, qv, lane, sb0, sb1);
      if (J >= 2) qk_chunk<D>(kL1, qv, lane, sa0, sa1);
      __syncthreads();  // every wave has read K(n) from buffer 0
      dma_k(kL0, chunk_of(n + 2));
      hb = mask_chunk(n, sb0, sb1);
      if (J >= 2) ha = mask_chunk(n + 1, sa0, sa1);
      st.rescale(st.softmax(sb0, sb1, qsc * ks0, hb, pa));
      dma_wait();
      __syncthreads();
    }
  }
  // Every load issued so far has completed; saying so keeps the loop's own
  // prefetch loads from being waited on before the first MFMA.
  __builtin_amdgcn_s_waitcnt(0);
  int pre1 = 0, pre3 = 0;  // block mask: chunks of entries n+1 and n+3 for the next step
  if constexpr (SPARSE) {
    pre1 = chunk_of(n + 1);
    pre3 = chunk_of(n + 3);
  }

  // CHK false: S(n+1) and S(n+2) are visible in full to every row (no masking
  // check, every row has keys in entry n+1).
  auto step = [&](auto par, auto chk, v16i& cs0, v16i& cs1, bool& has_c, PTile<PV>& p_cur, v16i& ns0,
                  v16i& ns1, bool& has_n, PTile<PV>& p_nxt) {
    constexpr int P = decltype(par)::value;  // parity of the step
    constexpr bool CHK = decltype(chk)::value;
    int8_t* k_rd = P ? kL1 : kL0;            // K(n+2)
    int8_t* k_wr = P ? kL0 : kL1;            // receives K(n+3)
    uint8_t* v_rd = P ? vL1 : vL0;           // V(n)
    uint8_t* v_wr = P ? vL0 : vL1;           // receives V(n+1)
    constexpr int NQK = 2 * D / 32;                               // S MFMAs
    constexpr int NPV = (PV == PVFP8) ? NCB + 1 : 4 * NCB + 4;    // P.V and row-sum MFMAs
    constexpr int NRD = NQK + ((PV == PVFP8) ? 2 * NCB : 4 * NCB);  // LDS operand reads
    constexpr int VPER = (PV == PVFP8) ? 12 : 5;                  // softmax slice per MFMA
    const float c_mid = qsc * ksn1;
    const int ch1 = SPARSE ? pre1 : chunk_of(n + 1), ch3 = SPARSE ? pre3 : chunk_of(n + 3);
    __builtin_amdgcn_sched_barrier(0);
    dma_k(k_wr, ch3);
    dma_v(v_wr, ch1);
    const int e_nxt = load_e(ch1);
    const float ks3 = load_ks(ch3);
    float alpha;
    if constexpr (PP) {
      __builtin_amdgcn_s_setprio(1);
      qk_chunk<D>(k_rd, qv, lane, ns0, ns1);
      st.pv(p_cur, v_rd, e_cur, lane);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 + KI + VI, 0);  // the loads
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);            // the first operand reads
#pragma unroll
      for (int g = 0; g < NQK + NPV; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // one MFMA
        if (g + 8 < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
      }
      asm volatile("" : "+v"(ns0), "+v"(ns1));
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_s_barrier();  // end of the MFMA phase
      __builtin_amdgcn_sched_barrier(0);
      alpha = st.softmax(cs0, cs1, c_mid, CHK ? has_c : true, p_nxt);
      p_nxt.pin();
      __builtin_amdgcn_sched_barrier(0);
    } else {
      qk_chunk<D>(k_rd, qv, lane, ns0, ns1);
      st.pv(p_cur, v_rd, e_cur, lane);
      alpha = st.softmax(cs0, cs1, c_mid, CHK ? has_c : true, p_nxt);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 + KI + VI, 0);  // the loads
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);            // the first operand reads
#pragma unroll
      for (int g = 0; g < NQK + NPV; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPER, 0);  // a slice of the softmax
        if (g + 4 < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
      }
      // Pin the region's results here so that no earlier pass moves the S
      // MFMAs or the softmax out of it.
      asm volatile("" : "+v"(ns0), "+v"(ns1));
      p_nxt.pin();
      __builtin_amdgcn_sched_barrier(0);
    }
    st.rescale(alpha);  // rare: some row's running max moved (after P(n) V(n))
    if constexpr (CHK) {
      if (n + 2 >= v_full) has_n = mask_chunk(n + 2, ns0, ns1);  // rare: S(n+2) is a boundary chunk
    }
    if constexpr (SPARSE) {  // the next step's chunks, read from LDS ahead of the wait
      pre1 = chunk_of(n + 2);
      pre3 = chunk_of(n + 4);
    }
    dma_wait();
    __syncthreads();
    e_cur = e_nxt;
    ksn1 = ksn2;
    ksn2 = ks3;
    ++n;
  };
  using NoChk = std::integral_constant<bool, false>;
  using Chk = std::integral_constant<bool, true>;
  if (J >= 1) {
    int left = J - 1;  // pipelined steps
    if (PP && grp == 1 && left > 0) __builtin_amdgcn_s_barrier();  // one phase behind group 0
    if constexpr (!CACHE) {
      // the leading steps whose S(n+2) lies below v_full, in pairs
      for (int fast = min(J - 1, v_full - v_lo - 2); fast >= 2; fast -= 2) {
        step(P0{}, NoChk{}, sa0, sa1, ha, pa, sb0, sb1, hb, pb);
        step(P1{}, NoChk{}, sb0, sb1, hb, pb, sa0, sa1, ha, pa);
        left -= 2;
      }
    }
    while (left >= 2) {
      step(P0{}, Chk{}, sa0, sa1, ha, pa, sb0, sb1, hb, pb);
      step(P1{}, Chk{}, sb0, sb1, hb, pb, sa0, sa1, ha, pa);
      left -= 2;
    }
    if (PP && grp == 0 && J > 1) __builtin_amdgcn_s_barrier();  // as many barriers as group 1
    // the last entry's P.V (its V is in buffer (J-1)&1)
    if (left == 1) {
      step(P0{}, Chk{}, sa0, sa1, ha, pa, sb0, sb1, hb, pb);
      st.pv(pb, vL1, e_cur, lane);
    } else {
      st.pv(pa, vL0, e_cur, lane);
    }
  }
  v16f* o = st.o;
  const float m = st.m;

  // ---- epilogue: normalise, store
  const float ltot = st.ls[0];  // already summed over both lane halves
  if (qi >= A.Nq) return;
  if (A.splits == 1) {
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // a row with no visible key: 0
    uint16_t* orow = static_cast<uint16_t*>(A.o) + b * A.os_b + h * A.os_h + static_cast<int64_t>(qi) * A.os_n;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int chn = 32 * cb + 8 * g + 4 * h2;
        const uint32_t w0 = Pack16<DT>::pack(o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv);
        const uint32_t w1 = Pack16<DT>::pack(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + chn) = make_uint2(w0, w1);
      }
  } else {
    const int64_t prow = (static_cast<int64_t>(split) * A.B * A.H + bh) * A.Nq_pad + qi;
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    float* po = A.part_o + prow * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int chn = 32 * cb + 8 * g + 4 * h2;
        *reinterpret_cast<float4*>(po + chn) =
            make_float4(o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv, o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
      }
    if (h2 == 0) *reinterpret_cast<float2*>(A.part_ml + 2 * prow) = make_float2(m, ltot);
  }
}

// Merge split partials: O = sum_s w_s O_s / sum_s w_s with w_s = l_s 2^(m_s - M).
// One thread per (row, 4 channels).
template <int D, int DT>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs A) {
  constexpr int G = D / 4;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rows = static_cast<int64_t>(A.B) * A.H * A.Nq_pad;
  if (t >= rows * G) return;
  const int64_t row = t / G;
  const int g = t % G;
  const int bh = row / A.Nq_pad;
  const int qi = row % A.Nq_pad;
  if (qi >= A.Nq) return;
  const int b = bh / A.H, h = bh % A.H;
  float M = -__builtin_inff();
  for (int s = 0; s < A.splits; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(A.part_ml + 2 * ((static_cast<int64_t>(s) * A.B * A.H) * A.Nq_pad + row));
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s = 0; s < A.splits; ++s) {
    const int64_t prow = (static_cast<int64_t>(s) * A.B * A.H) * A.Nq_pad + row;
    const float2 ml = *reinterpret_cast<const float2*>(A.part_ml + 2 * prow);
    if (!(ml.y > 0.f)) continue;
    const float wgt = ml.y * __builtin_amdgcn_exp2f(ml.x - M);
    const float4 v = *reinterpret_cast<const float4*>(A.part_o + prow * D + 4 * g);
    acc[0] += wgt * v.x;
    acc[1] += wgt * v.y;
    acc[2] += wgt * v.z;
    acc[3] += wgt * v.w;
    wsum += wgt;
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;  // no split saw a key: 0
  uint16_t* orow = static_cast<uint16_t*>(A.o) + b * A.os_b + h * A.os_h + static_cast<int64_t>(qi) * A.os_n;
  *reinterpret_cast<uint2*>(orow + 4 * g) =
      make_uint2(Pack16<DT>::pack(acc[0] * inv, acc[1] * inv), Pack16<DT>::pack(acc[2] * inv, acc[3] * inv));
}

// Exact int32 scores of 32x64 tiles through qk_chunk (test support).
struct DebugTiles {
  int n;
  int t[128][3];
};

template <int D>
__global__ __launch_bounds__(64) void debug_scores_kernel(AttnArgs A, DebugTiles T, int32_t* out) {
  __shared__ __attribute__((aligned(16))) int8_t klds[64 * D];
  const int lane = threadIdx.x, h2 = lane >> 5, r32 = lane & 31;
  const int bh = T.t[blockIdx.x][0], q0 = T.t[blockIdx.x][1], k0 = T.t[blockIdx.x][2];
  load_k_chunk<D, 64>(klds, A.kc + (static_cast<int64_t>(bh) * A.Nkv_pad + k0) * D, lane);
  __syncthreads();
  v4i qv[D / 32];
  load_q<D>(qv, A.qc + (static_cast<int64_t>(bh) * A.Nq_pad + q0 + r32) * D, h2);
  v16i s0, s1;
  qk_chunk<D>(klds, qv, lane, s0, s1);
  int32_t* o = out + static_cast<int64_t>(blockIdx.x) * 32 * 64 + r32 * 64 + 16 * h2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    o[i] = s0[i] - SBIAS;
    o[32 + i] = s1[i] - SBIAS;
  }
}

// ---------------------------------------------------------------- launchers
static AttnArgs make_args(const AttnLaunch& L) {
  AttnArgs A{};
  A.qc = L.bufs.q_codes;
  A.qscale = L.bufs.q_scale;
  A.kc = L.bufs.k_codes;
  A.kscale = L.bufs.k_scale;
  A.vt = L.bufs.v_t;
  A.ve = L.bufs.v_e8m0;
  A.o = L.o;
  A.os_b = L.os[0];
  A.os_h = L.os[1];
  A.os_n = L.os[2];
  A.part_o = static_cast<float*>(L.bufs.partial);
  A.part_ml = L.bufs.partial
                  ? static_cast<float*>(L.bufs.partial) +
                        static_cast<int64_t>(L.splits) * L.B * L.H * L.Nq_pad * L.d
                  : nullptr;
  A.B = L.B;
  A.H = L.H;
  A.Nq = L.Nq;
  A.Nq_pad = L.Nq_pad;
  A.Nkv_pad = L.Nkv_pad;
  A.nqt = L.Nq_pad / BQ;
  A.splits = L.splits;
  // work items: 256-row tiles for the ping-pong shape (no block mask), else
  // 128-row blocks
  A.total = L.B * L.H * L.splits * (L.block_mask ? A.nqt : (A.nqt + 1) / 2);
  A.sigma = L.sigma;
  A.frame_len = L.frame_len;
  A.frame_stride = L.frame_stride;
  A.sink_frames = L.sink_frames;
  A.window_frames = L.window_frames;
  A.cpf_magic = L.cpf_magic;
  A.block_mask = L.block_mask;
  A.mask_nkc = L.mask_nkc;
  A.bi = L.bi;
  for (int i = 0; i < MAXB_ARGS; ++i) A.order[i] = L.order[i];
  return A;
}

template <int D, int PV, int DT>
static hipError_t attn_impl(const AttnLaunch& L, hipStream_t st) {
  const AttnArgs A = make_args(L);
  if (L.block_mask)
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_SPARSE, false>), dim3(A.total), dim3(256), 0, st, A);
  else if (L.frame_stride > 0)
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_CACHE, true>), dim3(A.total), dim3(512), 0, st, A);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_DENSE, true>), dim3(A.total), dim3(512), 0, st, A);
  if (L.splits > 1) {
    const int64_t threads = static_cast<int64_t>(L.B) * L.H * L.Nq_pad * (D / 4);
    hipLaunchKernelGGL((attn_combine_kernel<D, DT>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, st, A);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t attn_d(const AttnLaunch& L, hipStream_t st) {
  if (L.pv_mode == PVFP8)
    return L.dtype == DT_BF16 ? attn_impl<D, PVFP8, DT_BF16>(L, st) : attn_impl<D, PVFP8, DT_F16>(L, st);
  return L.dtype == DT_BF16 ? attn_impl<D, PV16, DT_BF16>(L, st) : attn_impl<D, PV16, DT_F16>(L, st);
}

hipError_t launch_attention(const AttnLaunch& L, hipStream_t st) {
  return L.d == 128 ? attn_d<128>(L, st) : attn_d<64>(L, st);
}

hipError_t launch_debug_scores(const AttnLaunch& L, const int32_t* tiles, int ntiles, int32_t* out,
                               hipStream_t st) {
  const AttnArgs A = make_args(L);
  for (int base = 0; base < ntiles; base += 128) {
    DebugTiles T{};
    T.n = ntiles - base < 128 ? ntiles - base : 128;
    for (int i = 0; i < T.n; ++i)
      for (int k = 0; k < 3; ++k) T.t[i][k] = tiles[3 * (base + i) + k];
    int32_t* o = out + static_cast<int64_t>(base) * 32 * 64;
    if (L.d == 128)
      hipLaunchKernelGGL(debug_scores_kernel<128>, dim3(T.n), dim3(64), 0, st, A, T, o);
    else
      hipLaunchKernelGGL(debug_scores_kernel<64>, dim3(T.n), dim3(64), 0, st, A, T, o);
  }
  return hipGetLastError();
}

}  // namespace sage
