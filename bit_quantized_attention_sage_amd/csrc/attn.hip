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
// A workgroup ("ping-pong") is 8 waves = two 128-row query blocks (two Q
// scales) of one (b, h) and optionally one of several KV splits.  Waves w
// and w+4 sit on the same SIMD; group 0 (waves 0-3) runs one phase ahead of
// group 1, and each chunk step is two phases split by a barrier: the MFMAs,
// then the softmax.  So on every SIMD one wave's matrix work meets the
// other's vector work, which the hardware overlaps, instead of each wave
// interleaving both (measured on gfx950: one wave issues plain FP32 VALU ops
// every ~5 cycles, two every ~2.5; exp and the FP8 conversion take ~8.4
// cycles per wave instruction either way).  On contiguous keys and over a
// frame cache the two blocks share every staged K/V chunk (group 0 stages
// them); under a block mask each block walks its own kept chunks, staged by
// its own group into its own buffers, for as many steps as the longer list
// has (the shorter list's missing entries are masked out).
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
#include <mutex>
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
// F = F0 + S 2^-26 (F0 = 1/(2 pi) rounded to float32), so the softmax reads
// the score as a float without a conversion: F and F0 lie in [1/8, 1/4), so
// F - F0 = S 2^-26 exactly (Sterbenz), and fma(F - F0, c 2^26, -mref) is
// fp32(S c - mref) rounded once, as the scheme defines it.  (The row maximum
// is taken on the integer bits, which order like S.)
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
  int64_t vt_hb;    // bytes of one (b,h)'s V^T operand
  const int* pick;  // per-head P.V mode: this launch's heads ([0] = count,
                    // then b*H + h in batch order); null: every head
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

  // Softmax of one chunk, in two halves.  head: the row maximum over the
  // chunk (the two lane halves hold the same query), the lazy running-max
  // update (the row adopts the chunk maximum only when it exceeds m by more
  // than TAU), then p = 2^x for the scores in s0 rounded into P's first half;
  // returns alpha (1 for rows that kept m), by which the caller rescales O
  // and the row sums when any row of the wave moved.  tail: the same for s1
  // into P's second half.  x = fp32(S c - mref) is rounded once, as the
  // scheme defines it: F - F0 = S 2^-26 exactly, then one FMA.  The row
  // sums of the rounded P are taken on the matrix cores in pv().
  // `has`: this row has a visible key in the chunk (rows without one keep m).
  float xc_, xk_;  // c 2^26 and -mref of the chunk being converted
  bool moved_;     // some row of the wave adopted a new maximum in the last softmax

  __device__ __forceinline__ float softmax_head(const v16i& s0, const v16i& s1, float c, bool has,
                                                PTile<PV>& P) {
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
    // tm = fp32(S c), m + TAU and m - tm each rounded on their own, as the
    // scheme defines them (the _rn forms keep the compiler from fusing them)
    const float tm = __fmul_rn(static_cast<float>(mx - SBIAS), c);
    const bool upd = has && (tm > __fadd_rn(m, TAU));
    // (a ballot here, long before the rescale test reads it: a test on a
    // compare issued after the softmax would wait for the whole softmax)
    moved_ = __ballot(upd) != 0;
    const float alpha = upd ? __builtin_amdgcn_exp2f(__fsub_rn(m, tm)) : 1.0f;
    m = upd ? tm : m;
    xk_ = -(m - static_cast<float>(SHIFT));
    // c 2^26, exact; a zero scale (all-zero Q or K block: every score 0)
    // becomes the smallest normal float, so that MASKED keys (F = -inf)
    // still give -inf and the others x = -mref up to S 2^-126
    xc_ = fmaxf(c, 1.17549435e-38f) * 67108864.0f;
    exps<0>(s0, P);
    return alpha;
  }
  __device__ __forceinline__ void softmax_tail(const v16i& s1, PTile<PV>& P) { exps<1>(s1, P); }
  __device__ __forceinline__ float softmax(const v16i& s0, const v16i& s1, float c, bool has, PTile<PV>& P) {
    const float alpha = softmax_head(s0, s1, c, has, P);
    softmax_tail(s1, P);
    return alpha;
  }

  template <int HALF>
  __device__ __forceinline__ void exps(const v16i& s, PTile<PV>& P) {
    const float f0 = __builtin_bit_cast(float, SBIAS);
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // (copy the element out first: a bit cast of a vector subscript reads element 0)
      const int bi = s[i];
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(__builtin_bit_cast(float, bi) - f0, xc_, xk_));
    }
    if constexpr (PV == PVFP8) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        P.b[4 * HALF + k] = static_cast<int>(pack_e4m3x4_into(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]));
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) P.w[8 * HALF + k] = Pack16<DT>::pack(p[2 * k], p[2 * k + 1]);
    }
  }

  // O and l as the MFMA phase leaves them: without this the compiler may sink
  // the phase's P.V MFMAs (pure operations whose results are next used a step
  // later) past the phase's barrier into the softmax phase
  __device__ __forceinline__ void pin_acc() {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) asm volatile("" : "+v"(o[cb]));
    asm volatile("" : "+v"(ls));
  }

  // O and l times alpha, when some row moved (alpha is 1 for the others)
  __device__ __forceinline__ void rescale(float alpha) {
    if (moved_) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
      ls[0] *= alpha;
    }
  }

  // O += P V over the chunk, and with SUMS the row sums of P (in FP8 mode
  // after the P.V MFMAs, with 16-bit P.V one after each K step's four); e8:
  // this lane's four E8M0 bytes (FP8 mode; byte cb scales channel block cb
  // of the lane's 32-key block).
  template <bool SUMS>
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
      if constexpr (SUMS) rowsums(P, lane);
    } else {
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
        if constexpr (SUMS) rowsum16(P, lane, mu);
      }
    }
  }

  // Row sums of P on the matrix cores (no LDS operand): l += P times the
  // selector of lsum_select.  rowsum16 is K step mu of the 16-bit form.
  __device__ __forceinline__ void rowsum16(const PTile<PV>& P, int lane, int mu) {
    const int s1 = lsum_select(lane, DT == DT_BF16 ? 0x3F803F80 : 0x3C003C00);  // 1.0 pairs
    const v4i sel = {s1, s1, s1, s1};
    const v4i pbv = {static_cast<int>(P.w[4 * mu]), static_cast<int>(P.w[4 * mu + 1]),
                     static_cast<int>(P.w[4 * mu + 2]), static_cast<int>(P.w[4 * mu + 3])};
    if (DT == DT_BF16)
      ls = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, sel), __builtin_bit_cast(v8bf, pbv),
                                                   ls, 0, 0, 0);
    else
      ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, sel), __builtin_bit_cast(v8h, pbv),
                                                  ls, 0, 0, 0);
  }
  __device__ __forceinline__ void rowsums(const PTile<PV>& P, int lane) {
    if constexpr (PV == PVFP8) {
      const int s1 = lsum_select(lane, 0x38383838);  // e4m3 1.0 = 0x38
      const v8i sel = {s1, s1, s1, s1, s1, s1, s1, s1};
      ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, P.b, ls, 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int mu = 0; mu < 4; ++mu) rowsum16(P, lane, mu);
    }
  }

};

// Key layouts / chunk lists of the fused kernel.
enum { KV_DENSE = 0,    // contiguous keys, every chunk up to the tile's range end
       KV_CACHE = 1,    // frame cache: the sink frames' chunks, then the window's
       KV_SPARSE = 2 }; // contiguous keys, only the chunks the block mask keeps
constexpr int MAX_LIST = 4096;  // kept-chunk list of a tile (LDS, 2 bytes each)

// The key chunks one work item visits, in order, and which keys of a chunk
// each query row sees.  A work item is a tile of query rows [row_first,
// row_last] of one (b, h) and one KV split.  Each batch's chunks form one
// ordered list, the same for every tile; split s takes entries
// [s*n/S, (s+1)*n/S) of it, and the tile visits the entries of that part that
// its rows can see, as entries [v_lo, v_hi) of its own list:
//  * contiguous keys: the batch's chunks [0, ceil(kv_len/64)); the tile's
//    list is the prefix up to its last row's range end; entry v is chunk v;
//    a row sees the prefix [0, re) of the keys;
//  * block mask: the same parts of the batch's chunks; the tile's list is
//    the chunks of its part that the mask keeps (and its last row can see),
//    compacted in order into LDS; entries then run from 0;
//  * frame cache: the chunks some row of the batch sees -- the sink frames',
//    then the window frames' from the first query's window start through the
//    last query's frame (up to its last token); the tile's own list is built
//    the same way over its rows (entry v is chunk v for v < a0, else chunk
//    b1 + (v - a0)); a row sees the valid slots of the frames of its window.
// List entries below v_full are visible in full to every row of the tile.
template <int MODE>
struct WorkList {
  int v_lo, v_hi, v_full;
  int kv_len, F, FS, sink, window;
  uint32_t cpf_magic;
  int re;                 // contiguous keys: this row's range end
  int full_end;           // contiguous keys: the first row's range end
  int fq, fq_lo, fq_hi;   // frame cache: this row's frame, the tile's first / last rows' frames
  int a0, b1;             // frame cache: the tile list's sink / window cut
  const uint16_t* slist;  // block mask: the kept chunks of the tile

  // physical chunk of list entry v; contiguous keys: v itself (the loads
  // clamp it to the head's last chunk); frame cache and block mask: clamped
  // to the item's range first
  __device__ __forceinline__ int chunk_of(int v) const {
    if constexpr (MODE == KV_DENSE) {
      return v;
    } else if constexpr (MODE == KV_SPARSE) {
      if (v_hi <= v_lo) return 0;
      v = max(min(v, v_hi - 1), v_lo);
      return __builtin_amdgcn_readfirstlane(static_cast<int>(slist[v]));
    } else {
      v = max(min(v, v_hi - 1), 0);
      return v < a0 ? v : b1 + (v - a0);
    }
  }
  // block mask: the list entry of v (clamped like chunk_of) as a vector
  // register, for a read issued well before its value is needed.  An empty
  // list reads entry 0, which becomes chunk 0: with LATE_SELECT when the
  // value moves to a scalar register (entry_chunk), else in the vector
  // register at once (a select right after the read waits for it there).
  template <bool LATE_SELECT>
  __device__ __forceinline__ int entry_of(int v) const {
    const int e = slist[max(min(v, v_hi - 1), v_lo)];
    return LATE_SELECT || v_hi > v_lo ? e : 0;
  }
  template <bool LATE_SELECT>
  __device__ __forceinline__ int entry_chunk(int e) const {
    const int c = __builtin_amdgcn_readfirstlane(e);
    return !LATE_SELECT || v_hi > v_lo ? c : 0;
  }
  // frame of cache chunk ch: ch / (FS/64) by a multiply-high with the host's
  // rounded-up reciprocal (exact for ch < 2^20, FS/64 < 2^11); with one chunk
  // per frame the reciprocal (2^32) does not fit and f = ch
  __device__ __forceinline__ int frame_of(int ch) const {
    return FS == 64 ? ch : static_cast<int>(__umulhi(static_cast<uint32_t>(ch), cpf_magic));
  }
  // every row of the tile sees all 64 keys of chunk ch (wave-uniform)
  __device__ __forceinline__ bool chunk_full(int ch) const {
    if constexpr (MODE != KV_CACHE) return (ch + 1) * 64 <= full_end;
    const int f = frame_of(ch);
    const int t0 = (ch - f * (FS / 64)) * 64;
    const int vc = min(min(F - t0, kv_len - (f * F + t0)), 64);
    const bool all = f <= fq_lo && (window == 0 || f < sink || f >= fq_hi - window);
    return vc >= 64 && all;
  }
  // this row sees the first row_lim(ch) keys of chunk ch
  __device__ __forceinline__ int row_lim(int ch) const {
    if constexpr (MODE != KV_CACHE) return re - ch * 64;
    const int f = frame_of(ch);
    const int t0 = (ch - f * (FS / 64)) * 64;
    const int vc = min(min(F - t0, kv_len - (f * F + t0)), 64);
    const bool vis = f <= fq && (window == 0 || f < sink || f >= fq - window);
    return vis ? vc : 0;
  }
};

// Build the list of one work item (see WorkList).  NT threads take part
// (the block-mask list is compacted by the whole workgroup; the call holds
// barriers then, so every thread of the workgroup must make it).
template <int MODE, int NT>
__device__ __forceinline__ WorkList<MODE> make_worklist(const AttnArgs& A, int b, int bh, int mask_tile, int split,
                                                        int row_first, int row_last, int qi_valid, int tid,
                                                        uint16_t* slist, int* scnt) {
  WorkList<MODE> L;
  const int kv_len = A.bi.kv_len[b], q_pos0 = A.bi.q_pos0[b], F = A.frame_len;
  L.kv_len = kv_len;
  L.F = F;
  L.FS = MODE == KV_CACHE ? A.frame_stride : 0;
  L.sink = A.sink_frames;
  L.window = A.window_frames;
  L.cpf_magic = A.cpf_magic;
  L.re = L.full_end = L.fq = L.fq_lo = L.fq_hi = L.a0 = L.b1 = 0;
  L.slist = slist;
  if constexpr (MODE != KV_CACHE) {
    L.re = F > 0 ? min(kv_len, ((q_pos0 + qi_valid) / F + 1) * F) : kv_len;
    const int first_end = F > 0 ? min(kv_len, ((q_pos0 + row_first) / F + 1) * F) : kv_len;
    const int last_end = F > 0 ? min(kv_len, ((q_pos0 + row_last) / F + 1) * F) : kv_len;
    const int nch = (kv_len + 63) / 64;
    L.v_lo = split * nch / A.splits;
    L.v_hi = min((split + 1) * nch / A.splits, (last_end + 63) / 64);
    L.full_end = first_end;
    L.v_full = first_end / 64;
    if constexpr (MODE == KV_SPARSE) {
      // the chunks of [v_lo, v_hi) the mask keeps, compacted in order by the
      // whole workgroup (ballot + per-wave counts); `below` counts those
      // visible in full to every row
      constexpr int NW = NT / 64;
      const int lane = tid & 63, w = tid >> 6;
      const int nfull = first_end / 64;
      const uint8_t* mrow = A.block_mask + (static_cast<int64_t>(bh) * A.nqt + mask_tile) * A.mask_nkc;
      // (the loop runs to the split's end, the same for every thread of the
      // workgroup: its barriers are the workgroup's)
      const int split_hi = (split + 1) * nch / A.splits;
      int total = 0, below = 0;
      for (int c0 = L.v_lo; c0 < split_hi; c0 += NT) {
        const int c = c0 + tid;
        const bool keep = c < L.v_hi && mrow[c] != 0;
        const uint64_t bk = __ballot(keep), bf = __ballot(keep && c < nfull);
        if (lane == 0) {
          scnt[w] = __popcll(bk);
          scnt[NW + w] = __popcll(bf);
        }
        __syncthreads();
        int off = total;
        for (int i = 0; i < w; ++i) off += scnt[i];
        const int rank = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bk >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bk), 0));
        if (keep) slist[off + rank] = static_cast<uint16_t>(c);
        for (int i = 0; i < NW; ++i) {
          total += scnt[i];
          below += scnt[NW + i];
        }
        __syncthreads();
      }
      L.v_lo = 0;
      L.v_hi = total;
      L.v_full = below;
    }
  } else {
    const int FS = L.FS, cpf = FS / 64;
    L.fq = (q_pos0 + qi_valid) / F;
    L.fq_lo = (q_pos0 + row_first) / F;
    L.fq_hi = (q_pos0 + row_last) / F;
    const int end_chunk = (L.fq_hi * FS + min(F, kv_len - L.fq_hi * F) + 63) / 64;
    int nv = end_chunk;
    if (A.window_frames > 0) {
      L.a0 = min(min(A.sink_frames, L.fq_hi + 1) * cpf, end_chunk);
      L.b1 = max(min(max(A.sink_frames, L.fq_lo - A.window_frames) * cpf, end_chunk), L.a0);
      nv = L.a0 + (end_chunk - L.b1);
    }
    // the batch's list over all its query rows, cut into the splits' parts;
    // tile_count(V): entries of the tile's list whose chunk lies before the
    // chunk of batch entry V
    const int FQ_lo = q_pos0 / F, FQ_hi = (q_pos0 + A.Nq - 1) / F;
    const int END = (FQ_hi * FS + min(F, kv_len - FQ_hi * F) + 63) / 64;
    int A0 = 0, B1 = 0;
    if (A.window_frames > 0) {
      A0 = min(min(A.sink_frames, FQ_hi + 1) * cpf, END);
      B1 = max(min(max(A.sink_frames, FQ_lo - A.window_frames) * cpf, END), A0);
    }
    const int NV = A0 + (END - B1);
    const int a0 = L.a0, b1 = L.b1;
    auto tile_count = [&](int V) -> int {
      if (V >= NV) return nv;
      const int ch = V < A0 ? V : B1 + (V - A0);
      return min(ch, a0) + max(0, min(ch, end_chunk) - b1);
    };
    L.v_lo = tile_count(split * NV / A.splits);
    L.v_hi = tile_count((split + 1) * NV / A.splits);
    L.v_full = 0;  // no shortcut over a frame cache
  }
  return L;
}

// Staging of K and V^T chunks from HBM straight into LDS: raw buffer loads
// that write LDS (no registers), issued by the four waves of one group.
// Lane l of DMA instruction i of the group's wave w fills LDS granule
// (4i + w)*64 + l of the buffer;
// its global source is chosen so that the buffer ends up in the swizzled
// layouts above.  Every chunk index is clamped to the head's last padded
// chunk, so all reads stay inside the head's slice; the prefetches that the
// clamp redirects are never consumed.  The K scale and this lane's four E8M0
// bytes of a chunk are plain loads into registers.
template <int D, int PV>
struct Stager {
  static constexpr int VBYTES = (PV == PVFP8) ? 1 : 2;
  static constexpr int KB = 64 * D;            // bytes of a K chunk
  static constexpr int VBC = 64 * D * VBYTES;  // bytes of a V^T chunk
  static constexpr int KI = KB / 4096;         // 1 KB DMA instructions per wave, K
  static constexpr int VI = VBC / 4096;        // ... and V
  static_assert(KI >= 1 && KI <= 2 && VI >= 1 && VI <= 4, "staging shape");
  __amdgpu_buffer_rsrc_t krs, vrs, ers, srs;
  int last, w, lane;
  // source offset, inside a chunk, of the 16 bytes this lane's DMA
  // instruction i brings to LDS granule (4i + w)*64 + lane
  __device__ __forceinline__ int koff(int i) const {
    constexpr int G = D / 16;
    const int sidx = (4 * i + w) * 64 + lane, key = sidx / G, gp = sidx % G;
    return key * D + ((gp ^ k_swz<D>(key)) << 4);
  }
  __device__ __forceinline__ int voff(int i) const {
    constexpr int GR = VRow<PV>::GR;
    const int sidx = (4 * i + w) * 64 + lane, c = sidx / GR, gp = sidx % GR;
    return c * VRow<PV>::BYTES + ((gp ^ VRow<PV>::swz(c)) << 4);
  }

  __device__ __forceinline__ void init(const AttnArgs& A, int bh, int wave, int lane) {
    const int nkc = A.Nkv_pad / 64;
    const int8_t* kbase = A.kc + static_cast<int64_t>(bh) * A.Nkv_pad * D;
    const uint8_t* vbase = static_cast<const uint8_t*>(A.vt) + static_cast<int64_t>(bh) * A.vt_hb;
    const uint8_t* ebase = A.ve + static_cast<int64_t>(bh) * nkc * 256;
    const float* ksc = A.kscale + static_cast<int64_t>(bh) * nkc;
    krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kbase), 0, nkc * KB, 0x00020000);
    vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase), 0, nkc * VBC, 0x00020000);
    ers = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ebase), 0, PV == PVFP8 ? nkc * 256 : 0,
                                            0x00020000);
    srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ksc), 0, nkc * 4, 0x00020000);
    w = wave & 3;
    this->lane = lane;
    last = nkc - 1;  // chunk indices are clamped: prefetches past the end go unused
  }
  __device__ __forceinline__ void dma_k(int8_t* dst, int ch) const {
    ch = min(ch, last);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      // (the offset goes through a local: any other expression as this
      // builtin's argument makes the host pass drop the kernel's launch stub)
      const int off = koff(i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, dst + (4 * i + w) * 1024, 16, off, ch * KB, 0, 0);
    }
  }
  __device__ __forceinline__ void dma_v(uint8_t* dst, int ch) const {
    ch = min(ch, last);
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int off = voff(i);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, dst + (4 * i + w) * 1024, 16, off, ch * VBC, 0, 0);
    }
  }
  __device__ __forceinline__ float load_ks(int ch) const {
    ch = min(ch, last);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 0, ch * 4, 0));
  }
  __device__ __forceinline__ int load_e(int ch, int lane) const {
    ch = min(ch, last);
    return PV == PVFP8 ? __builtin_amdgcn_raw_buffer_load_b32(ers, lane * 4, ch * 256, 0) : 0;
  }
};

__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Decode a work item (batch by decreasing kv_len, head, split, query tile)
// from a physical workgroup id: the tiles of one (b, h, split) share an XCD.
// With a head list (PICK: per-head P.V mode) the items are those of the
// listed heads, in list order; the launch has room for every head, and the
// kernel returns at once in workgroups past the list's items.
struct Item {
  int b, h, split, qt, bh;
  __device__ __forceinline__ Item(const AttnArgs& A, int ntile) {
    const int L = xcd_group_remap(blockIdx.x, A.total, ntile);
    const int per_b = A.H * A.splits * ntile;
    b = A.order[L / per_b];
    int rem = L % per_b;
    h = rem / (A.splits * ntile);
    rem %= A.splits * ntile;
    split = rem / ntile;
    qt = rem % ntile;
    bh = b * A.H + h;
  }
  __device__ __forceinline__ Item(const AttnArgs& A, int ntile, int total) {
    const int per_bh = A.splits * ntile;
    const int L = xcd_group_remap(blockIdx.x, total, ntile);
    bh = A.pick[1 + L / per_bh];
    b = bh / A.H;
    h = bh - b * A.H;
    const int rem = L % per_bh;
    split = rem / ntile;
    qt = rem % ntile;
  }
};

__device__ __forceinline__ int pick_items(const AttnArgs& A, int ntile) { return A.pick[0] * A.splits * ntile; }

// Normalise and store this lane's row of O, or (with KV splits) its
// unnormalised-by-merge partial: O / l and (m, l).
template <int D, int DT>
__device__ __forceinline__ void store_row(const AttnArgs& A, const v16f* o, float m, float ltot, int b, int h,
                                          int bh, int split, int qi, int h2) {
  constexpr int NCB = D / 32;
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // a row with no visible key: 0
  if (A.splits == 1) {
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

// Masking at boundaries (the last chunks of a row's range, frame padding,
// window edges, entries past the shorter list of a block-mask pair), in two
// parts.  needs_mask: whether list entry v needs masking for some row of the
// workgroup (wave-uniform, scalar work).  apply_mask: keys a row does not see
// get the MASKED score; returns whether this row has a visible key in the
// chunk.
// (ch: the chunk of entry v)
template <int MODE>
__device__ __forceinline__ bool needs_mask(const WorkList<MODE>& wl, int v, int ch) {
  if constexpr (MODE == KV_SPARSE) {
    if (v >= wl.v_hi) return true;  // past this block's list (the pair's other list is longer)
  }
  return !wl.chunk_full(ch);
}
template <int D, int PV, int DT, int MODE>
__device__ __forceinline__ bool apply_mask(const WorkList<MODE>& wl, WaveState<D, PV, DT>& st, int v, v16i& s0,
                                           v16i& s1, int h2) {
  const int lim = (MODE == KV_SPARSE && v >= wl.v_hi) ? 0 : wl.row_lim(wl.chunk_of(v));
  st.mask(s0, s1, lim - 16 * h2);
  return lim > 0;
}
template <int D, int PV, int DT, int MODE>
__device__ __forceinline__ bool mask_chunk(const WorkList<MODE>& wl, WaveState<D, PV, DT>& st, int v, v16i& s0,
                                           v16i& s1, int h2) {
  if (!needs_mask(wl, v, wl.chunk_of(v))) return true;
  asm volatile("");  // keep this a real branch
  return apply_mask(wl, st, v, s0, s1, h2);
}

template <int D, int PV, int DT, int MODE, bool PICK>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnArgs A) {
  constexpr bool SPARSE = MODE == KV_SPARSE;
  constexpr int NWAVE = 8;
  constexpr int NCB = D / 32;                    // 32-channel blocks of O
  // Under a block mask each 128-row Q block keeps its own chunks: a ping-pong
  // workgroup then holds two chunk lists, and each group stages its own
  // list's chunks into its own buffers.
  constexpr int NLIST = SPARSE ? 2 : 1;
  using SG = Stager<D, PV>;
  // Two buffers each (per list), as separate objects so that the compiler can
  // tell the buffer being filled by DMA from the one being read.
  __shared__ __attribute__((aligned(16))) int8_t kLs0[NLIST * SG::KB];
  __shared__ __attribute__((aligned(16))) int8_t kLs1[NLIST * SG::KB];
  __shared__ __attribute__((aligned(16))) uint8_t vLs0[NLIST * SG::VBC];
  __shared__ __attribute__((aligned(16))) uint8_t vLs1[NLIST * SG::VBC];
  __shared__ uint16_t slist[SPARSE ? NLIST * MAX_LIST : 1];  // kept chunks of each list, ascending
  __shared__ int scnt[2 * NWAVE];
  __shared__ int slen[2 * NLIST];  // block mask + ping-pong: each list's length and fully visible prefix

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5;

  const int ntile = (A.nqt + 1) / 2;  // tiles of two 128-row Q blocks
  int pick_total = 0;
  if constexpr (PICK) {
    pick_total = pick_items(A, ntile);
    if (static_cast<int>(blockIdx.x) >= pick_total) return;  // uniform, before any barrier
  }
  const Item it = PICK ? Item(A, ntile, pick_total) : Item(A, ntile);
  const int b = it.b, h = it.h, split = it.split, qt = it.qt, bh = it.bh;
  // this wave's group, its place in the group and its 128-row Q block (the
  // second block of the last tile may lie past Nq: its rows load the last
  // real block and store nothing)
  const int grp = w >> 2, w4 = w & 3;
  const int qb = 2 * qt + grp;
  const int qbl = min(qb, A.nqt - 1);
  const int qi = qb * BQ + w4 * 32 + (lane & 31);
  const int qi_valid = min(qi, A.Nq - 1);
  const int lst = NLIST > 1 ? grp : 0;  // this wave's list
  int8_t* const kL0 = kLs0 + lst * SG::KB;
  int8_t* const kL1 = kLs1 + lst * SG::KB;
  uint8_t* const vL0 = vLs0 + lst * SG::VBC;
  uint8_t* const vL1 = vLs1 + lst * SG::VBC;
  const int row_first = (NLIST > 1 ? qbl : 2 * qt) * BQ;
  const int row_last = min(row_first + (NLIST > 1 ? BQ : NWAVE * 32), A.Nq) - 1;
  const WorkList<MODE> wl =
      NLIST > 1 ? make_worklist<MODE, 256>(A, b, bh, qbl, split, row_first, row_last, qi_valid, tid & 255,
                                           slist + lst * MAX_LIST, scnt + 8 * lst)
                : make_worklist<MODE, NWAVE * 64>(A, b, bh, qt, split, row_first, row_last, qi_valid, tid, slist,
                                                  scnt);
  const int v_lo = wl.v_lo;
  // The loop's trip counts are the workgroup's (its barriers are shared):
  // with two lists, the longer list's length and the shorter fully visible
  // prefix; the shorter list's missing entries are masked out.
  int J = max(0, wl.v_hi - v_lo), v_full = wl.v_full;
  if constexpr (NLIST > 1) {
    if (tid == 256 * lst) {
      slen[lst] = J;
      slen[2 + lst] = v_full;
    }
    __syncthreads();
    J = max(slen[0], slen[1]);
    v_full = min(slen[2], slen[3]);
  }

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

  SG sg;
  sg.init(A, bh, w, lane);
  // group 0 stages the chunks of a shared list, each group those of its own
  const bool stager = NLIST > 1 || grp == 0;
  auto dma_k = [&](int8_t* dst, int ch) { if (stager) sg.dma_k(dst, ch); };
  auto dma_v = [&](uint8_t* dst, int ch) { if (stager) sg.dma_v(dst, ch); };
  auto chunk_of = [&](int v) { return wl.chunk_of(v); };
  auto mask_at = [&](int v, v16i& s0, v16i& s1) { return mask_chunk(wl, st, v, s0, s1, h2); };

  // Software pipeline within each wave over three chunks: step j (list entry
  // n = v_lo + j) enters with S(n+1) and P(n) in registers, K(n+2) in K buffer
  // j&1 and V(n) in V buffer j&1.  It issues the DMA of K(n+3) and V(n+1),
  // then two phases split by a barrier: the S MFMAs of entry n+2 and the P.V
  // MFMAs of entry n (at raised wave priority, with the operand reads 8
  // ahead), and the softmax of entry n+1 (preceded, for a boundary chunk, by
  // its masking, decided a step earlier); then the (rare) rescale by entry
  // n+1's alpha, the wait for this step's DMA and the barrier.  Group 1 runs the same steps one phase behind group 0
  // (one extra barrier before its first step, group 0 one after its last),
  // so on every SIMD one wave's matrix work meets the other wave's softmax,
  // and the buffers a step fills are the ones their readers finished with in
  // the step before.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  v16i sa0{}, sa1{}, sb0{}, sb1{};
  PTile<PV> pa, pb;
  bool ha = true, hb = true;    // the rows' visibility flags of the chunks in sa, sb
  bool na = false, nb = false;  // the chunks in sa, sb still need masking (decided a step ahead)
  int n = v_lo;
  int e_cur = sg.load_e(chunk_of(n), lane);
  float ksn1 = sg.load_ks(chunk_of(n + 1)), ksn2 = sg.load_ks(chunk_of(n + 2));  // K scales of n+1, n+2
  // Prologue: K(n) and V(n) in buffers 0, K(n+1) in K buffer 1; then S(n+1),
  // P(n) and K(n+2) in K buffer 0.
  {
    const float ks0 = sg.load_ks(chunk_of(n));
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
      hb = mask_at(n, sb0, sb1);
      if (J >= 2) ha = mask_at(n + 1, sa0, sa1);
      st.rescale(st.softmax(sb0, sb1, qsc * ks0, hb, pa));
      dma_wait();
      __syncthreads();
    }
  }
  // Every load issued so far has completed; saying so keeps the loop's own
  // prefetch loads from being waited on before the first MFMA.
  __builtin_amdgcn_s_waitcnt(0);
  // The next step's chunks of entries n+1 and n+3, computed a phase ahead:
  // under a block mask (LDS reads), and over a frame cache with 16-bit P.V
  // (frame arithmetic, moved out of that mode's longer MFMA phase).
  constexpr bool AHEAD = SPARSE || (MODE == KV_CACHE && PV != PVFP8);
  int pre1 = 0, pre3 = 0;
  if constexpr (AHEAD) {
    pre1 = chunk_of(n + 1);
    pre3 = chunk_of(n + 3);
  }

  // CHK false: S(n+1) and S(n+2) are visible in full to every row (no masking
  // check, every row has keys in entry n+1).
  auto step = [&](auto par, auto chk, v16i& cs0, v16i& cs1, bool& has_c, bool& nd_c, PTile<PV>& p_cur,
                  v16i& ns0, v16i& ns1, bool& has_n, bool& nd_n, PTile<PV>& p_nxt) {
    constexpr int P = decltype(par)::value;  // parity of the step
    constexpr bool CHK = decltype(chk)::value;
    int8_t* k_rd = P ? kL1 : kL0;            // K(n+2)
    int8_t* k_wr = P ? kL0 : kL1;            // receives K(n+3)
    uint8_t* v_rd = P ? vL1 : vL0;           // V(n)
    uint8_t* v_wr = P ? vL0 : vL1;           // receives V(n+1)
    constexpr int NQK = 2 * D / 32;                               // S MFMAs
    constexpr int NPV = (PV == PVFP8) ? NCB + 1 : 4 * NCB + 4;    // P.V and row-sum MFMAs
    constexpr int NRD = NQK + ((PV == PVFP8) ? 2 * NCB : 4 * NCB);  // LDS operand reads
    const float c_mid = qsc * ksn1;
    const int ch1 = AHEAD ? pre1 : chunk_of(n + 1), ch3 = AHEAD ? pre3 : chunk_of(n + 3);
    // S(n+2) a boundary chunk?  Scalar work, placed in the phase that has
    // room for it: the MFMA phase in FP8 mode (its softmax phase is the longer
    // one), after the softmax with 16-bit P.V (the other way round).
    constexpr bool DECIDE_EARLY = PV == PVFP8 && !SPARSE;
    // 16-bit P.V on contiguous keys: the four row-sum MFMAs open the phase
    // (they read no LDS operand, so they fill the wait for the first K
    // reads; measured 1% faster on the large workload, 0.5% under a block
    // mask).  In FP8 mode (2% slower that way) and over a frame cache (no
    // faster) they stay with the P.V MFMAs.
    constexpr bool SUMS_FIRST = PV != PVFP8 && MODE != KV_CACHE;
    if constexpr (CHK && DECIDE_EARLY) {
      nd_n = n + 2 >= v_full && needs_mask(wl, n + 2, chunk_of(n + 2));
      has_n = true;
    }
    __builtin_amdgcn_sched_barrier(0);
    dma_k(k_wr, ch3);
    dma_v(v_wr, ch1);
    const int e_nxt = sg.load_e(ch1, lane);
    const float ks3 = sg.load_ks(ch3);
    float alpha;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (SUMS_FIRST) st.rowsums(p_cur, lane);
    qk_chunk<D>(k_rd, qv, lane, ns0, ns1);
    st.template pv<!SUMS_FIRST>(p_cur, v_rd, e_cur, lane);
    __builtin_amdgcn_sched_group_barrier(0x020, 2 + SG::KI + SG::VI, 0);  // the loads
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                    // the first operand reads
#pragma unroll
    for (int g = 0; g < NQK + NPV; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // one MFMA
      if (g + 8 < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
    }
    asm volatile("" : "+v"(ns0), "+v"(ns1));
    // (FP8 P.V, boundary-checked steps -- every step over a frame cache: the
    // checks let the compiler sink the P.V MFMAs into the softmax phase, the
    // longer one)
    if constexpr (PV == PVFP8 && CHK && !SPARSE) st.pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_barrier();  // end of the MFMA phase
    __builtin_amdgcn_sched_barrier(0);
    // block mask: the next step's chunks, read from LDS here and moved to
    // scalar registers after the softmax, which hides the read's latency
    // (16-bit P.V: the empty-list select after the softmax, so that the
    // phase does not wait for these reads at its start -- 0.7% faster; in
    // FP8 mode that way the compiler spills and the kernel is 9% slower)
    constexpr bool LATE_SELECT = PV != PVFP8;
    const int e1 = SPARSE ? wl.template entry_of<LATE_SELECT>(n + 2) : 0;
    const int e3 = SPARSE ? wl.template entry_of<LATE_SELECT>(n + 4) : 0;
    if constexpr (SPARSE && LATE_SELECT) __builtin_amdgcn_sched_barrier(0);  // (the reads stay at the phase start)
    if constexpr (CHK) {
      if (nd_c) {  // rare: entry n+1 is a boundary chunk
        asm volatile("");  // keep this a real branch
        has_c = apply_mask(wl, st, n + 1, cs0, cs1, h2);
      }
    }
    alpha = st.softmax(cs0, cs1, c_mid, CHK ? has_c : true, p_nxt);
    p_nxt.pin();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (SPARSE) {
      pre1 = wl.template entry_chunk<LATE_SELECT>(e1);
      pre3 = wl.template entry_chunk<LATE_SELECT>(e3);
    } else if constexpr (AHEAD) {
      pre1 = chunk_of(n + 2);
      pre3 = chunk_of(n + 4);
    }
    if constexpr (CHK && !DECIDE_EARLY) {  // (block mask: the chunk of entry n+2 is pre1)
      nd_n = n + 2 >= v_full && needs_mask(wl, n + 2, AHEAD ? pre1 : chunk_of(n + 2));
      has_n = true;
    }
    st.rescale(alpha);  // rare: some row's running max moved (after P(n) V(n))
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
    if (grp == 1 && left > 0) __builtin_amdgcn_s_barrier();  // one phase behind group 0
    if constexpr (MODE != KV_CACHE) {
      // the leading steps whose S(n+2) lies below v_full, in pairs
      for (int fast = min(J - 1, v_full - v_lo - 2); fast >= 2; fast -= 2) {
        step(P0{}, NoChk{}, sa0, sa1, ha, na, pa, sb0, sb1, hb, nb, pb);
        step(P1{}, NoChk{}, sb0, sb1, hb, nb, pb, sa0, sa1, ha, na, pa);
        left -= 2;
      }
    }
    while (left >= 2) {
      step(P0{}, Chk{}, sa0, sa1, ha, na, pa, sb0, sb1, hb, nb, pb);
      step(P1{}, Chk{}, sb0, sb1, hb, nb, pb, sa0, sa1, ha, na, pa);
      left -= 2;
    }
    if (grp == 0 && J > 1) __builtin_amdgcn_s_barrier();  // as many barriers as group 1
    // the last entry's P.V (its V is in buffer (J-1)&1)
    if (left == 1) {
      step(P0{}, Chk{}, sa0, sa1, ha, na, pa, sb0, sb1, hb, nb, pb);
      st.template pv<true>(pb, vL1, e_cur, lane);
    } else {
      st.template pv<true>(pa, vL0, e_cur, lane);
    }
  }
  if (qi >= A.Nq) return;
  store_row<D, DT>(A, st.o, st.m, st.ls[0], b, h, bh, split, qi, h2);
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

// ------------------------------------------------- allocation-free scratch
// Split-KV partial results of sage_attn_fwd_quantized_noalloc: a file-scope
// device array, one copy per GPU, held until the process ends.  In host code
// `scratch` is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, fetched once per device with that device current.
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

hipError_t scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ------------------------------------------------- per-head P.V mode lists
// One workgroup lists the heads of each mode, in batch order (A.order) and
// head order: pick[0] = count and pick[1..] the 16-bit heads (some
// channel-balance exponent != 0), pick[1 + BH] = count and pick[2 + BH..] the
// FP8 heads (every exponent 0).
template <int D>
__global__ __launch_bounds__(256) void pick_heads_kernel(AttnArgs A, const int8_t* __restrict__ shift,
                                                         int* __restrict__ pick) {
  __shared__ int cnt[2][4];
  const int n = A.B * A.H, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = lane ? (~uint64_t{0} >> (64 - lane)) : 0;
  int base16 = 0, base8 = 0;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + threadIdx.x;
    const bool valid = i < n;
    int bh = 0;
    bool moved = false;
    if (valid) {
      bh = A.order[i / A.H] * A.H + i % A.H;
      const int8_t* sp = shift + static_cast<int64_t>(bh) * D;
#pragma unroll 8
      for (int c = 0; c < D; ++c) moved |= sp[c] != 0;
    }
    const uint64_t m16 = __ballot(valid && moved), m8 = __ballot(valid && !moved);
    if (lane == 0) {
      cnt[0][w] = __popcll(m16);
      cnt[1][w] = __popcll(m8);
    }
    __syncthreads();
    int o16 = base16, o8 = base8;
    for (int k = 0; k < w; ++k) {
      o16 += cnt[0][k];
      o8 += cnt[1][k];
    }
    if (valid) {
      if (moved) pick[1 + o16 + __popcll(m16 & below)] = bh;
      else pick[2 + n + o8 + __popcll(m8 & below)] = bh;
    }
    for (int k = 0; k < 4; ++k) {
      base16 += cnt[0][k];
      base8 += cnt[1][k];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    pick[0] = base16;
    pick[1 + n] = base8;
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
  // work items: 256-row tiles of the ping-pong workgroup
  A.total = L.B * L.H * L.splits * ((A.nqt + 1) / 2);
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
  A.vt_hb = L.vt_hb;
  A.pick = nullptr;
  return A;
}

template <int D, int PV, int DT, bool PICK>
static void attn_launch(const AttnArgs& A, bool sparse, bool cache, hipStream_t st) {
  if (sparse)
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_SPARSE, PICK>), dim3(A.total), dim3(512), 0, st, A);
  else if (cache)
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_CACHE, false>), dim3(A.total), dim3(512), 0, st, A);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, PV, DT, KV_DENSE, PICK>), dim3(A.total), dim3(512), 0, st, A);
}

// One launch of the fused kernel in the P.V mode of the call, or (PVAUTO) the
// head lists, then one launch per mode over its own heads; then the merge of
// the KV splits.
template <int D, int DT>
static hipError_t attn_impl(const AttnLaunch& L, hipStream_t st) {
  AttnArgs A = make_args(L);
  const bool sparse = L.block_mask != nullptr, cache = L.frame_stride > 0;
  if (L.pv_mode == PVAUTO) {
    hipLaunchKernelGGL(pick_heads_kernel<D>, dim3(1), dim3(256), 0, st, A, L.bufs.chan_shift, L.pick);
    A.pick = L.pick;
    attn_launch<D, PV16, DT, true>(A, sparse, cache, st);
    A.pick = L.pick + 1 + L.B * L.H;
    attn_launch<D, PVFP8, DT, true>(A, sparse, cache, st);
    A.pick = nullptr;
  } else if (L.pv_mode == PVFP8) {
    attn_launch<D, PVFP8, DT, false>(A, sparse, cache, st);
  } else {
    attn_launch<D, PV16, DT, false>(A, sparse, cache, st);
  }
  if (L.splits > 1) {
    const int64_t threads = static_cast<int64_t>(L.B) * L.H * L.Nq_pad * (D / 4);
    hipLaunchKernelGGL((attn_combine_kernel<D, DT>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, st, A);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t attn_d(const AttnLaunch& L, hipStream_t st) {
  return L.dtype == DT_BF16 ? attn_impl<D, DT_BF16>(L, st) : attn_impl<D, DT_F16>(L, st);
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
