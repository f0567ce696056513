// Shared device-side definitions of the quantized attention library (gfx950).
//
// The scheme's constants live here and only here on the GPU side.  The pages
// fix none of them (podcast notes, section "02:48 There were clearly faster
// compute units on the hardware": only "low-bit"); they are this library's
// stated design.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int BQ = 128;          // query tokens per Q scale block
constexpr int BK = 64;           // key tokens per K scale block = softmax chunk
constexpr int VB = 32;           // key tokens per FP8 V scale (E8M0) block
constexpr int QMAX = 127;        // symmetric INT8 range
constexpr int KMEAN_CHUNK = 128; // tokens per first-level partial sum of the K mean
constexpr float TAU = 4.0f;      // lazy running-max threshold (log2 units)
constexpr int PSHIFT_FP8 = 4;    // P stored as e4m3(p * 2^4) in FP8 mode
constexpr int PSHIFT_16 = 0;
constexpr int NPAD = 128;        // Nq and Nkv are padded to multiples of this
constexpr int MAXB = 256;        // largest batch handled through kernel arguments

enum { DT_F16 = 0, DT_BF16 = 1 };
enum { PV16 = 0, PVFP8 = 1, PVAUTO = 2 };  // PVAUTO: per (b,h) from the channel-balance exponents

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// 16-bit storage types; conversions below are explicit and round to nearest even.
struct bf16_t { uint16_t x; };
struct f16_t { uint16_t x; };

__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v.x) << 16);
}
__device__ __forceinline__ float to_f32(f16_t v) {
  _Float16 h;
  __builtin_memcpy(&h, &v.x, 2);
  return static_cast<float>(h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  _Float16 h;
  uint16_t b = static_cast<uint16_t>(bits16);
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

// Two floats -> packed pair of bf16 (RNE; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  uint32_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}
// Two floats -> packed pair of fp16 (RNE, v_cvt_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &ha, 2);
  __builtin_memcpy(&ub, &hb, 2);
  return static_cast<uint32_t>(ua) | (static_cast<uint32_t>(ub) << 16);
}
// Four floats (|x| <= 448) -> four OCP e4m3fn bytes, RNE (v_cvt_pk_fp8_f32).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

// As pack_e4m3x4, without first zeroing the destination: the first convert
// keeps the upper half of its `old` operand, which the second overwrites.
// `old` is a's own register (dead after that convert), so nothing is copied.
__device__ __forceinline__ uint32_t pack_e4m3x4_into(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return static_cast<uint32_t>(r);
}

template <int DT> struct Pack16;
template <> struct Pack16<DT_BF16> {
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ float lo(uint32_t w) { return bf16_bits_to_f32(w & 0xFFFFu); }
  static __device__ __forceinline__ float hi(uint32_t w) { return bf16_bits_to_f32(w >> 16); }
};
template <> struct Pack16<DT_F16> {
  static __device__ __forceinline__ uint32_t pack(float a, float b) { return pack_f16x2(a, b); }
  static __device__ __forceinline__ float lo(uint32_t w) { return f16_bits_to_f32(w & 0xFFFFu); }
  static __device__ __forceinline__ float hi(uint32_t w) { return f16_bits_to_f32(w >> 16); }
};

// max(a, b, c): the compiler emits one v_max3_i32 for it.  (Written in
// C++, not inline asm, so that the compiler's hazard checks cover it: an asm
// instruction that reads or overwrites the registers of a matrix op still in
// flight gets no wait states.)
__device__ __forceinline__ int max3_i32(int a, int b, int c) { return max(max(a, b), c); }

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

// Row of a 64-row tile that row r of subtile u of a 32x32x32 i8 MFMA's A
// operand loads.  With this order, accumulator register i of lane l (output
// row 8*(i/4) + 4*(l/32) + i%4) holds tile row 32*u + 16*(l/32) + i: each
// lane half gets 16 consecutive tile rows.
__device__ __forceinline__ int a_row_key(int r, int u) {
  return 32 * u + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3);
}

// 16-byte granule swizzle of a 64-row tile of D bytes per row in LDS:
// granule g of row k is stored at slot g ^ swz(k).  A ds_read_b128 is served
// 16 lanes at a time from 64 four-byte banks; the 16 rows such a group reads
// (a_row_key order: {0..3, 16..19, 4..7, 20..23} + 8t) then land on 16
// distinct 16-byte bank slots.  The same holds for 8-lane groups over 32
// banks.
template <int D>
__device__ __forceinline__ int k_swz(int key) {
  const int b0 = key & 1, b1 = (key >> 1) & 1, b2 = (key >> 2) & 1, b4 = (key >> 4) & 1;
  if constexpr (D == 128) return b1 | (b4 << 1) | ((b0 ^ b2) << 2);
  else return (b1 ^ b2) | (b4 << 1);
}

// Logical tile index of a physical workgroup id so that the workgroups one XCD
// runs (ids x, x+8, x+16, ... go to XCD x) form one contiguous logical range:
// neighbouring query tiles of the same head then share K/V in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int q = total / 8, r = total % 8;
  const int x = pid % 8, k = pid / 8;
  return x * q + (x < r ? x : r) + k;
}

// Logical tile index of a physical workgroup id when the logical order is a
// sequence of groups of `gsize` consecutive tiles that should share an XCD
// (the query tiles of one head share its K and V in that XCD's L2).  Groups
// are dealt round-robin to the 8 XCDs -- XCD x, whose k-th workgroup is
// physical id 8k + x, runs groups x, x + 8, ... in order, each group's tiles
// consecutively -- so that work ordered by decreasing size is spread evenly
// over the XCDs.  Ids beyond the last complete round of 8 groups map to
// themselves (a bijection on [0, total)).
__device__ __forceinline__ int xcd_group_remap(int pid, int total, int gsize) {
  const int full = total / (8 * gsize) * (8 * gsize);
  if (pid >= full) return pid;
  const int x = pid % 8, k = pid / 8;
  return (8 * (k / gsize) + x) * gsize + k % gsize;
}

}  // namespace sage
