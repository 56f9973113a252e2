// attn_common.hpp -- device helpers shared by the gfx950 attention kernels.
//
// Matrix-core layout facts used throughout (v_mfma_f32_32x32x16_bf16, one
// wave64; h = lane / 32):
//   A operand (32 x 16): lane holds A[lane % 32][8h + e], e = 0..7
//   B operand (16 x 32): lane holds B[8h + e][lane % 32]
//   C/D       (32 x 32): lane holds D[8 (r / 4) + 4h + (r % 4)][lane % 32], r = 0..15
// Only the pairing of A's and B's reduction index matters for a product, so a
// kernel may assign any physical index to the logical slot (h, e) as long as
// both operands use the same assignment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSub = 32;  // rows of one query sub-block = side of one MFMA output tile

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16: A lane holds A[lane % 16][8 (lane / 16) + e],
// B lane holds B[8 (lane / 16) + e][lane % 16], D lane holds
// D[4 (lane / 16) + r][lane % 16], r = 0..3.
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row sums on the matrix cores.  A bf16x8 operand laid out for the 32x32x16
// product with lane = query (lane % 32) and 8 keys per lane, read as the B
// operand of the 16x16x32 product, puts query 16 (g & 1) + n in column n of
// lane group g = lane / 16.  Against this selector as A (1 where bit 2 of the
// row matches bit 0 of the lane group), row m of column n sums the 16 keys of
// query 16 ((m >> 2) & 1) + n, so every element a lane receives in D is the
// key sum of its own query lane % 32.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
  const __bf16 v = (__bf16)((((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = v;
  return a;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 of two values, packed low/high (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Eight fp32 values -> one bf16x8 operand (element e from v[e]).
__device__ __forceinline__ bf16x8 to_bf16x8(float v0, float v1, float v2, float v3, float v4,
                                            float v5, float v6, float v7) {
  u32x4 u;
  u[0] = pack_bf16x2(v0, v1);
  u[1] = pack_bf16x2(v2, v3);
  u[2] = pack_bf16x2(v4, v5);
  u[3] = pack_bf16x2(v6, v7);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x as a bf16 pair: low half the rounded value, high half the rounding
// residual, also rounded.  Their fp32 sum restores x to about 2^-17 relative.
__device__ __forceinline__ uint32_t split2_bf16(float x) {
  const uint32_t hi = pack_bf16x2(x, 0.0f);
  const uint32_t lo = pack_bf16x2(x - __uint_as_float(hi << 16), 0.0f);
  return hi | (lo << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Exchange a value with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// The values a lane pair (l, l^32) holds, in half order, on both lanes:
// .h0 from the lane in the lower half, .h1 from the lane in the upper half.
// One v_permlane32_swap: it exchanges the upper half of its first operand with
// the lower half of its second; fed the same value twice, the first result
// holds the lower-half values in both halves and the second the upper-half
// values.
struct HalfPair {
  float h0, h1;
};
__device__ __forceinline__ HalfPair halves(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float both_halves_max(float x) {
  const HalfPair p = halves(x);
  return fmaxf(p.h0, p.h1);
}
__device__ __forceinline__ float both_halves_sum(float x) {
  const HalfPair p = halves(x);
  return p.h0 + p.h1;
}

// Buffer resource over `bytes` bytes starting at `base` (raw buffer, 32-bit
// data format).  The hardware range check makes every load at a byte offset
// at or past `bytes` return zeros, so a tile running off the end of a
// sequence needs no mask, clamp or branch; the offsets stay 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
// A byte offset past every range make_rsrc is given (those stay below 2^31
// bytes): a load there returns zeros, the usual way to mask single lanes of a
// buffer load.
constexpr uint32_t kNoOffset = 0x80000000u;
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voffset, 0, 0));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace attn
