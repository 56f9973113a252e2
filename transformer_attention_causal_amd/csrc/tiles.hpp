// tiles.hpp -- LDS tile geometry and operand-fragment helpers shared by the
// bf16 forward and backward kernels (layout facts in attn_common.hpp).
#pragma once

#include "attn_common.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kBN = 64;         // keys per LDS tile (row kernels)
constexpr float kNoRow = 1e30f;            // log-sum-exp given to positions with no row

// LDS tile geometry for head dimension D (64 or 128).
template <int D>
struct Geom {
  static constexpr int kKRow = D + 8;          // K / Q rows in LDS: D bf16 + 8 pad
  static constexpr int kKTile = kBN * kKRow;   // bf16 elements per K buffer
  static constexpr int kChunks = D / 16;       // 32x32x16 MFMA steps over d
  static constexpr int kOBlocks = D / 32;      // 32-row blocks of O^T
};
constexpr int kKRow = Geom<64>::kKRow;
constexpr int kKTile = Geom<64>::kKTile;

// Query index (within a wave's 32 rows) of accumulator element r in lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Load one 16-byte chunk of row `row` of a [T][D] bf16 array; zeros for rows
// outside [0, T).
template <int D = kHeadDim>
__device__ __forceinline__ u32x4 load_row_chunk(const __bf16 *base, int row, int T, int chunk) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if ((unsigned)row < (unsigned)T) z = *reinterpret_cast<const u32x4 *>(base + (size_t)row * D + chunk * 8);
  return z;
}

// A/B operand fragment for d-chunk c of a 64-wide bf16 row held in LDS.
__device__ __forceinline__ bf16x8 lds_frag(const __bf16 *row, int c, int h) {
  return *reinterpret_cast<const bf16x8 *>(row + 16 * c + 8 * h);
}

// The dim-major (transposed) operand of a block held row-major in LDS
// (`blk`, rows of `stride` bf16), read with the transposing LDS load: lane (i = lane % 32,
// h = lane / 32) gets column c0 + i of rows r0 + 4h + {0..3} and
// r0 + 8 + 4h + {0..3}, i.e. element r of the other operand's accumulator
// order.  Each ds_read_b64_tr_b16 works on groups of 16 lanes: group lane
// 4k + m addresses row k of the four rows, columns 4m .. 4m + 3 of the
// group's 16, and lane n of the group receives column n of all four rows.
// Addresses are 8-byte aligned when c0 is a multiple of 4 and the stride a
// multiple of 4 elements.
__device__ __forceinline__ bf16x8 lds_tr_frag(const __bf16 *blk, int stride, int r0, int c0) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((address_space(3))) const __bf16 lds_bf16;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int row = r0 + 4 * (g >> 1) + (n >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (n & 3);
  lds_bf16 *p = (lds_bf16 *)(blk + row * stride + col);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 8 * stride));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  const u32x4 u = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, u);
}

// Blocks read both ways -- 16-byte row fragments (lds_frag) and the
// transposing load -- have a layout of their own per head dimension.
//  * D = 128: rows of D bf16 without padding, the 16-byte chunks of each row
//    permuted: logical chunk c of row r sits at chunk c ^ swz(r),
//    swz(r) = ((r & 3) << 2) | ((r >> 2) & 3).  With the LDS banks 256
//    bytes around (one row), sixteen consecutive rows read at one logical
//    chunk hit sixteen different 16-byte bank groups, the four rows times
//    four aligned chunks that half a wave reads with the transposing load
//    cover all 256 bytes once, and the 16-byte row stores stay
//    conflict-free.  Padding cannot serve both reads at once.
//  * D = 64: rows padded by 8 bf16, as the row-read tiles.  The row reads
//    are conflict-free, and the transposing reads meet 2-way conflicts on
//    half of their banks, which costs less there than the swizzle's address
//    arithmetic (measured).
// The permutation stays inside the row, so every access stays inside the
// block.
template <int D>
struct DualRows {
  static constexpr int kRow = D == 64 ? D + 8 : D;   // row stride, bf16
};

template <int D>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (D == 64) return c;
  else return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
}

// Element offset of (row r, element e) in such a block; e's low three bits
// stay inside the 16-byte chunk.
template <int D>
__device__ __forceinline__ int swz_off(int r, int e) {
  return r * DualRows<D>::kRow + swz_chunk<D>(r, e >> 3) * 8 + (e & 7);
}

// lds_frag for row r of such a block.
template <int D>
__device__ __forceinline__ bf16x8 lds_frag_swz(const __bf16 *blk, int r, int c, int h) {
  return *reinterpret_cast<const bf16x8 *>(blk + swz_off<D>(r, 16 * c + 8 * h));
}

// lds_tr_frag for such a block (the same lanes, rows and columns).
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_frag_swz(const __bf16 *blk, int r0, int c0) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int row = r0 + 4 * (g >> 1) + (n >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (n & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(blk + swz_off<D>(row, col)));
  const s16x4 hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(blk + swz_off<D>(row + 8, col)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  const u32x4 u = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 pack8(const float *v) {
  return to_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
}

// O^T[d][query] += V^T[d][keys of sub-tile t] * P^T[keys][query] for every
// 32-row block o[i] of d, with V^T read transposed from the row-major V
// tile (`v_lds`, rows of VR bf16).  pf0/pf1 hold keys 0..15 / 16..31 of the
// sub-tile in the accumulator-layout order.
template <int D, int VR>
__device__ __forceinline__ void pv_update_d(f32x16 *o, const __bf16 *v_lds, int t, const bf16x8 &pf0,
                                            const bf16x8 &pf1) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int i = 0; i < Geom<D>::kOBlocks; ++i)
      o[i] = mfma32(lds_tr_frag(v_lds, VR, 32 * t + 16 * c, 32 * i), c == 0 ? pf0 : pf1, o[i]);
  }
}

}  // namespace attn
