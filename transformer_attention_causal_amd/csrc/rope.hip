// rope.hip -- rotary position embedding of Q and K ahead of the attention
// kernels ("YaRN > Attention Temperature Scaling", code cell In[16]: each
// token's query and key are rotated at its position with the per-pair
// frequencies -- YaRN's gamma already applied -- before the scores are taken).
//
// Dimension pair m is (2m, 2m+1); row t of a head sits at position pos0 + t
// and its pair m turns counter-clockwise by theta = (pos0 + t) * freq[m]:
//   (a, b) -> (a cos theta - b sin theta, a sin theta + b cos theta).
// The angle is formed and reduced to [-pi, pi] in double precision (the
// product of an integer position below 2^31 and a float frequency is exact
// there), so long contexts lose nothing to the angle; sine and cosine of the
// reduced angle and the rotation are fp32; the result is rounded once to the
// storage type.
//
// One memory-bound pass over the rows: each key row is rotated once per call
// and then read by every query block, instead of being rotated again in each
// of the T/128 tile loads that read it.
#include "launch.hpp"

#include <hip/hip_runtime.h>

namespace attn {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

__device__ __forceinline__ void turn(float a, float b, double pos, float f, float &x, float &y) {
  const double th = pos * (double)f;
  const double r = th - kTwoPi * __builtin_rint(th * (1.0 / kTwoPi));
  float s, c;
  sincosf((float)r, &s, &c);
  x = __builtin_fmaf(a, c, -b * s);
  y = __builtin_fmaf(a, s, b * c);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_r __attribute__((ext_vector_type(2)));
typedef float f32x2_r __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2_r f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_r));
}

// bf16: one thread per 16-byte chunk (4 pairs) of a row.
__global__ void __launch_bounds__(256) rope_bf16_kernel(RopeArgs a) {
  const int cpr = a.D / 8;   // chunks per row
  const size_t n = (size_t)a.BH * a.rows * cpr;
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n) return;
  const int c = (int)(u % cpr);
  const size_t rr = u / cpr;
  const int row = (int)(rr % a.rows);
  const size_t bh = rr / a.rows;
  const u32x4_t in = *reinterpret_cast<const u32x4_t *>(
      reinterpret_cast<const __bf16 *>(a.x) + (bh * a.in_stride + row) * a.D + 8 * c);
  const double pos = (double)(a.pos0 + row);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(in[i] << 16), hi = __uint_as_float(in[i] & 0xffff0000u);
    float x, y;
    turn(lo, hi, pos, a.freq[4 * c + i], x, y);
    o[i] = pack2(x, y);
  }
  *reinterpret_cast<u32x4_t *>(reinterpret_cast<__bf16 *>(a.y) + (bh * a.out_stride + row) * a.D +
                               8 * c) = o;
}

// fp32: one thread per 16-byte chunk (2 pairs) of a row.
__global__ void __launch_bounds__(256) rope_f32_kernel(RopeArgs a) {
  const int cpr = a.D / 4;
  const size_t n = (size_t)a.BH * a.rows * cpr;
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= n) return;
  const int c = (int)(u % cpr);
  const size_t rr = u / cpr;
  const int row = (int)(rr % a.rows);
  const size_t bh = rr / a.rows;
  const f32x4_t in = *reinterpret_cast<const f32x4_t *>(
      reinterpret_cast<const float *>(a.x) + (bh * a.in_stride + row) * a.D + 4 * c);
  const double pos = (double)(a.pos0 + row);
  float x0, y0, x1, y1;
  turn(in[0], in[1], pos, a.freq[2 * c], x0, y0);
  turn(in[2], in[3], pos, a.freq[2 * c + 1], x1, y1);
  const f32x4_t o = {x0, y0, x1, y1};
  *reinterpret_cast<f32x4_t *>(reinterpret_cast<float *>(a.y) + (bh * a.out_stride + row) * a.D +
                               4 * c) = o;
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, int bf16, hipStream_t s) {
  const size_t n = (size_t)a.BH * a.rows * (a.D / (bf16 ? 8 : 4));
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (bf16) hipLaunchKernelGGL(rope_bf16_kernel, grid, block, 0, s, a);
  else hipLaunchKernelGGL(rope_f32_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace attn
