// peaks.hip -- measured ceilings of one MI355X (gfx950) for the roofline
// figures: the bf16 matrix-core rate of a loop of independent 32x32x16 MFMAs,
// and the HBM rate of a streaming read.  Not part of the attention path:
// libattn_peaks.so is loaded by the benchmark only.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/attn_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;   // independent accumulators per wave

// Each wave issues `iters` rounds of kChains independent MFMAs; the operands
// depend on the lane so the work cannot be folded, and the result is written
// so it cannot be dropped.
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float *out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((t + e) & 7);
    b[e] = (__bf16)(float)((t * 3 + e) & 7);
  }
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += c[k][0] + c[k][15];
  out[(size_t)blockIdx.x * 256 + t] = s;
}

// Grid-stride streaming read of n 16-byte words, eight loads in flight per
// lane, non-temporal; the words are folded into one value that is written
// only if it equals a marker, so the loads stay live.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4 *__restrict__ p, size_t n,
                                                          uint32_t *out) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9e3779b9u) out[0] = acc;
}

}  // namespace

extern "C" {

int attn_peak_mfma_bf16(int iters, int workgroups, float *out, void *hip_stream) {
  if (iters <= 0 || workgroups <= 0 || !out) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(hip_stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

double attn_peak_mfma_bf16_flops(int iters, int workgroups) {
  return (double)iters * workgroups * 4 /* waves */ * kChains * (2.0 * 32 * 32 * 16);
}

int attn_peak_stream_read(const void *src, size_t bytes, uint32_t *out, int workgroups,
                          void *hip_stream) {
  if (!src || !out || bytes < 16 || workgroups <= 0 || (reinterpret_cast<uintptr_t>(src) & 15u))
    return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(hip_stream),
                     reinterpret_cast<const u32x4 *>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
