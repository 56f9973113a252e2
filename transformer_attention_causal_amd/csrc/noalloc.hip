// noalloc.hip -- attn_fwd_noalloc: the forward pass with its dilution
// workspace in a fixed device array owned by the library, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in this file.  Each GPU the library runs on holds its own
// copy from the time the code object is loaded until the process ends.  The
// array's name is only a host-side stand-in for it: its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device at the
// first call there and kept, and that address is what the kernels receive.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "launch.hpp"

namespace {

// The dilution workspace: per query row one fp32 log-sum-exp, per (32-row
// query block, earlier key) one 32-bit committed-demand entry, and on small
// grids the key-range partials.  128 MiB holds B*H = 16 heads at T = 8192,
// d = 64 or 128 (about 68 MB).  No kernel needs any of it cleared: every
// entry is written before it is read within one call.
constexpr size_t kScratchBytes = size_t(128) << 20;
static_assert(kScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "header and library disagree");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The scratch array's device address on the current device (NULL on error).
void *scratch_on_current_device(hipError_t *err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  *err = g_err[dev];
  return g_ptr[dev];
}

}  // namespace

extern "C" {

int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int B, int H, int T,
                     int d, float tau, int mode, float eps, int dtype, void *hip_stream) {
  // every argument check comes before any device call
  const int st = attn::validate_fwd(q, k, v, out, B, H, T, d, tau, mode, eps, dtype);
  if (st != ATTN_OK) return st;
  if (mode == ATTN_TEMPERED)   // needs no workspace
    return attn_fwd(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, nullptr, 0, hip_stream);
  const size_t need = attn_fwd_workspace_bytes(B, H, T, d, mode, dtype);
  if (need == 0) return ATTN_EINVAL;
  if (need > kScratchBytes) return ATTN_ESCRATCH;
  hipError_t e = hipSuccess;
  void *ws = scratch_on_current_device(&e);
  if (!ws) return attn::record_hip_error(e);
  return attn_fwd(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, ws, kScratchBytes, hip_stream);
}

}  // extern "C"
