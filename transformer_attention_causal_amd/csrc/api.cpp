// api.cpp -- the extern "C" boundary of libattn.so (declared in include/attn.h).
//
// Validates arguments on the host, sizes and carves the caller's workspace,
// and enqueues the kernels on the caller's stream.  Nothing here allocates
// device memory, synchronises, throws or aborts.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

thread_local char g_hip_error[160] = "no HIP error recorded";

int fail_hip(hipError_t e) {
  std::snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s", hipGetErrorString(e));
  return ATTN_EHIP;
}

}  // namespace

namespace attn {
int record_hip_error(hipError_t e) { return fail_hip(e); }
}  // namespace attn

namespace {

// gfx950 check, once per device.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ENOTSUP;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                     std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
                        ? 1
                        : 0;
  });
  return g_dev_ok[dev] ? ATTN_OK : ATTN_ENOTSUP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Do [a, a+na) and [b, b+nb) share a byte?  A NULL pointer (an absent
// optional argument) overlaps nothing.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace layout of a dilution forward over keys 0..Tk-1 with Tq query rows
// (Tq = Tk for a whole prefill): [lse2: BH*Tq][committed demand], then, when
// the row stages split their keys (small grids), the per-range partials
// [BH*Tq*ks*2][BH*Tq*ks*d].
struct FwdWorkspace {
  int ksplit;
  size_t lse_bytes, cin_bytes, ml_bytes, o_bytes, total;
};

bool prefill_workspace(int B, int H, int Tq, int Tk, int d, int dtype, FwdWorkspace *ws) {
  const size_t BH = (size_t)B * H;
  if (BH > (size_t)INT32_MAX) return false;
  const int vrow0 = attn::first_block_row(Tk, Tq);
  ws->ksplit = attn::row_ksplit((int)BH, Tk, Tq, dtype == ATTN_BF16);
  ws->lse_bytes = round_up(BH * (size_t)Tq * sizeof(float));
  ws->cin_bytes = round_up(BH * attn::cin_floats_per_head(Tk, vrow0) * sizeof(float));
  ws->ml_bytes = ws->ksplit > 1 ? round_up(BH * (size_t)Tq * ws->ksplit * 2 * sizeof(float)) : 0;
  ws->o_bytes = ws->ksplit > 1 ? round_up(BH * (size_t)Tq * ws->ksplit * d * sizeof(float)) : 0;
  ws->total = ws->lse_bytes + ws->cin_bytes + ws->ml_bytes + ws->o_bytes;
  return true;
}

bool fwd_workspace_layout(int B, int H, int T, int d, int dtype, FwdWorkspace *ws) {
  return prefill_workspace(B, H, T, T, d, dtype, ws);
}

// Decode: chunk of keys per workgroup.
constexpr int kDecChunk = 2048;

struct DecWorkspace {
  int splits;
  size_t scores_bytes, ml_bytes, o_bytes, total;
};

bool dec_workspace(int S, int H, int Lcap, int d, DecWorkspace *ws) {
  const size_t SH = (size_t)S * H;
  if (SH > (size_t)INT32_MAX) return false;
  ws->splits = (Lcap + kDecChunk - 1) / kDecChunk;
  if (SH * (size_t)ws->splits > (size_t)INT32_MAX) return false;
  ws->scores_bytes = round_up(SH * (size_t)Lcap * sizeof(float));
  ws->ml_bytes = round_up(SH * ws->splits * 2 * sizeof(float));
  ws->o_bytes = round_up(SH * ws->splits * (size_t)(d + 1) * sizeof(float));
  ws->total = ws->scores_bytes + ws->ml_bytes + ws->o_bytes;
  return true;
}

// Head dimensions with kernels (forward, prefill, backward): 64 and 128 for
// both storage types.
bool head_dim_ok(int d, int dtype) {
  return (d == 64 || d == 128) && (dtype == ATTN_BF16 || dtype == ATTN_F32);
}

bool shape_ok(int B, int H, int T) {
  if (B <= 0 || H <= 0 || T <= 0) return false;
  if (T >= (1 << 24)) return false;
  // element counts must fit the kernels' 64-bit offsets and 32-bit grids
  const size_t BH = (size_t)B * H;
  if (BH > (size_t)INT32_MAX / 1024) return false;
  // at most 2^32 rows in all (q alone would then exceed 512 GiB, more than a
  // device holds): every launch's block count, such as B*H*ceil(T/128) or
  // B*H*T*d/256 for the per-element passes, then stays below 2^31
  if (BH * (size_t)T > ((size_t)1 << 32)) return false;
  return true;
}

// The kernels address one head's T rows of d elements with 32-bit byte
// offsets (buffer loads whose range is the bytes from a tile to the end of
// the head): T * d * element size must stay below 2^31.
bool rows_fit(int T, int d, int dtype) {
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  return (size_t)T * (size_t)d * esz <= (size_t)INT32_MAX;
}

}  // namespace

extern "C" {

size_t attn_fwd_workspace_bytes(int B, int H, int T, int d, int mode, int dtype) {
  if (!shape_ok(B, H, T) || !head_dim_ok(d, dtype) || !rows_fit(T, d, dtype)) return 0;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
  if (mode != ATTN_DILUTION) return 0;
  FwdWorkspace ws;
  if (!fwd_workspace_layout(B, H, T, d, dtype, &ws)) return 0;
  return ws.total;
}

}  // extern "C"

namespace {

// Argument checks shared by the forward entry points.  `v`/`out` may be NULL
// for the stages that do not read or write them.
int check_fwd(const void *q, const void *k, const void *v, const void *out, int B, int H, int T,
              int d, float tau, float eps, int dtype, const float *lse_out,
              const float *demand_out, const float *rowsum_out = nullptr) {
  if (!q || !k) return ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || (out && !aligned16(out)))
    return ATTN_EINVAL;
  if (!shape_ok(B, H, T)) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (!std::isfinite(tau) || tau < 0.0f) return ATTN_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f) return ATTN_EINVAL;
  if (!head_dim_ok(d, dtype)) return ATTN_ENOTSUP;
  if (!rows_fit(T, d, dtype)) return ATTN_EINVAL;
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  const size_t nbytes = (size_t)B * H * (size_t)T * d * esz;
  if (out && (overlaps(out, nbytes, q, nbytes) || overlaps(out, nbytes, k, nbytes) ||
              (v && overlaps(out, nbytes, v, nbytes))))
    return ATTN_EINVAL;
  // the optional [B,H,T] fp32 outputs may not alias any tensor argument or each other
  const size_t rbytes = (size_t)B * H * (size_t)T * sizeof(float);
  const void *rs[3] = {lse_out, demand_out, rowsum_out};
  for (int i = 0; i < 3; ++i) {
    const void *r = rs[i];
    if (!r) continue;
    if (!aligned16(r)) return ATTN_EINVAL;
    if (overlaps(r, rbytes, q, nbytes) || overlaps(r, rbytes, k, nbytes) ||
        (v && overlaps(r, rbytes, v, nbytes)) || (out && overlaps(r, rbytes, out, nbytes)))
      return ATTN_EINVAL;
    for (int j = 0; j < i; ++j)
      if (rs[j] && overlaps(r, rbytes, rs[j], rbytes)) return ATTN_EINVAL;
  }
  return ATTN_OK;
}

}  // namespace

namespace attn {
int validate_fwd(const void *q, const void *k, const void *v, const void *out, int B, int H, int T,
                 int d, float tau, int mode, float eps, int dtype) {
  if (!v || !out) return ATTN_EINVAL;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return ATTN_EINVAL;
  return check_fwd(q, k, v, out, B, H, T, d, tau, eps, dtype, nullptr, nullptr);
}
}  // namespace attn

namespace {

// The workspace is written (the row log-sum-exps and the committed-demand
// table), so it may not overlap any tensor argument or optional output; `v`,
// `out` and the row outputs may be NULL.
int check_workspace(const void *q, const void *k, const void *v, const void *out, int B, int H,
                    int T, int d, int dtype, void *workspace, size_t workspace_bytes,
                    const float *lse_out, const float *demand_out, const float *rowsum_out,
                    FwdWorkspace *ws) {
  if (!fwd_workspace_layout(B, H, T, d, dtype, ws)) return ATTN_EINVAL;
  if (!workspace || workspace_bytes < ws->total || !aligned16(workspace)) return ATTN_EWORKSPACE;
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  const size_t nbytes = (size_t)B * H * (size_t)T * d * esz;
  const size_t rbytes = (size_t)B * H * (size_t)T * sizeof(float);
  const size_t n = ws->total;
  if (overlaps(workspace, n, q, nbytes) || overlaps(workspace, n, k, nbytes) ||
      overlaps(workspace, n, v, nbytes) || overlaps(workspace, n, out, nbytes) ||
      overlaps(workspace, n, lse_out, rbytes) || overlaps(workspace, n, demand_out, rbytes) ||
      overlaps(workspace, n, rowsum_out, rbytes))
    return ATTN_EINVAL;
  return ATTN_OK;
}

attn::FwdArgs make_args(const void *q, const void *k, const void *v, void *out, int B, int H,
                        int T, int d, float tau, float eps, void *workspace,
                        const FwdWorkspace &ws) {
  attn::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.BH = B * H;
  a.T = a.Tq = a.kstride = T;
  a.vrow0 = 0;
  a.D = d;
  // logits are tau <q,k> / sqrt(d); the kernels work in base 2
  a.c2 = (float)((double)tau / std::sqrt((double)d) * 1.4426950408889634);
  a.eps = eps;
  a.ksplit = 1;
  if (workspace) {
    char *wsp = static_cast<char *>(workspace);
    a.lse2 = reinterpret_cast<float *>(wsp);
    a.cin = reinterpret_cast<float *>(wsp + ws.lse_bytes);
    if (ws.ksplit > 1) {
      a.ksplit = ws.ksplit;
      a.part_ml = reinterpret_cast<float *>(wsp + ws.lse_bytes + ws.cin_bytes);
      a.part_o = reinterpret_cast<float *>(wsp + ws.lse_bytes + ws.cin_bytes + ws.ml_bytes);
    }
  }
  return a;
}

int finish(hipError_t e) { return e == hipSuccess ? ATTN_OK : fail_hip(e); }

}  // namespace

extern "C" {

int attn_dilution_lse(const void *q, const void *k, int B, int H, int T, int d, float tau,
                      int dtype, void *workspace, size_t workspace_bytes, float *lse_out,
                      void *hip_stream) {
  int st = check_fwd(q, k, nullptr, nullptr, B, H, T, d, tau, 0.0f, dtype, lse_out, nullptr);
  FwdWorkspace ws{};
  if (st == ATTN_OK)
    st = check_workspace(q, k, nullptr, nullptr, B, H, T, d, dtype, workspace, workspace_bytes,
                         lse_out, nullptr, nullptr, &ws);
  if (st == ATTN_OK) st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a = make_args(q, k, nullptr, nullptr, B, H, T, d, tau, 0.0f, workspace, ws);
  a.lse_nat = lse_out;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  return finish(dtype == ATTN_BF16 ? attn::launch_rows_bf16(attn::kRowLse, a, s)
                                   : attn::launch_rows_f32(attn::kRowLse, a, s));
}

int attn_dilution_committed(const void *q, const void *k, int B, int H, int T, int d, float tau,
                            float eps, int dtype, void *workspace, size_t workspace_bytes,
                            float *demand_out, void *hip_stream) {
  int st = check_fwd(q, k, nullptr, nullptr, B, H, T, d, tau, eps, dtype, nullptr, demand_out);
  FwdWorkspace ws{};
  if (st == ATTN_OK)
    st = check_workspace(q, k, nullptr, nullptr, B, H, T, d, dtype, workspace, workspace_bytes,
                         nullptr, demand_out, nullptr, &ws);
  if (st == ATTN_OK) st = check_device();
  if (st != ATTN_OK) return st;
  // the table holds committed + eps: stage 3 adds no eps for these keys
  attn::FwdArgs a = make_args(q, k, nullptr, nullptr, B, H, T, d, tau, eps, workspace, ws);
  a.demand_out = demand_out;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  return finish(dtype == ATTN_BF16 ? attn::launch_colsum_bf16(a, s) : attn::launch_colsum_f32(a, s));
}

int attn_dilution_shares(const void *q, const void *k, const void *v, void *out, int B, int H,
                         int T, int d, float tau, float eps, int dtype, void *workspace,
                         size_t workspace_bytes, void *hip_stream) {
  if (!v || !out) return ATTN_EINVAL;
  int st = check_fwd(q, k, v, out, B, H, T, d, tau, eps, dtype, nullptr, nullptr);
  FwdWorkspace ws{};
  if (st == ATTN_OK)
    st = check_workspace(q, k, v, out, B, H, T, d, dtype, workspace, workspace_bytes, nullptr,
                         nullptr, nullptr, &ws);
  if (st == ATTN_OK) st = check_device();
  if (st != ATTN_OK) return st;
  attn::FwdArgs a = make_args(q, k, v, out, B, H, T, d, tau, eps, workspace, ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  return finish(dtype == ATTN_BF16 ? attn::launch_rows_bf16(attn::kRowShare, a, s)
                                   : attn::launch_rows_f32(attn::kRowShare, a, s));
}

int attn_fwd_ex(const void *q, const void *k, const void *v, void *out, int B, int H, int T,
                int d, float tau, int mode, float eps, int dtype, void *workspace,
                size_t workspace_bytes, float *lse_out, float *demand_out, float *rowsum_out,
                void *hip_stream) {
  if (!v || !out) return ATTN_EINVAL;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return ATTN_EINVAL;
  if (mode == ATTN_TEMPERED && (demand_out || rowsum_out)) return ATTN_EINVAL;
  int st = check_fwd(q, k, v, out, B, H, T, d, tau, eps, dtype, lse_out, demand_out, rowsum_out);
  if (st != ATTN_OK) return st;
  FwdWorkspace ws{};
  if (mode == ATTN_DILUTION) {
    st = check_workspace(q, k, v, out, B, H, T, d, dtype, workspace, workspace_bytes, lse_out,
                         demand_out, rowsum_out, &ws);
    if (st != ATTN_OK) return st;
  }
  st = check_device();
  if (st != ATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool bf16 = dtype == ATTN_BF16;
  if (mode == ATTN_TEMPERED) {
    attn::FwdArgs a = make_args(q, k, v, out, B, H, T, d, tau, eps, nullptr, ws);
    a.lse_nat = lse_out;
    return finish(bf16 ? attn::launch_rows_bf16(attn::kRowTempered, a, s)
                       : attn::launch_rows_f32(attn::kRowTempered, a, s));
  }
  attn::FwdArgs a = make_args(q, k, v, out, B, H, T, d, tau, eps, workspace, ws);
  // stage 1: row log-sum-exp (and the optional natural-log copy)
  a.lse_nat = lse_out;
  hipError_t e = bf16 ? attn::launch_rows_bf16(attn::kRowLse, a, s)
                      : attn::launch_rows_f32(attn::kRowLse, a, s);
  if (e != hipSuccess) return fail_hip(e);
  a.lse_nat = nullptr;
  // stage 2: demand committed before each 32-row query block
  a.demand_out = demand_out;
  e = bf16 ? attn::launch_colsum_bf16(a, s) : attn::launch_colsum_f32(a, s);
  if (e != hipSuccess) return fail_hip(e);
  a.demand_out = nullptr;
  // stage 3: shares, share@V, renormalisation
  a.rowsum_out = rowsum_out;
  return finish(bf16 ? attn::launch_rows_bf16(attn::kRowShare, a, s)
                     : attn::launch_rows_f32(attn::kRowShare, a, s));
}

int attn_fwd(const void *q, const void *k, const void *v, void *out, int B, int H, int T, int d,
             float tau, int mode, float eps, int dtype, void *workspace, size_t workspace_bytes,
             void *hip_stream) {
  return attn_fwd_ex(q, k, v, out, B, H, T, d, tau, mode, eps, dtype, workspace, workspace_bytes,
                     nullptr, nullptr, nullptr, hip_stream);
}

size_t attn_prefill_workspace_bytes(int B, int H, int Tq, int Tk, int d, int mode, int dtype) {
  if (!shape_ok(B, H, Tk) || Tq < 1 || Tq > Tk || !head_dim_ok(d, dtype)) return 0;
  if (!rows_fit(Tk, d, dtype)) return 0;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
  if (mode != ATTN_DILUTION) return 0;
  FwdWorkspace ws;
  if (!prefill_workspace(B, H, Tq, Tk, d, dtype, &ws)) return 0;
  return ws.total;
}

}  // extern "C"

namespace {

// The rotated rows of a prefill with rotary position embedding: Q [B,H,Tq,d]
// and the cache's first Tk keys at the cache's stride [B,H,Lcap,d], in the
// storage type, ahead of the attention workspace.
struct RopeWorkspace {
  size_t q_bytes, k_bytes, total;
};

bool rope_workspace(int B, int H, int Tq, int Lcap, int d, int dtype, RopeWorkspace *rw) {
  const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
  rw->q_bytes = round_up((size_t)B * H * (size_t)Tq * d * esz);
  rw->k_bytes = round_up((size_t)B * H * (size_t)Lcap * d * esz);
  rw->total = rw->q_bytes + rw->k_bytes;
  return true;
}

// attn_prefill and attn_prefill_rope.  With rope_freq, Q and the keys are
// rotated into the head of the workspace first and the attention kernels
// read them from there; the attention workspace follows.
int prefill_common(const void *q, const void *kcache, const void *vcache, void *out, int B, int H,
                   int Tq, int Tk, int Lcap, int d, float tau, const float *tau_bh, int mode,
                   float eps, int dtype, const float *rope_freq, int pos0,
                   const float *demand_in, float *demand_out, float *lse_out, float *rowsum_out,
                   void *workspace, size_t workspace_bytes, void *hip_stream) {

  if (!q || !kcache || !vcache || !out) return ATTN_EINVAL;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return ATTN_EINVAL;
  if (mode == ATTN_TEMPERED && (demand_in || demand_out || rowsum_out)) return ATTN_EINVAL;
  if (!shape_ok(B, H, Lcap) || Tq < 1 || Tk < Tq || Lcap < Tk) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (!std::isfinite(tau) || tau < 0.0f) return ATTN_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f) return ATTN_EINVAL;
  if (!head_dim_ok(d, dtype)) return ATTN_ENOTSUP;
  if (!rows_fit(Lcap, d, dtype)) return ATTN_EINVAL;
  const void *ptrs[9] = {q, kcache, vcache, out, demand_in, demand_out, lse_out, rowsum_out, tau_bh};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return ATTN_EINVAL;
  const size_t BH = (size_t)B * H, esz = dtype == ATTN_BF16 ? 2 : 4;
  const size_t qbytes = BH * Tq * d * esz, cbytes = BH * (size_t)Lcap * d * esz;
  const size_t rbytes = BH * Tq * sizeof(float), dbytes = BH * (size_t)Lcap * sizeof(float);
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, kcache, cbytes) ||
      overlaps(out, qbytes, vcache, cbytes))
    return ATTN_EINVAL;
  // every fp32 output is disjoint from the tensors and the other outputs;
  // demand_out may be demand_in itself (an in-place update) but no partial overlap
  auto hits_tensor = [&](const void *p, size_t n) {
    return overlaps(p, n, q, qbytes) || overlaps(p, n, kcache, cbytes) ||
           overlaps(p, n, vcache, cbytes) || overlaps(p, n, out, qbytes);
  };
  if (hits_tensor(lse_out, rbytes) || hits_tensor(rowsum_out, rbytes) ||
      hits_tensor(demand_out, dbytes))
    return ATTN_EINVAL;
  if (overlaps(lse_out, rbytes, demand_out, dbytes) || overlaps(lse_out, rbytes, rowsum_out, rbytes) ||
      overlaps(rowsum_out, rbytes, demand_out, dbytes))
    return ATTN_EINVAL;
  if (overlaps(demand_in, dbytes, lse_out, rbytes) || overlaps(demand_in, dbytes, rowsum_out, rbytes))
    return ATTN_EINVAL;
  if (overlaps(demand_in, dbytes, out, qbytes)) return ATTN_EINVAL;
  const size_t tbytes = BH * sizeof(float);
  if (tau_bh && (hits_tensor(tau_bh, tbytes) || overlaps(tau_bh, tbytes, lse_out, rbytes) ||
                 overlaps(tau_bh, tbytes, rowsum_out, rbytes) ||
                 overlaps(tau_bh, tbytes, demand_out, dbytes)))
    return ATTN_EINVAL;
  if (demand_in && demand_out && demand_in != demand_out &&
      overlaps(demand_in, dbytes, demand_out, dbytes))
    return ATTN_EINVAL;
  if (rope_freq) {
    if ((reinterpret_cast<uintptr_t>(rope_freq) & 3u) != 0) return ATTN_EINVAL;
    if (pos0 < 0 || (long)pos0 + Tk > (long)INT32_MAX) return ATTN_EINVAL;
    const size_t fbytes = (size_t)(d / 2) * sizeof(float);
    if (hits_tensor(rope_freq, fbytes) || overlaps(rope_freq, fbytes, lse_out, rbytes) ||
        overlaps(rope_freq, fbytes, rowsum_out, rbytes) ||
        overlaps(rope_freq, fbytes, demand_out, dbytes))
      return ATTN_EINVAL;
  }
  RopeWorkspace rw{};
  if (rope_freq) rope_workspace(B, H, Tq, Lcap, d, dtype, &rw);
  FwdWorkspace ws{};
  size_t need = rw.total;
  if (mode == ATTN_DILUTION) {
    if (!prefill_workspace(B, H, Tq, Tk, d, dtype, &ws)) return ATTN_EINVAL;
    need += ws.total;
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ATTN_EWORKSPACE;
    // the workspace is written: it may not overlap any argument
    if (hits_tensor(workspace, need) || overlaps(workspace, need, lse_out, rbytes) ||
        overlaps(workspace, need, rowsum_out, rbytes) ||
        overlaps(workspace, need, demand_out, dbytes) ||
        overlaps(workspace, need, demand_in, dbytes) ||
        overlaps(workspace, need, tau_bh, BH * sizeof(float)) ||
        overlaps(workspace, need, rope_freq, (size_t)(d / 2) * sizeof(float)))
      return ATTN_EINVAL;
  }
  int st = check_device();
  if (st != ATTN_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool bf16 = dtype == ATTN_BF16;
  char *attn_ws = workspace ? static_cast<char *>(workspace) + rw.total : nullptr;
  if (rope_freq) {
    // rotate the chunk's query rows (positions pos0 + P ..) and the keys
    // (positions pos0 ..) into the workspace; the kernels read those
    char *wq = static_cast<char *>(workspace), *wk = wq + rw.q_bytes;
    attn::RopeArgs r{};
    r.BH = (int)BH;
    r.D = d;
    r.freq = rope_freq;
    r.x = q;
    r.y = wq;
    r.rows = Tq;
    r.in_stride = r.out_stride = (size_t)Tq;
    r.pos0 = (long)pos0 + (Tk - Tq);
    hipError_t e = attn::launch_rope(r, bf16, s);
    if (e != hipSuccess) return fail_hip(e);
    r.x = kcache;
    r.y = wk;
    r.rows = Tk;
    r.in_stride = r.out_stride = (size_t)Lcap;
    r.pos0 = pos0;
    e = attn::launch_rope(r, bf16, s);
    if (e != hipSuccess) return fail_hip(e);
    q = wq;
    kcache = wk;
  }
  attn::FwdArgs a = make_args(q, kcache, vcache, out, B, H, Tk, d, tau, eps,
                              mode == ATTN_DILUTION ? attn_ws : nullptr, ws);
  a.Tq = Tq;
  a.kstride = Lcap;
  a.vrow0 = attn::first_block_row(Tk, Tq);
  if (tau_bh) {
    // the kernels scale by tau_bh[bh] * log2(e) / sqrt(d)
    a.tau_bh = tau_bh;
    a.c2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  }
  a.lse_nat = lse_out;
  if (mode == ATTN_TEMPERED)
    return finish(bf16 ? attn::launch_rows_bf16(attn::kRowTempered, a, s)
                       : attn::launch_rows_f32(attn::kRowTempered, a, s));
  hipError_t e = bf16 ? attn::launch_rows_bf16(attn::kRowLse, a, s)
                      : attn::launch_rows_f32(attn::kRowLse, a, s);
  if (e != hipSuccess) return fail_hip(e);
  a.lse_nat = nullptr;
  a.demand_in = demand_in;
  a.demand_out = demand_out;
  e = bf16 ? attn::launch_colsum_bf16(a, s) : attn::launch_colsum_f32(a, s);
  if (e != hipSuccess) return fail_hip(e);
  a.demand_in = nullptr;
  a.demand_out = nullptr;
  a.rowsum_out = rowsum_out;
  return finish(bf16 ? attn::launch_rows_bf16(attn::kRowShare, a, s)
                     : attn::launch_rows_f32(attn::kRowShare, a, s));
}

}  // namespace

extern "C" {

int attn_prefill(const void *q, const void *kcache, const void *vcache, void *out, int B, int H,
                 int Tq, int Tk, int Lcap, int d, float tau, const float *tau_bh, int mode,
                 float eps, int dtype, const float *demand_in, float *demand_out, float *lse_out,
                 float *rowsum_out, void *workspace, size_t workspace_bytes, void *hip_stream) {
  return prefill_common(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh, mode, eps,
                        dtype, nullptr, 0, demand_in, demand_out, lse_out, rowsum_out, workspace,
                        workspace_bytes, hip_stream);
}

size_t attn_prefill_rope_workspace_bytes(int B, int H, int Tq, int Tk, int Lcap, int d, int mode,
                                         int dtype) {
  if (!shape_ok(B, H, Lcap) || Tq < 1 || Tq > Tk || Tk > Lcap || !head_dim_ok(d, dtype)) return 0;
  if (!rows_fit(Lcap, d, dtype)) return 0;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return 0;
  RopeWorkspace rw;
  rope_workspace(B, H, Tq, Lcap, d, dtype, &rw);
  size_t total = rw.total;
  if (mode == ATTN_DILUTION) {
    FwdWorkspace ws;
    if (!prefill_workspace(B, H, Tq, Tk, d, dtype, &ws)) return 0;
    total += ws.total;
  }
  return total;
}

int attn_prefill_rope(const void *q, const void *kcache, const void *vcache, void *out, int B,
                      int H, int Tq, int Tk, int Lcap, int d, float tau, const float *tau_bh,
                      int mode, float eps, int dtype, const float *rope_freq, int pos0,
                      const float *demand_in, float *demand_out, float *lse_out,
                      float *rowsum_out, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
  if (!rope_freq) return ATTN_EINVAL;
  return prefill_common(q, kcache, vcache, out, B, H, Tq, Tk, Lcap, d, tau, tau_bh, mode, eps,
                        dtype, rope_freq, pos0, demand_in, demand_out, lse_out, rowsum_out,
                        workspace, workspace_bytes, hip_stream);
}

}  // extern "C"

namespace {

// Workspace layout of a backward pass: per-row fp32 arrays (lse2, 1/r,
// delta/r, rho, then <q_i, dQ_i / c> in one partial sum per slice of d that
// the dq kernel splits the head dimension into), then for dilution the
// committed demand and the later blocks' gradient sums, per (32-row block,
// key); for fp32 the [B,H,T,d] softmax-weighted keys; for bf16 the fp32
// [B,H,T,d] partial key gradients sum_i p_ij dp_ij q_i and, per row, each
// 128-key block's part of rho ([B*H][ceil(T/128)][T] fp32).
constexpr size_t kBwdFixedRowArrays = 4;
struct BwdWorkspace {
  int tslices;
  size_t row_bytes, cin_bytes, gin_bytes, pk_bytes, dkp_bytes, rhop_bytes, total;
};

// Per-row partial sums of the rows' dL/dtau terms: every dq kernel covers all
// of d in one workgroup, so one.
int bwd_tslices(int, int) { return 1; }

bool bwd_workspace(int B, int H, int T, int d, int mode, int dtype, BwdWorkspace *ws) {
  const size_t BH = (size_t)B * H;
  if (BH > (size_t)INT32_MAX) return false;
  ws->tslices = bwd_tslices(d, dtype);
  ws->row_bytes = round_up(BH * (size_t)T * sizeof(float));
  ws->cin_bytes = mode == ATTN_DILUTION ? round_up(BH * attn::cin_floats_per_head(T, 0) * 4) : 0;
  ws->gin_bytes = mode == ATTN_DILUTION ? round_up(BH * attn::gin_floats_per_head(T) * 4) : 0;
  const bool dil = mode == ATTN_DILUTION, bf16 = dtype == ATTN_BF16;
  const size_t nkb = ((size_t)T + 127) / 128;
  ws->pk_bytes = dil && !bf16 ? round_up(BH * (size_t)T * d * sizeof(float)) : 0;
  ws->dkp_bytes = dil && bf16 ? round_up(BH * (size_t)T * d * sizeof(float)) : 0;
  ws->rhop_bytes = dil && bf16 ? round_up(BH * nkb * (size_t)T * sizeof(float)) : 0;
  ws->total = (kBwdFixedRowArrays + ws->tslices) * ws->row_bytes + ws->cin_bytes + ws->gin_bytes +
              ws->pk_bytes + ws->dkp_bytes + ws->rhop_bytes;
  return true;
}

}  // namespace

extern "C" {

size_t attn_bwd_workspace_bytes(int B, int H, int T, int d, int mode, int dtype) {
  if (!shape_ok(B, H, T) || (dtype != ATTN_BF16 && dtype != ATTN_F32)) return 0;
  if (!head_dim_ok(d, dtype) || !rows_fit(T, d, dtype)) return 0;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return 0;
  BwdWorkspace ws;
  if (!bwd_workspace(B, H, T, d, mode, dtype, &ws)) return 0;
  return ws.total;
}

int attn_bwd_ex(const void *q, const void *k, const void *v, const void *out, const void *dout,
                const float *lse, const float *rowsum, void *dq, void *dk, void *dv, int B, int H,
                int T, int d, float tau, const float *tau_bh, int mode, float eps, int dtype,
                float *dtau_out, const void *fwd_workspace, size_t fwd_workspace_bytes,
                void *workspace, size_t workspace_bytes, void *hip_stream) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv) return ATTN_EINVAL;
  if (mode != ATTN_TEMPERED && mode != ATTN_DILUTION) return ATTN_EINVAL;
  if (mode == ATTN_DILUTION && !rowsum) return ATTN_EINVAL;
  const void *ptrs[9] = {q, k, v, out, dout, lse, dq, dk, dv};
  for (const void *p : ptrs)
    if (!aligned16(p)) return ATTN_EINVAL;
  if (rowsum && !aligned16(rowsum)) return ATTN_EINVAL;
  if ((tau_bh && !aligned16(tau_bh)) || (dtau_out && !aligned16(dtau_out))) return ATTN_EINVAL;
  if (!shape_ok(B, H, T)) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (!std::isfinite(tau) || tau < 0.0f) return ATTN_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f) return ATTN_EINVAL;
  if (!head_dim_ok(d, dtype)) return ATTN_ENOTSUP;
  if (!rows_fit(T, d, dtype)) return ATTN_EINVAL;
  // the three gradients may not alias each other or any input
  const size_t nbytes = (size_t)B * H * (size_t)T * d * (dtype == ATTN_BF16 ? 2 : 4);
  const size_t rbytes = (size_t)B * H * (size_t)T * sizeof(float);
  const void *grads[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (const void *in : {q, k, v, out, dout})
      if (overlaps(grads[i], nbytes, in, nbytes)) return ATTN_EINVAL;
    if (overlaps(grads[i], nbytes, lse, rbytes) || (rowsum && overlaps(grads[i], nbytes, rowsum, rbytes)))
      return ATTN_EINVAL;
    for (int j = 0; j < i; ++j)
      if (overlaps(grads[i], nbytes, grads[j], nbytes)) return ATTN_EINVAL;
  }
  const size_t tbytes = (size_t)B * H * sizeof(float);
  if (tau_bh)
    for (const void *g : grads)
      if (overlaps(g, nbytes, tau_bh, tbytes)) return ATTN_EINVAL;
  if (dtau_out) {
    const void *tensors[8] = {q, k, v, out, dout, dq, dk, dv};
    for (const void *in : tensors)
      if (overlaps(dtau_out, tbytes, in, nbytes)) return ATTN_EINVAL;
    if (overlaps(dtau_out, tbytes, lse, rbytes) ||
        (rowsum && overlaps(dtau_out, tbytes, rowsum, rbytes)) ||
        (tau_bh && overlaps(dtau_out, tbytes, tau_bh, tbytes)))
      return ATTN_EINVAL;
  }
  BwdWorkspace ws;
  if (!bwd_workspace(B, H, T, d, mode, dtype, &ws)) return ATTN_EINVAL;
  if (!workspace || workspace_bytes < ws.total || !aligned16(workspace)) return ATTN_EWORKSPACE;
  // the workspace is written: it may not overlap any argument
  {
    const void *tensors[8] = {q, k, v, out, dout, dq, dk, dv};
    for (const void *t : tensors)
      if (overlaps(workspace, ws.total, t, nbytes)) return ATTN_EINVAL;
    if (overlaps(workspace, ws.total, lse, rbytes) || overlaps(workspace, ws.total, rowsum, rbytes) ||
        overlaps(workspace, ws.total, tau_bh, tbytes) ||
        overlaps(workspace, ws.total, dtau_out, tbytes))
      return ATTN_EINVAL;
  }
  // the dilution forward's workspace (read only): its committed-demand table
  // replaces the backward's own; ignored for ATTN_TEMPERED
  const char *fwd_cin = nullptr;
  if (fwd_workspace && mode == ATTN_DILUTION) {
    FwdWorkspace fw;
    if (!fwd_workspace_layout(B, H, T, d, dtype, &fw)) return ATTN_EINVAL;
    if (fwd_workspace_bytes < fw.total || !aligned16(fwd_workspace)) return ATTN_EWORKSPACE;
    const size_t fbytes = fw.total;
    for (const void *g : grads)
      if (overlaps(g, nbytes, fwd_workspace, fbytes)) return ATTN_EINVAL;
    if (overlaps(workspace, ws.total, fwd_workspace, fbytes) ||
        overlaps(dtau_out, tbytes, fwd_workspace, fbytes))
      return ATTN_EINVAL;
    fwd_cin = static_cast<const char *>(fwd_workspace) + fw.lse_bytes;
  }
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;

  attn::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.dout = dout;
  a.lse = lse;
  a.rowsum = rowsum;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  char *wsp = static_cast<char *>(workspace);
  a.lse2 = reinterpret_cast<float *>(wsp);
  a.invr = reinterpret_cast<float *>(wsp + ws.row_bytes);
  a.dri = reinterpret_cast<float *>(wsp + 2 * ws.row_bytes);
  a.rho = reinterpret_cast<float *>(wsp + 3 * ws.row_bytes);
  a.trow = reinterpret_cast<float *>(wsp + kBwdFixedRowArrays * ws.row_bytes);
  a.tslices = ws.tslices;
  char *wtail = wsp + (kBwdFixedRowArrays + ws.tslices) * ws.row_bytes;
  if (mode == ATTN_DILUTION) {
    // the kernels only read the table when the forward's is given
    a.cin = fwd_cin ? reinterpret_cast<float *>(const_cast<char *>(fwd_cin))
                    : reinterpret_cast<float *>(wtail);
    a.cin_given = fwd_cin ? 1 : 0;
    a.gin = reinterpret_cast<float *>(wtail + ws.cin_bytes);
    char *wt = wtail + ws.cin_bytes + ws.gin_bytes;
    if (ws.pk_bytes) a.pk = wt;
    wt += ws.pk_bytes;
    if (ws.dkp_bytes) a.dkp = reinterpret_cast<float *>(wt);
    wt += ws.dkp_bytes;
    if (ws.rhop_bytes) a.rhop = reinterpret_cast<float *>(wt);
  }
  a.BH = B * H;
  a.T = T;
  a.D = d;
  const double rsd = 1.0 / std::sqrt((double)d);
  // with tau_bh the kernels multiply c and c2 by head bh's multiplier
  const double c = tau_bh ? rsd : (double)tau * rsd;
  a.c = (float)c;
  a.c2 = (float)(c * 1.4426950408889634);
  a.rsd = (float)rsd;
  a.tau_bh = tau_bh;
  a.dtau = dtau_out;
  a.eps = eps;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  hipError_t e = dtype == ATTN_BF16 ? attn::launch_bwd_bf16(mode, a, s)
                                    : attn::launch_bwd_f32(mode, a, s);
  return e == hipSuccess ? ATTN_OK : fail_hip(e);
}

int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
             const float *lse, const float *rowsum, void *dq, void *dk, void *dv, int B, int H,
             int T, int d, float tau, int mode, float eps, int dtype, void *workspace,
             size_t workspace_bytes, void *hip_stream) {
  return attn_bwd_ex(q, k, v, out, dout, lse, rowsum, dq, dk, dv, B, H, T, d, tau, nullptr, mode,
                     eps, dtype, nullptr, nullptr, 0, workspace, workspace_bytes, hip_stream);
}

size_t attn_decode_workspace_bytes(int S, int H, int Lcap, int d) {
  if (S <= 0 || H <= 0 || Lcap <= 0 || (d != 64 && d != 128)) return 0;
  DecWorkspace ws;
  if (!dec_workspace(S, H, Lcap, d, &ws)) return 0;
  return ws.total;
}

int attn_decode_ex(const void *q, const void *kcache, const void *vcache, float *demand, void *out,
                   int S, int H, int Lcap, const int32_t *kv_len, int d, float tau,
                   const float *tau_sh, float eps, int dtype, void *workspace,
                   size_t workspace_bytes, void *hip_stream) {
  if (!q || !kcache || !vcache || !demand || !out) return ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(demand) ||
      !aligned16(out) || (tau_sh && !aligned16(tau_sh)))
    return ATTN_EINVAL;
  if (S <= 0 || H <= 0 || Lcap <= 0) return ATTN_EINVAL;
  if (!std::isfinite(tau) || tau < 0.0f) return ATTN_EINVAL;
  if (!std::isfinite(eps) || eps < 0.0f) return ATTN_EINVAL;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if ((d != 64 && d != 128) || dtype != ATTN_BF16) return ATTN_ENOTSUP;
  DecWorkspace ws;
  if (!dec_workspace(S, H, Lcap, d, &ws)) return ATTN_EINVAL;
  const size_t cache_bytes = (size_t)S * H * (size_t)Lcap * d * 2;
  const size_t out_bytes = (size_t)S * H * d * 2;
  const size_t dem_bytes = (size_t)S * H * (size_t)Lcap * 4;
  if (overlaps(out, out_bytes, kcache, cache_bytes) || overlaps(out, out_bytes, vcache, cache_bytes) ||
      overlaps(out, out_bytes, demand, dem_bytes) || overlaps(out, out_bytes, q, out_bytes) ||
      overlaps(demand, dem_bytes, kcache, cache_bytes) ||
      overlaps(demand, dem_bytes, vcache, cache_bytes) || overlaps(demand, dem_bytes, q, out_bytes))
    return ATTN_EINVAL;
  const size_t tau_bytes = (size_t)S * H * 4;
  if (tau_sh && (overlaps(tau_sh, tau_bytes, out, out_bytes) || overlaps(tau_sh, tau_bytes, demand, dem_bytes)))
    return ATTN_EINVAL;
  if (!workspace || workspace_bytes < ws.total || !aligned16(workspace)) return ATTN_EWORKSPACE;
  // the workspace is written (scores and per-chunk partials): it may not
  // overlap any argument
  if (overlaps(workspace, ws.total, q, out_bytes) || overlaps(workspace, ws.total, kcache, cache_bytes) ||
      overlaps(workspace, ws.total, vcache, cache_bytes) ||
      overlaps(workspace, ws.total, demand, dem_bytes) || overlaps(workspace, ws.total, out, out_bytes) ||
      overlaps(workspace, ws.total, tau_sh, tau_bytes) ||
      overlaps(workspace, ws.total, kv_len, (size_t)S * sizeof(int32_t)))
    return ATTN_EINVAL;
  const int dev_status = check_device();
  if (dev_status != ATTN_OK) return dev_status;

  attn::DecodeArgs a{};
  a.q = q;
  a.kc = kcache;
  a.vc = vcache;
  a.demand = demand;
  a.out = out;
  a.kv_len = kv_len;
  a.S = S;
  a.H = H;
  a.Lcap = Lcap;
  a.splits = ws.splits;
  a.chunk = kDecChunk;
  a.D = d;
  a.tau_sh = tau_sh;
  // logits in base 2: tau <q,k> / sqrt(d) * log2(e); with tau_sh the kernels
  // multiply by tau_sh[s*H+h] themselves
  a.c2 = (float)((tau_sh ? 1.0 : (double)tau) / std::sqrt((double)d) * 1.4426950408889634);
  a.eps = eps;
  char *wsp = static_cast<char *>(workspace);
  a.scores = reinterpret_cast<float *>(wsp);
  a.part_ml = reinterpret_cast<float *>(wsp + ws.scores_bytes);
  a.part_o = reinterpret_cast<float *>(wsp + ws.scores_bytes + ws.ml_bytes);
  hipError_t e = attn::launch_decode(a, reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ATTN_OK : fail_hip(e);
}

int attn_decode(const void *q, const void *kcache, const void *vcache, float *demand, void *out,
                int S, int H, int Lcap, const int32_t *kv_len, int d, float tau, float eps,
                int dtype, void *workspace, size_t workspace_bytes, void *hip_stream) {
  return attn_decode_ex(q, kcache, vcache, demand, out, S, H, Lcap, kv_len, d, tau, nullptr, eps,
                        dtype, workspace, workspace_bytes, hip_stream);
}

double attn_yarn_tau(double s) {
  if (!(s >= 1.0)) return std::nan("");
  return std::sqrt(0.1 * std::log(s) + 1.0);
}

const char *attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_ENOTSUP:
      return "unsupported (head dim must be 64 or 128; decode needs bf16 storage; device must be "
             "gfx950)";
    case ATTN_EWORKSPACE: return "workspace missing, misaligned or too small";
    case ATTN_EHIP: return g_hip_error;
    case ATTN_ESCRATCH:
      return "shape needs more workspace than attn_fwd_noalloc's fixed scratch array holds "
             "(ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
