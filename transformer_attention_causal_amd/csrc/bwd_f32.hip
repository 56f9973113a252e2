// bwd_f32.hip -- fp32 backward kernels (vector ALU only), head dimension D =
// 64 or 128 (a template parameter of every kernel).
//
// The exact gradients of both operators, for fp32 storage where full single
// precision is required.  The chain rule is the bf16 backward's
// ("DilutionAttention v0.1.0 - results", "The operator", differentiated; the
// release trains with exact gradients, "Everything behind these charts"):
//   dsigma_ij = (dA_ij - delta_i) / r_i,  g_ij = dsigma_ij p_ij / D_ij^2,
//   dp_ij = dsigma_ij / D_ij - G_ij (G: inclusive suffix of g down column j),
//   dS_ij = p_ij (dp_ij - rho_i),  rho_i = sum_j p_ij dp_ij,
//   dQ_i = c sum_j dS_ij k_j,  dK_j = c sum_i dS_ij q_i,  dV_j = sum_i a_ij dO_i,
// and dL/dtau = sum_i <q_i, dQ_i / c> / sqrt(d) ("Learning to Focus", sec. 2.2:
// the temperature is learned).  Tempered: dS_ij = p_ij (dA_ij - delta_i).
//
// A query row (dQ) or a key column (the column passes) is owned by d/64
// lanes: one at d = 64, two at d = 128 (lanes l and l + 32), each holding 64
// dims of the row's Q and dO (or K and V) in registers and accumulating the
// gradient for those dims; dot products over d add the two lanes' halves.
// A workgroup is four such waves, and the other operand's rows stream
// through LDS in 64-row tiles that the four waves share, read as broadcasts.
// With the own rows in registers the LDS holds only the shared tiles, so a
// CU runs a wave on each of its SIMDs at d = 128 too.
//
// The denominators match the fp32 forward's exactly: D = max(committed + eps,
// FLT_MIN) + the inclusive prefix of the bids inside the 32-row query block,
// with committed read from the fp32 forward's table.  The scans inside a
// block run over lanes in the dQ kernel (shuffles across the 32 lanes of the
// block) and over the rows a lane walks in the column kernels.
#include "attn_common.hpp"
#include "launch.hpp"

#include <float.h>

namespace attn {

constexpr int kBR = 64;   // rows or keys per LDS tile
constexpr int kFWB = 4;   // waves per workgroup, sharing each LDS tile
constexpr int kWB = 64 * kFWB;   // threads per workgroup
constexpr int kDS = 64;   // dims of a row each lane holds

// Lane geometry for head dimension D: kL lanes per row (or key), each with
// kDS dims; kPer rows per wave; kRows rows per workgroup.
template <int D>
struct LaneGeomF32 {
  static constexpr int kL = D / kDS;
  static constexpr int kPer = 64 / kL;
  static constexpr int kRows = kPer * kFWB;
};

// The full dot product from the kL lanes' parts (lanes l and l + 32).
template <int D>
__device__ __forceinline__ float row_dot(float part) {
  if constexpr (D > kDS) return both_halves_sum(part);
  return part;
}

constexpr float kInvDMaxF32 = 18446744073709551616.0f;   // 2^64: 1/D clamp (eps = 0 only)
constexpr float kNoRowBwdF32 = 1e30f;                    // lse2 of a position past T

__device__ __forceinline__ float head_tau_f32(const BwdArgs &a, int bh) {
  return a.tau_bh ? a.tau_bh[bh] : 1.0f;
}

// <x, y> over D elements (global memory), associated as the kernels'
// row_dot forms it: one fma chain per kDS dims, the chains' sums added, so
// that delta_i and <dO_i, v_j> round alike (with o_i = v_j, at T = 1, they
// are equal and dS vanishes exactly).
template <int D>
__device__ __forceinline__ float dotd(const float *x, const float *y) {
  float total = 0.0f;
#pragma unroll
  for (int e0 = 0; e0 < D; e0 += kDS) {
    float s = 0.0f;
#pragma unroll 16
    for (int e = e0; e < e0 + kDS; ++e) s = __builtin_fmaf(x[e], y[e], s);
    total = e0 == 0 ? s : total + s;
  }
  return total;
}

// <x, y> over kDS dims, x in LDS (read as a broadcast) and y this lane's
// part of its row in registers; one fma chain, element 0 first.  A
// scheduling barrier after every 32 elements keeps the compiler from
// hoisting all the LDS reads ahead of the chain (which needs many registers
// beside the own rows).
__device__ __forceinline__ float dot_lr(const float *x, const float (&y)[kDS]) {
  float s = 0.0f;
#pragma unroll
  for (int e0 = 0; e0 < kDS; e0 += 32) {
#pragma unroll
    for (int e = e0; e < e0 + 32; ++e) s = __builtin_fmaf(x[e], y[e], s);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// acc[e] += w * row[e] over kDS dims (row in LDS), in chunks of 32 with a
// scheduling barrier after each, as in dot_lr.
__device__ __forceinline__ void axpy_slice(float (&acc)[kDS], float w, const float *row) {
#pragma unroll
  for (int e0 = 0; e0 < kDS; e0 += 32) {
#pragma unroll
    for (int e = e0; e < e0 + 32; ++e) acc[e] = __builtin_fmaf(w, row[e], acc[e]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Dims [d0, d0 + kDS) of row `row` of a [T][D] fp32 array into registers
// (zeros past T).
template <int D>
__device__ __forceinline__ void load_own_row(float (&x)[kDS], const float *src, int row, int T,
                                             int d0) {
  const bool ok = row < T;
  const float *r = src + (size_t)(ok ? row : 0) * D + d0;   // row 0 exists: T >= 1
#pragma unroll
  for (int e = 0; e < kDS; e += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(r + e);
    x[e] = ok ? v[0] : 0.0f;
    x[e + 1] = ok ? v[1] : 0.0f;
    x[e + 2] = ok ? v[2] : 0.0f;
    x[e + 3] = ok ? v[3] : 0.0f;
  }
}

// Per row: log2-domain lse, 1/r and delta/r (tempered: 1 and delta).
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_f32_kernel(BwdArgs a, int dilution) {
  const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (size_t)a.BH * a.T) return;
  const float *O = reinterpret_cast<const float *>(a.o) + row * D;
  const float *G = reinterpret_cast<const float *>(a.dout) + row * D;
  const float delta = dotd<D>(O, G);
  a.lse2[row] = a.lse[row] * kLog2e;
  if (dilution) {
    const float ir = 1.0f / a.rowsum[row];
    a.invr[row] = ir;
    a.dri[row] = delta * ir;
  } else {
    a.invr[row] = 1.0f;
    a.dri[row] = delta;
  }
}

// Rows [i0, i0 + 64) of Q and dO and their per-row scalars into LDS, by all
// kWB threads of the workgroup; rows past T read as zeros with an lse2 that
// makes their bids 0.
template <int D>
struct RowTileF32 {
  float q[kBR * D], g[kBR * D];
  float lse2[kBR], invr[kBR], dri[kBR], rho[kBR];
};

template <int D>
__device__ __forceinline__ void load_row_tile(RowTileF32<D> &s, const BwdArgs &a, const float *Q,
                                              const float *G, size_t rbase, int i0, int tid,
                                              bool with_rho) {
  const int T = a.T;
  for (int u = tid; u < kBR * D; u += kWB) {
    const int row = i0 + u / D;
    const bool ok = row < T;
    s.q[u] = ok ? Q[(size_t)i0 * D + u] : 0.0f;
    s.g[u] = ok ? G[(size_t)i0 * D + u] : 0.0f;
  }
  if (tid < kBR) {
    const int row = i0 + tid;
    const bool ok = row < T;
    s.lse2[tid] = ok ? a.lse2[rbase + row] : kNoRowBwdF32;
    s.invr[tid] = ok ? a.invr[rbase + row] : 0.0f;
    s.dri[tid] = ok ? a.dri[rbase + row] : 0.0f;
    s.rho[tid] = (ok && with_rho) ? a.rho[rbase + row] : 0.0f;
  }
}

// The terms of one (row, key) pair of a dilution block walk: the bid, the
// running inclusive prefix, 1/D, sigma, dsigma and g.
struct PairF32 {
  float p, invd, sg, dsg, g;
};

template <bool CLAMP>
__device__ __forceinline__ PairF32 pair_terms(float s, float da, float c2, float lse2, float invr,
                                              float dri, bool vis, float basev, float &incl) {
  PairF32 t;
  t.p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.0f;
  incl += t.p;
  const float r = 1.0f / (basev + incl);
  t.invd = CLAMP ? fminf(r, kInvDMaxF32) : r;
  t.sg = t.p * t.invd;
  t.dsg = __builtin_fmaf(da, invr, -dri);
  t.g = t.dsg * t.sg * t.invd;
  return t;
}

// Later blocks' g sums: for each key and 32-row block, the sum of g over
// every block below it, walking the blocks from the last one up.
template <bool CLAMP, int D>
__global__ void __launch_bounds__(kWB, 1) bwd_gsum_f32_kernel(BwdArgs a, int ntiles) {
  using LG = LaneGeomF32<D>;
  __shared__ __attribute__((aligned(16))) RowTileF32<D> st;
  const int tid = threadIdx.x, t = tid & 63, w = tid >> 6;
  const int sub = t / LG::kPer;          // which kDS dims of the row this lane holds
  const int bh = blockIdx.x % a.BH, kb = blockIdx.x / a.BH;
  const int T = a.T, kw0 = kb * LG::kRows + LG::kPer * w, j = kw0 + t % LG::kPer;
  const int d0 = kDS * sub;
  const size_t head = (size_t)bh * T * D, rbase = (size_t)bh * T;
  const float *Q = reinterpret_cast<const float *>(a.q) + head;
  const float *K = reinterpret_cast<const float *>(a.k) + head;
  const float *V = reinterpret_cast<const float *>(a.v) + head;
  const float *G = reinterpret_cast<const float *>(a.dout) + head;
  const float *cin = a.cin + (size_t)bh * cin_floats_per_head(T, 0);
  float *gin = a.gin + (size_t)bh * gin_floats_per_head(T);
  const float c2 = a.c2 * head_tau_f32(a, bh);
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  float kv[kDS], vv[kDS];
  load_own_row<D>(kv, K, j, T, d0);
  load_own_row<D>(vv, V, j, T, d0);
  float running = 0.0f;
  // tiles from the last down to the first that sees the workgroup's keys;
  // a wave skips the tiles above its own keys (it still meets every barrier)
  for (int tile = ntiles - 1; tile >= (kb * LG::kRows) / kBR; --tile) {
    const int i0 = tile * kBR;
    __syncthreads();
    load_row_tile(st, a, Q, G, rbase, i0, tid, false);
    __syncthreads();
    if (kw0 >= T || tile < kw0 / kBR) continue;
#pragma unroll 1
    for (int half = 1; half >= 0; --half) {
      const int b = 2 * tile + half;
      if (32 * b >= T) continue;
      const bool has = j < 32 * (b + 1) && j < T;   // the key has an entry for block b
      const float basev = fmaxf((has ? cin[cin_block_offset(b, 0) + j] : 0.0f) + a.eps, eps_floor);
      float incl = 0.0f, gsum = 0.0f;
#pragma unroll 1
      for (int r = 0; r < 32; ++r) {
        const int i = 32 * b + r, li = 32 * half + r;
        if (i >= T) break;
        const float s = row_dot<D>(dot_lr(&st.q[li * D + d0], kv));
        const float da = row_dot<D>(dot_lr(&st.g[li * D + d0], vv));
        const PairF32 pt = pair_terms<CLAMP>(s, da, c2, st.lse2[li], st.invr[li], st.dri[li],
                                             j <= i, basev, incl);
        gsum += pt.g;
      }
      if (has && sub == 0) gin[(size_t)16 * b * (b + 1) + j] = running;
      running += gsum;
    }
  }
}

// dQ (and rho, and the rows' dL/dtau terms): lane = query row.
template <bool DIL, bool CLAMP, int D>
__global__ void __launch_bounds__(kWB, 1) bwd_dq_f32_kernel(BwdArgs a, int nqb) {
  using LG = LaneGeomF32<D>;
  __shared__ __attribute__((aligned(16))) float sK[kBR * D];
  __shared__ __attribute__((aligned(16))) float sV[kBR * D];
  const int tid = threadIdx.x, t = tid & 63, w = tid >> 6;
  const int sub = t / LG::kPer, d0 = kDS * sub;
  const int bh = blockIdx.x % a.BH, qb = nqb - 1 - blockIdx.x / a.BH;   // heaviest first
  const int T = a.T, qw0 = qb * LG::kRows + LG::kPer * w, i = qw0 + t % LG::kPer;
  const bool live = i < T;
  const int qs = i >> 5;
  const size_t head = (size_t)bh * T * D, rbase = (size_t)bh * T;
  const float *Q = reinterpret_cast<const float *>(a.q) + head;
  const float *K = reinterpret_cast<const float *>(a.k) + head;
  const float *V = reinterpret_cast<const float *>(a.v) + head;
  const float *G = reinterpret_cast<const float *>(a.dout) + head;
  const float tb = head_tau_f32(a, bh), c2 = a.c2 * tb, cs = a.c * tb;
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  float q[kDS], gd[kDS];   // this lane's dims of the row's Q and dO
  load_own_row<D>(q, Q, i, T, d0);
  load_own_row<D>(gd, G, i, T, d0);
  float x[kDS];
#pragma unroll
  for (int e = 0; e < kDS; ++e) x[e] = 0.0f;
  const float lse2 = live ? a.lse2[rbase + i] : kNoRowBwdF32;
  const float invr = live ? a.invr[rbase + i] : 0.0f;
  const float dri = live ? a.dri[rbase + i] : 0.0f;
  const float *cin_blk = a.cin + (size_t)bh * cin_floats_per_head(T, 0) + cin_block_offset(qs, 0);
  const float *gin_blk = a.gin + (size_t)bh * gin_floats_per_head(T) + (size_t)16 * qs * (qs + 1);
  float rho = 0.0f;
  // keys the workgroup's rows see, and this wave's (none for a wave past T)
  const int kend = min(qb * LG::kRows + LG::kRows, T);
  const int kend_w = qw0 < T ? min(qw0 + LG::kPer, T) : 0;
  for (int j0 = 0; j0 < kend; j0 += kBR) {
    __syncthreads();
    for (int u = tid; u < kBR * D; u += kWB) {
      const bool ok = j0 + u / D < T;
      sK[u] = ok ? K[(size_t)j0 * D + u] : 0.0f;
      sV[u] = ok ? V[(size_t)j0 * D + u] : 0.0f;
    }
    __syncthreads();
    const int jn = min(kBR, kend_w - j0);   // wave-uniform; <= 0 past the wave's keys
#pragma unroll 1
    for (int jj = 0; jj < jn; ++jj) {
      const int j = j0 + jj;
      const float s = row_dot<D>(dot_lr(&sK[jj * D + d0], q));
      const float da = row_dot<D>(dot_lr(&sV[jj * D + d0], gd));
      const bool vis = live && j <= i;
      float e;
      if constexpr (DIL) {
        // every lane of the 32-row block runs this for the same key: the
        // prefix of the bids and the suffix of g are scans over those lanes
        // (each 32-lane half of the wave holds one block's rows); lanes past
        // T may sit in a block past the last one: they read nothing (their
        // bids and g are 0, so the scans are unchanged)
        const bool has = live && j < 32 * (qs + 1);
        const float basev = fmaxf((has ? cin_blk[j] : 0.0f) + a.eps, eps_floor);
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.0f;
        float incl = p;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          const float o = __shfl_up(incl, off, 32);
          if ((t & 31) >= off) incl += o;
        }
        const float rr = 1.0f / (basev + incl);
        const float invd = CLAMP ? fminf(rr, kInvDMaxF32) : rr;
        const float dsg = __builtin_fmaf(da, invr, -dri);
        const float g = dsg * (p * invd) * invd;
        float suf = g;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          const float o = __shfl_down(suf, off, 32);
          if ((t & 31) + off < 32) suf += o;
        }
        const float Gij = (has ? gin_blk[j] : 0.0f) + suf;
        e = p * __builtin_fmaf(dsg, invd, -Gij);
        rho += e;
      } else {
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.0f;
        e = p * (da - dri);
      }
      axpy_slice(x, e, &sK[jj * D + d0]);
    }
  }
  // the dL/dtau row term covers all d: the kL lanes' parts are added
  float tq = 0.0f;
  float u[kDS];
  const float *PK = DIL ? reinterpret_cast<const float *>(a.pk) + head + (size_t)(live ? i : 0) * D + d0
                        : nullptr;
#pragma unroll
  for (int d = 0; d < kDS; ++d) {
    u[d] = DIL ? __builtin_fmaf(-rho, live ? PK[d] : 0.0f, x[d]) : x[d];
    tq = __builtin_fmaf(q[d], u[d], tq);
  }
  tq = row_dot<D>(tq);
  if (!live) return;
  const size_t ridx = rbase + i;
  float *dQ = reinterpret_cast<float *>(a.dq) + head + (size_t)i * D + d0;
  if (DIL && sub == 0) a.rho[ridx] = rho;   // every lane of the row forms the same rho
#pragma unroll
  for (int d = 0; d < kDS; ++d) dQ[d] = u[d] * cs;
  if (a.dtau && sub == 0) a.trow[ridx] = tq;
}

// dK and dV: lane = key column, walking the 32-row blocks that see it, top
// down.  A block is walked twice: first for g of each row (kept in LDS, then
// summed from the bottom row up into its inclusive suffix), then for the
// gradients with G = (later blocks) + that suffix.
template <bool DIL, bool CLAMP, int D>
__global__ void __launch_bounds__(kWB, 1) bwd_dkdv_f32_kernel(BwdArgs a, int ntiles) {
  using LG = LaneGeomF32<D>;
  __shared__ __attribute__((aligned(16))) RowTileF32<D> st;
  // per wave, per row of a block, per lane: g, then its suffix
  __shared__ float sSuf[DIL ? kFWB : 1][DIL ? 32 : 1][64];
  const int tid = threadIdx.x, t = tid & 63, w = tid >> 6;
  const int sub = t / LG::kPer, d0 = kDS * sub;
  const int bh = blockIdx.x % a.BH, kb = blockIdx.x / a.BH;
  const int T = a.T, kw0 = kb * LG::kRows + LG::kPer * w, j = kw0 + t % LG::kPer;
  const size_t head = (size_t)bh * T * D, rbase = (size_t)bh * T;
  const float *Q = reinterpret_cast<const float *>(a.q) + head;
  const float *K = reinterpret_cast<const float *>(a.k) + head;
  const float *V = reinterpret_cast<const float *>(a.v) + head;
  const float *G = reinterpret_cast<const float *>(a.dout) + head;
  const float *cin = a.cin + (size_t)bh * cin_floats_per_head(T, 0);
  const float *gin = a.gin + (size_t)bh * gin_floats_per_head(T);
  const float tb = head_tau_f32(a, bh), c2 = a.c2 * tb, cs = a.c * tb;
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  float kv[kDS], vv[kDS];   // this lane's dims of the key's K and V rows
  load_own_row<D>(kv, K, j, T, d0);
  load_own_row<D>(vv, V, j, T, d0);
  float dk[kDS], dv[kDS];
#pragma unroll
  for (int e = 0; e < kDS; ++e) dk[e] = dv[e] = 0.0f;
  float(*suf_w)[64] = sSuf[DIL ? w : 0];
  // tiles from the first that sees the workgroup's keys down; a wave skips
  // the tiles above its own keys (it still meets every barrier)
  for (int tile = (kb * LG::kRows) / kBR; tile < ntiles; ++tile) {
    const int i0 = tile * kBR;
    __syncthreads();
    load_row_tile(st, a, Q, G, rbase, i0, tid, DIL);
    __syncthreads();
    if (kw0 >= T || tile < kw0 / kBR) continue;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * tile + half;
      if (32 * b >= T) break;
      if constexpr (DIL) {
        const bool has = j < 32 * (b + 1) && j < T;
        const float basev =
            fmaxf((has ? cin[cin_block_offset(b, 0) + j] : 0.0f) + a.eps, eps_floor);
        const float later = has ? gin[(size_t)16 * b * (b + 1) + j] : 0.0f;
        const int nr = min(32, T - 32 * b);   // rows of the block
        float incl = 0.0f;
#pragma unroll 1
        for (int r = 0; r < nr; ++r) {
          const int i = 32 * b + r, li = 32 * half + r;
          const float s = row_dot<D>(dot_lr(&st.q[li * D + d0], kv));
          const float da = row_dot<D>(dot_lr(&st.g[li * D + d0], vv));
          suf_w[r][t] = pair_terms<CLAMP>(s, da, c2, st.lse2[li], st.invr[li], st.dri[li], j <= i,
                                          basev, incl).g;
        }
        // G inside the block: inclusive suffix of g, summed from the last row up
        float suf = later;
#pragma unroll 1
        for (int r = nr - 1; r >= 0; --r) {
          suf += suf_w[r][t];
          suf_w[r][t] = suf;
        }
        incl = 0.0f;
#pragma unroll 1
        for (int r = 0; r < nr; ++r) {
          const int i = 32 * b + r, li = 32 * half + r;
          const float s = row_dot<D>(dot_lr(&st.q[li * D + d0], kv));
          const float da = row_dot<D>(dot_lr(&st.g[li * D + d0], vv));
          const PairF32 pt = pair_terms<CLAMP>(s, da, c2, st.lse2[li], st.invr[li], st.dri[li],
                                               j <= i, basev, incl);
          const float Gij = suf_w[r][t];
          const float ds = pt.p * (__builtin_fmaf(pt.dsg, pt.invd, -Gij) - st.rho[li]);
          const float aw = pt.sg * st.invr[li];
          axpy_slice(dk, ds, &st.q[li * D + d0]);
          axpy_slice(dv, aw, &st.g[li * D + d0]);
        }
      } else {
#pragma unroll 1
        for (int r = 0; r < 32; ++r) {
          const int i = 32 * b + r, li = 32 * half + r;
          if (i >= T) break;
          const float s = row_dot<D>(dot_lr(&st.q[li * D + d0], kv));
          const float da = row_dot<D>(dot_lr(&st.g[li * D + d0], vv));
          const float p = j <= i ? exp2f(__builtin_fmaf(s, c2, -st.lse2[li])) : 0.0f;
          const float ds = p * (da - st.dri[li]);
          axpy_slice(dk, ds, &st.q[li * D + d0]);
          axpy_slice(dv, p, &st.g[li * D + d0]);
        }
      }
    }
  }
  if (j >= T) return;
  float *dK = reinterpret_cast<float *>(a.dk) + head + (size_t)j * D + d0;
  float *dV = reinterpret_cast<float *>(a.dv) + head + (size_t)j * D + d0;
#pragma unroll
  for (int e = 0; e < kDS; ++e) {
    dK[e] = dk[e] * cs;
    dV[e] = dv[e];
  }
}

hipError_t launch_dtau(const BwdArgs &a, hipStream_t s);

template <bool CLAMP, int D>
static hipError_t launch_bwd_f32_c(int mode, const BwdArgs &a, hipStream_t s) {
  const bool dil = mode == 1;
  const size_t rows = (size_t)a.BH * a.T;
  hipLaunchKernelGGL(bwd_prep_f32_kernel<D>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                     s, a, dil ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int ntiles = (a.T + kBR - 1) / kBR;   // 64-row tiles
  const int nwb = (a.T + LaneGeomF32<D>::kRows - 1) / LaneGeomF32<D>::kRows;   // workgroups per head
  const dim3 grid((unsigned)(nwb * a.BH)), block(kWB);
  if (dil) {
    FwdArgs f{};
    f.q = a.q;
    f.k = a.k;
    f.lse2 = a.lse2;
    f.cin = a.cin;
    f.BH = a.BH;
    f.T = f.Tq = f.kstride = a.T;
    f.D = D;
    f.ksplit = 1;
    f.tau_bh = a.tau_bh;
    f.c2 = a.c2;
    f.eps = a.eps;
    // the forward's table, when the caller passes it, holds the same values
    if (!a.cin_given) e = launch_colsum_f32(f, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gsum_f32_kernel<CLAMP, D>), grid, block, 0, s, a, ntiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // PK = softmax-weighted keys: the fp32 tempered forward with the keys as values
    FwdArgs t{};
    t.q = a.q;
    t.k = a.k;
    t.v = a.k;
    t.out = a.pk;
    t.BH = a.BH;
    t.T = t.Tq = t.kstride = a.T;
    t.D = D;
    t.ksplit = 1;
    t.tau_bh = a.tau_bh;
    t.c2 = a.c2;
    e = launch_rows_f32(kRowTempered, t, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<true, CLAMP, D>), grid, block, 0, s, a, nwb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dtau(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<true, CLAMP, D>), grid, block, 0, s, a, ntiles);
  } else {
    hipLaunchKernelGGL((bwd_dq_f32_kernel<false, false, D>), grid, block, 0, s, a, nwb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dtau(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<false, false, D>), grid, block, 0, s, a, ntiles);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_f32_d(int mode, const BwdArgs &a, hipStream_t s) {
  // as in the bf16 kernels, the 1/D clamp matters only for eps below 2^-63
  const bool clamp = mode == 1 && !(a.eps >= 1.0842021724855044e-19f);
  return clamp ? launch_bwd_f32_c<true, D>(mode, a, s) : launch_bwd_f32_c<false, D>(mode, a, s);
}

hipError_t launch_bwd_f32(int mode, const BwdArgs &a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_bwd_f32_d<64>(mode, a, s);
    case 128: return launch_bwd_f32_d<128>(mode, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
