// fwd_f32.hip -- fp32 forward kernels (vector ALU only; no bf16 anywhere),
// head dimension D = 64 or 128 (a template parameter).
//
// Same operations and the same three-pass structure as the bf16 kernels
// (tempered causal softmax attention -- "Learning to Focus: Focal Attention"
// sec. 2.1 eq. focal-const, "YaRN > Attention Temperature Scaling"; dilution
// attention -- "DilutionAttention v0.1.0 - results", "The operator"), for
// fp32 storage where full single precision is required.  One lane owns one
// query row (row kernels) or one key column (pass 2a); K/V or Q rows stream
// through LDS in 64-row tiles and are read as broadcasts.  The column prefix
// inside a 32-row query block is a shuffle scan across the 32 lanes that own
// those rows.
#include "attn_common.hpp"
#include "launch.hpp"

#include <float.h>

namespace attn {

constexpr int kFR = 64;           // rows per wave, and keys (or rows) per LDS tile
constexpr int kFW = 4;            // waves per workgroup: they share each LDS tile
constexpr int kFB = kFR * kFW;    // rows (row kernels) or keys (column sums) per workgroup
constexpr float kNoRowF32 = 1e30f;  // log-sum-exp of a position that holds no row

// Rows of up to this many keys keep the d = 64 tempered kernel's single
// output accumulator (two waves per SIMD); longer rows take the tiled form
// below, which holds full single precision at one wave per SIMD.
constexpr int kUntiledMaxT = 2048;

template <int MODE, int D, bool TILED>
__global__ void __launch_bounds__(kFB) rows_f32_kernel(FwdArgs a, int nqb) {
  __shared__ __attribute__((aligned(16))) float sK[kFR * D];
  __shared__ __attribute__((aligned(16))) float sV[MODE == kRowLse ? 4 : kFR * D];
  // Rows are positions: query row r of Q is position P + r (P = 0 for a
  // whole prefill); blocks start at position vrow0 <= P, and lanes at
  // positions before P hold no row.
  const int tid = threadIdx.x, t = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x % a.BH;
  // heaviest blocks first; block b covers positions vrow0 + kFB b ..
  const int qb = nqb - 1 - blockIdx.x / a.BH;
  const int T = a.T, Tq = a.Tq, P = T - Tq;
  const int q0 = a.vrow0 + qb * kFB + kFR * w;   // this wave's first position
  const int i = q0 + t;  // this lane's position
  const int li = i - P;  // and its query row
  const bool live = (unsigned)li < (unsigned)Tq;
  const size_t qhead = (size_t)bh * Tq * D, khead = (size_t)bh * a.kstride * D;
  const float c2 = head_c2(a, bh);
  const float *Q = reinterpret_cast<const float *>(a.q) + qhead;
  const float *K = reinterpret_cast<const float *>(a.k) + khead;
  const float *V = reinterpret_cast<const float *>(a.v) + khead;

  // Long rows keep full single precision: the row sum l is a compensated
  // (Kahan) sum, and the output accumulates per 64-key tile (acct, from zero)
  // before the tile is added to the running acc, so rounding grows with
  // 64 + T/64 terms rather than T.  Against the running max m both hold
  // scaled values; a_tile is the product of this tile's rescale factors.
  // Untiled (TILED = false, the d = 64 tempered kernel on rows of up to
  // kUntiledMaxT keys) the key loop accumulates straight into acc.
  constexpr bool kTiled = TILED && MODE != kRowLse;
  float q[D], acc[D], acct[kTiled ? D : 1];
  float *ta = kTiled ? acct : acc;   // what the key loop accumulates into
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = live ? Q[(size_t)li * D + e] : 0.0f;
    acc[e] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f, lc = 0.0f, lse2 = 0.0f;
  // l += x, compensated (lc carries the rounding of the additions so far)
  auto add_l = [&](float x) {
    const float y = x - lc;
    const float t2 = l + y;
    lc = (t2 - l) - y;
    l = t2;
  };
  const int qs = i >> 5;
  const float *cin_blk = nullptr;
  if constexpr (MODE == kRowShare) {
    lse2 = live ? a.lse2[(size_t)bh * Tq + li] : 0.0f;
    cin_blk = a.cin + (size_t)bh * cin_floats_per_head(T, a.vrow0) + cin_block_offset(qs, a.vrow0);
  }
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  // this wave's keys: none when all its positions lie past T or before P
  // (it still takes part in every barrier)
  const int kend = (q0 < T && q0 + kFR > P) ? min(q0 + kFR, T) : 0;
  const int kend_wg = min(a.vrow0 + qb * kFB + kFB, T);          // the workgroup's

  for (int j0 = 0; j0 < kend_wg; j0 += kFR) {
    __syncthreads();
    for (int u = tid; u < kFR * D; u += kFB) {
      const int row = j0 + u / D;
      sK[u] = row < T ? K[(size_t)j0 * D + u] : 0.0f;
      if constexpr (MODE != kRowLse) sV[u] = row < T ? V[(size_t)j0 * D + u] : 0.0f;
    }
    __syncthreads();
    const int jn = min(kFR, kend - j0);   // <= 0 once the wave's keys are done
    if constexpr (kTiled) {
#pragma unroll
      for (int e = 0; e < D; ++e) acct[e] = 0.0f;
    }
    float a_tile = 1.0f;
    for (int jj = 0; jj < jn; ++jj) {
      const int j = j0 + jj;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = __builtin_fmaf(q[e], sK[jj * D + e], s);
      const bool vis = (j <= i) && live;
      if constexpr (MODE == kRowTempered || MODE == kRowLse) {
        if (vis) {
          const float x = s * c2;
          const float m_new = fmaxf(m, x);
          const float alpha = exp2f(m - m_new);
          const float p = exp2f(x - m_new);
          l *= alpha;
          lc *= alpha;
          add_l(p);
          if constexpr (MODE == kRowTempered) {
            a_tile *= alpha;
#pragma unroll
            for (int e = 0; e < D; ++e) ta[e] = __builtin_fmaf(p, sV[jj * D + e], ta[e] * alpha);
          }
          m = m_new;
        }
      } else {
        const float p = vis ? exp2f(__builtin_fmaf(s, c2, -lse2)) : 0.0f;
        // inclusive prefix of the bids over the 32 rows of this lane's block
        float incl = p;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) {
          const float o = __shfl_up(incl, off, 32);
          if ((t & 31) >= off) incl += o;
        }
        // lanes with no row (past T, or before P) read nothing: past T their
        // block can lie beyond the table, and their bids are 0 anyway
        float base = (live && j < 32 * (qs + 1)) ? cin_blk[j] : 0.0f;
        base = fmaxf(base + a.eps, eps_floor);
        const float share = p / (base + incl);
        add_l(share);
#pragma unroll
        for (int e = 0; e < D; ++e) ta[e] = __builtin_fmaf(share, sV[jj * D + e], ta[e]);
      }
    }
    if constexpr (kTiled) {
      // the tile's sum into the running one (a_tile = 1 in the share pass)
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = __builtin_fmaf(acc[e], a_tile, acct[e]);
    }
  }
  if (!live) return;
  if constexpr (MODE == kRowTempered || MODE == kRowLse) {
    const float l2 = m + log2f(l);
    if (a.lse2) a.lse2[(size_t)bh * Tq + li] = l2;
    if (a.lse_nat) a.lse_nat[(size_t)bh * Tq + li] = l2 * kLn2;
  }
  if constexpr (MODE == kRowShare) {
    if (a.rowsum_out) a.rowsum_out[(size_t)bh * Tq + li] = l;
  }
  if constexpr (MODE != kRowLse) {
    float *O = reinterpret_cast<float *>(a.out) + qhead + (size_t)li * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; ++e) O[e] = acc[e] * inv;
  }
}

template <int D>
__global__ void __launch_bounds__(kFB) colsum_f32_kernel(FwdArgs a, int nkb) {
  __shared__ __attribute__((aligned(16))) float sQ[kFR * D];
  __shared__ float sL[kFR];
  // Positions i of the walk are query row i - P (P = 0 for a whole prefill);
  // positions before P, from vrow0 on, are no row and bid nothing.
  const int tid = threadIdx.x;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;
  const int T = a.T, Tq = a.Tq, P = T - Tq;
  const int k0 = kb * kFB;
  const int j = k0 + tid;  // this lane's key column
  const float *Q = reinterpret_cast<const float *>(a.q) + (size_t)bh * Tq * D;
  const float *K = reinterpret_cast<const float *>(a.k) + (size_t)bh * a.kstride * D;
  const float c2 = head_c2(a, bh);
  float *cin = a.cin + (size_t)bh * cin_floats_per_head(T, a.vrow0);

  float kv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) kv[e] = (j < T) ? K[(size_t)j * D + e] : 0.0f;
  // Each key's running demand is a compensated (Kahan) sum: a column can
  // receive a bid from every later row, up to T of them, and a plain fp32
  // running sum would lose the low bits of the small ones.  run - lost is
  // the demand so far.
  float run = (a.demand_in && j < T) ? a.demand_in[(size_t)bh * a.kstride + j] : 0.0f;
  float lost = 0.0f;
  for (int i0 = max(k0, a.vrow0); i0 < T; i0 += kFR) {
    __syncthreads();
    for (int u = tid; u < kFR * D; u += kFB) {
      const int lr = i0 + u / D - P;
      sQ[u] = (unsigned)lr < (unsigned)Tq ? Q[(size_t)lr * D + u % D] : 0.0f;
    }
    if (tid < kFR) {
      const int lt = i0 + tid - P;
      sL[tid] = (unsigned)lt < (unsigned)Tq ? a.lse2[(size_t)bh * Tq + lt] : kNoRowF32;
    }
    __syncthreads();
    const int in = min(kFR, T - i0);
    for (int ii = 0; ii < in; ++ii) {
      const int i = i0 + ii;
      if ((i & 31) == 0 && (i >> 5) >= (j >> 5) && j < T)
        cin[cin_block_offset(i >> 5, a.vrow0) + j] = run - lost;  // demand before block i/32
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = __builtin_fmaf(sQ[ii * D + e], kv[e], s);
      if (j <= i && i >= P) {
        const float y = exp2f(__builtin_fmaf(s, c2, -sL[ii])) - lost;
        const float t2 = run + y;
        lost = (t2 - run) - y;
        run = t2;
      }
    }
  }
  if (a.demand_out && j < T) a.demand_out[(size_t)bh * a.kstride + j] = run - lost;
}

template <int D>
static hipError_t launch_rows_f32_d(int mode, const FwdArgs &a, hipStream_t s) {
  const int nqb = (a.T - a.vrow0 + kFB - 1) / kFB;   // blocks from position vrow0
  dim3 grid((unsigned)(nqb * a.BH)), block(kFB);
  switch (mode) {
    case kRowTempered:
      if constexpr (D == 64) {
        if (a.T <= kUntiledMaxT) {
          hipLaunchKernelGGL((rows_f32_kernel<kRowTempered, D, false>), grid, block, 0, s, a, nqb);
          break;
        }
      }
      hipLaunchKernelGGL((rows_f32_kernel<kRowTempered, D, true>), grid, block, 0, s, a, nqb);
      break;
    case kRowLse:
      hipLaunchKernelGGL((rows_f32_kernel<kRowLse, D, true>), grid, block, 0, s, a, nqb);
      break;
    default:
      hipLaunchKernelGGL((rows_f32_kernel<kRowShare, D, true>), grid, block, 0, s, a, nqb);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_rows_f32(int mode, const FwdArgs &a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_rows_f32_d<64>(mode, a, s);
    case 128: return launch_rows_f32_d<128>(mode, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_colsum_f32(const FwdArgs &a, hipStream_t s) {
  const int nkb = (a.T + kFB - 1) / kFB;
  const dim3 grid((unsigned)(nkb * a.BH)), block(kFB);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(colsum_f32_kernel<64>, grid, block, 0, s, a, nkb); break;
    case 128: hipLaunchKernelGGL(colsum_f32_kernel<128>, grid, block, 0, s, a, nkb); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
