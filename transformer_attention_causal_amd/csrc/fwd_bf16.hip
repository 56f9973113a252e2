// fwd_bf16.hip -- bf16 forward kernels for gfx950 (matrix cores, LDS tiles).
//
// Operations (cited by page and section):
//  * Tempered causal attention: softmax of tau * <q_i,k_j> / sqrt(d) over the
//    visible keys j <= i, applied to V ("Learning to Focus: Focal Attention",
//    sec. 2.1 eq. focal-const with tau = 1/t; "YaRN > Attention Temperature
//    Scaling", sqrt(t) multiplier).
//  * Dilution attention ("DilutionAttention v0.1.0 - results", "The
//    operator"), computed in three passes:
//      pass 1  (kRowLse)   log-sum-exp of every query row (the softmax bids'
//                          normaliser),
//      pass 2a (colsum)    per 32-row query block, the demand each key has
//                          received from all earlier rows (exclusive column
//                          cumulative sum of the bids, taken block by block),
//      pass 2b (kRowShare) recompute the bids, finish the column prefix inside
//                          the block, form share = p / (committed + p + eps),
//                          and accumulate share@V and the share row sums.
//
// Work decomposition (one workgroup = 4 waves = 256 threads):
//  * row kernels: a workgroup owns 128 query rows, wave w the 32 rows
//    [q0+32w, q0+32w+32); K and V stream through LDS in 64-key tiles (double
//    buffered, one barrier per tile).  Scores of a 32x32 (key, query) block
//    come from four 32x32x16 bf16 MFMAs over d = 64.
//  * tempered / pass 1 keep scores as S^T (lane = query, 16 keys in
//    registers), so row maxima and sums are in-lane plus one exchange between
//    the two wave halves, and the bf16 bids feed the P@V MFMA directly as its
//    B operand.
//  * pass 2b keeps scores as S (lane = key, 16 queries in registers), so the
//    column prefix runs in-lane; the shares are then transposed to the S^T
//    layout by one MFMA against the identity (exact for bf16 values) to feed
//    share@V.
//  * pass 2a: a workgroup owns 128 keys (wave w 32 of them, held in
//    registers) and walks the 32-row query blocks below them in order,
//    carrying each key's running demand in a register.
#include "attn_common.hpp"
#include "launch.hpp"

#include <float.h>

namespace attn {

constexpr int kBM = 128;        // query rows per workgroup (row kernels)
constexpr int kBN = 64;         // keys per LDS tile (row kernels)
constexpr int kKRow = 72;       // LDS row stride of K tiles, bf16 (64 + 8 pad)
constexpr int kVRow = 68;       // LDS row stride of V^T tiles, bf16 (64 keys + 4 pad)
constexpr int kKTile = kBN * kKRow;        // bf16 elements per K buffer
constexpr int kVTile = kHeadDim * kVRow;   // bf16 elements per V^T buffer
constexpr float kRescaleSlack = 8.0f;      // log2 units the running max may lag

// Query index (within a wave's 32 rows) of accumulator element r in lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Load one 16-byte chunk of a [BH][T][64] bf16 tensor, zeros past the end.
__device__ __forceinline__ u32x4 load_row_chunk(const __bf16 *base, int row, int T, int chunk) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (row < T) z = *reinterpret_cast<const u32x4 *>(base + (size_t)row * kHeadDim + chunk * 8);
  return z;
}

// A/B operand fragment for d-chunk c of a 64-wide bf16 row held in LDS.
__device__ __forceinline__ bf16x8 lds_frag(const __bf16 *row, int c, int h) {
  return *reinterpret_cast<const bf16x8 *>(row + 16 * c + 8 * h);
}

// V^T operand for keys [16c+4h, +4) and [16c+8+4h, +4) of a 32-key sub-tile.
__device__ __forceinline__ bf16x8 lds_vfrag(const __bf16 *vrow, int c, int h) {
  u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + 16 * c + 4 * h);
  u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + 16 * c + 8 + 4 * h);
  u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, u);
}

template <int MODE>
__global__ void __launch_bounds__(256) rows_bf16_kernel(FwdArgs a, int nqb) {
  constexpr bool kNeedV = (MODE != kRowLse);
  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * kKTile];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kNeedV ? 2 * kVTile : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // heaviest query blocks first; consecutive workgroups take different heads
  const int bh = blockIdx.x % a.BH;
  const int qb = nqb - 1 - blockIdx.x / a.BH;
  const int T = a.T;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * w;              // first row of this wave
  const bool wave_live = qw0 < T;
  const size_t head = (size_t)bh * T * kHeadDim;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;

  const int kend = min(q0 + kBM, T);        // keys [0, kend) are visible to some row
  const int nkt = (kend + kBN - 1) / kBN;

  // Q fragments: lane holds Q[qw0 + l32][16c + 8h .. +8) -- usable as the B
  // operand of S^T = K Q^T and as the A operand of S = Q K^T.
  bf16x8 qf[4];
  {
    const int row = qw0 + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 u = load_row_chunk(Q, row, T, 2 * c + h);
      qf[c] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // tile loaders: K as [key][d] rows; V transposed to [d][key] on the way in.
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      kreg[i] = load_row_chunk(K, key0 + (u >> 3), T, u & 7);
    }
    if constexpr (kNeedV) {
      const int kp = tid & 31, dc = tid >> 5;
      vreg[0] = load_row_chunk(V, key0 + 2 * kp, T, dc);
      vreg[1] = load_row_chunk(V, key0 + 2 * kp + 1, T, dc);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16 *k = sK + buf * kKTile;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(k + (u >> 3) * kKRow + (u & 7) * 8) = kreg[i];
    }
    if constexpr (kNeedV) {
      __bf16 *vt = sV + buf * kVTile;
      const int kp = tid & 31, dc = tid >> 5;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a0 = vreg[0][i], a1 = vreg[1][i];
        const uint32_t even = (a0 & 0xffffu) | (a1 << 16);           // d = 8dc + 2i
        const uint32_t odd = (a0 >> 16) | (a1 & 0xffff0000u);        // d = 8dc + 2i + 1
        *reinterpret_cast<uint32_t *>(vt + (8 * dc + 2 * i) * kVRow + 2 * kp) = even;
        *reinterpret_cast<uint32_t *>(vt + (8 * dc + 2 * i + 1) * kVRow + 2 * kp) = odd;
      }
    }
  };

  // ---- per-mode state
  f32x16 o0 = zero16(), o1 = zero16();   // O^T[d][query]: d in [0,32) and [32,64)
  float m_run = -INFINITY, l_run = 0.0f; // tempered / lse: running max (scaled) and sum
  float rsum = 0.0f;                     // share: running share row sum (this half's keys)
  float lseq[16];                        // share: lse2 of this lane's 16 query rows
  bf16x8 ident[2];                       // share: identity operand for the transpose
  const float *cin_blk = nullptr;
  const int qs = qw0 >> 5;
  if constexpr (MODE == kRowShare) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = qw0 + acc_row(r, h);
      lseq[r] = row < T ? a.lse2[(size_t)bh * T + row] : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = (acc_row(8 * c + j, h) == l32) ? 1.0f : 0.0f;
      ident[c] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    cin_blk = a.cin + (size_t)bh * cin_floats_per_head(T) + (size_t)16 * qs * (qs - 1);
  }
  const float eps_floor = fmaxf(a.eps, FLT_MIN);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);
    const __bf16 *kt_lds = sK + buf * kKTile;
    const __bf16 *vt_lds = sV + (kNeedV ? buf * kVTile : 0);

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kb = kt * kBN + 32 * s;       // first key of this 32-key sub-tile
      if (!wave_live || kb > qw0) continue;   // wave-uniform: the sub-tile is in every row's future
      const bool diag = (kb == qw0);
      const __bf16 *krow = kt_lds + (32 * s + l32) * kKRow;

      if constexpr (MODE == kRowTempered || MODE == kRowLse) {
        // S^T[key][query] = K Q^T ; lane: query l32, keys kb + acc_row(r,h)
        f32x16 sc = zero16();
#pragma unroll
        for (int c = 0; c < 4; ++c) sc = mfma32(lds_frag(krow, c, h), qf[c], sc);
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = sc[r];
          if (diag && acc_row(r, h) > l32) v = -INFINITY;
          x[r] = v;
          tmax = fmaxf(tmax, v);
        }
        tmax = fmaxf(tmax, swap_halves(tmax));
        const float tmax2 = (tmax == -INFINITY) ? -INFINITY : tmax * a.c2;
        if (__ballot(tmax2 > m_run + kRescaleSlack) != 0ull) {
          const float m_new = fmaxf(m_run, tmax2);
          const float alpha = fast_exp2(m_run - m_new);
          l_run *= alpha;
          if constexpr (MODE == kRowTempered) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { o0[r] *= alpha; o1[r] *= alpha; }
          }
          m_run = m_new;
        }
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float y = (x[r] == -INFINITY) ? -INFINITY : __builtin_fmaf(x[r], a.c2, -m_run);
          p[r] = fast_exp2(y);
          l_run += p[r];
        }
        if constexpr (MODE == kRowTempered) {
          const bf16x8 pf0 = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          const bf16x8 pf1 = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
          const __bf16 *v0 = vt_lds + l32 * kVRow + 32 * s;
          const __bf16 *v1 = vt_lds + (32 + l32) * kVRow + 32 * s;
          o0 = mfma32(lds_vfrag(v0, 0, h), pf0, o0);
          o0 = mfma32(lds_vfrag(v0, 1, h), pf1, o0);
          o1 = mfma32(lds_vfrag(v1, 0, h), pf0, o1);
          o1 = mfma32(lds_vfrag(v1, 1, h), pf1, o1);
        }
      } else {
        // ---- pass 2b: S[query][key] = Q K^T ; lane: key kb + l32, queries acc_row(r,h)
        f32x16 sc = zero16();
#pragma unroll
        for (int c = 0; c < 4; ++c) sc = mfma32(qf[c], lds_frag(krow, c, h), sc);
        const int key = kb + l32;
        // demand committed on this key by all rows before this 32-row block
        float base = (kb < qw0) ? cin_blk[key] : 0.0f;
        base = fmaxf(base + a.eps, eps_floor);
        const bool tail = (qw0 + 32 > T);
        float p[16], run[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = fast_exp2(__builtin_fmaf(sc[r], a.c2, -lseq[r]));
          if (diag && l32 > acc_row(r, h)) v = 0.0f;
          if (tail && qw0 + acc_row(r, h) >= T) v = 0.0f;
          p[r] = v;
          run[r] = v;
        }
        // inclusive prefix of the bids down the 32 query rows of this block:
        // in-lane over runs of 4 consecutive rows, then across the two halves
        float mine[4], other[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          run[4 * g + 1] += run[4 * g];
          run[4 * g + 2] += run[4 * g + 1];
          run[4 * g + 3] += run[4 * g + 2];
          mine[g] = run[4 * g + 3];
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) other[g] = swap_halves(mine[g]);
        float acc_off = base;
        float share[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float off = acc_off + (h ? other[g] : 0.0f);
          acc_off += mine[g] + other[g];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            share[r] = p[r] * fast_rcp(run[r] + off);
          }
        }
        // transpose the shares to S^T (lane = query) with an identity MFMA
        const bf16x8 sb0 = to_bf16x8(share[0], share[1], share[2], share[3], share[4],
                                     share[5], share[6], share[7]);
        const bf16x8 sb1 = to_bf16x8(share[8], share[9], share[10], share[11], share[12],
                                     share[13], share[14], share[15]);
        f32x16 st = mfma32(sb0, ident[0], zero16());
        st = mfma32(sb1, ident[1], st);
#pragma unroll
        for (int r = 0; r < 16; ++r) rsum += st[r];
        const bf16x8 pf0 = to_bf16x8(st[0], st[1], st[2], st[3], st[4], st[5], st[6], st[7]);
        const bf16x8 pf1 = to_bf16x8(st[8], st[9], st[10], st[11], st[12], st[13], st[14], st[15]);
        const __bf16 *v0 = vt_lds + l32 * kVRow + 32 * s;
        const __bf16 *v1 = vt_lds + (32 + l32) * kVRow + 32 * s;
        o0 = mfma32(lds_vfrag(v0, 0, h), pf0, o0);
        o0 = mfma32(lds_vfrag(v0, 1, h), pf1, o0);
        o1 = mfma32(lds_vfrag(v1, 0, h), pf0, o1);
        o1 = mfma32(lds_vfrag(v1, 1, h), pf1, o1);
      }
    }

    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const int row = qw0 + l32;
  float denom;
  if constexpr (MODE == kRowShare) {
    denom = rsum + swap_halves(rsum);
  } else {
    denom = l_run + swap_halves(l_run);
    if (h == 0 && row < T) {
      const float lse2 = m_run + __builtin_log2f(denom);
      if (a.lse2) a.lse2[(size_t)bh * T + row] = lse2;
      if (a.lse_nat) a.lse_nat[(size_t)bh * T + row] = lse2 * kLn2;
    }
  }
  if constexpr (MODE != kRowLse) {
    if (row < T) {
      const float inv = 1.0f / denom;
      __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + head + (size_t)row * kHeadDim;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 8 * g + 4 * h;
        u32x2 lo, hi;
        lo[0] = pack_bf16x2(o0[4 * g] * inv, o0[4 * g + 1] * inv);
        lo[1] = pack_bf16x2(o0[4 * g + 2] * inv, o0[4 * g + 3] * inv);
        hi[0] = pack_bf16x2(o1[4 * g] * inv, o1[4 * g + 1] * inv);
        hi[1] = pack_bf16x2(o1[4 * g + 2] * inv, o1[4 * g + 3] * inv);
        *reinterpret_cast<u32x2 *>(O + d0) = lo;
        *reinterpret_cast<u32x2 *>(O + 32 + d0) = hi;
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2a

constexpr int kCB = 128;  // keys per workgroup (4 waves x 32)

__global__ void __launch_bounds__(256) colsum_bf16_kernel(FwdArgs a, int nkb, int nqs) {
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][32 * kKRow];
  __shared__ __attribute__((aligned(16))) float sL[2][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;          // longest column walks first
  const int T = a.T;
  const int kw0 = kb * kCB + 32 * w;          // first key of this wave
  const bool wave_live = kw0 < T;
  const int key = kw0 + l32;
  const size_t head = (size_t)bh * T * kHeadDim;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const float *L2 = a.lse2 + (size_t)bh * T;
  float *cin = a.cin + (size_t)bh * cin_floats_per_head(T);

  bf16x8 kf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) kf[c] = __builtin_bit_cast(bf16x8, load_row_chunk(K, key, T, 2 * c + h));

  const int qs0 = (kb * kCB) >> 5;
  u32x4 qreg;
  float lreg = 0.0f;
  auto load_q = [&](int qs) {
    const int row = 32 * qs + (tid >> 3);
    qreg = load_row_chunk(Q, row, T, tid & 7);
    if (tid < 32) lreg = (32 * qs + tid < T) ? L2[32 * qs + tid] : 0.0f;
  };
  auto store_q = [&](int buf) {
    *reinterpret_cast<u32x4 *>(&sQ[buf][(tid >> 3) * kKRow + (tid & 7) * 8]) = qreg;
    if (tid < 32) sL[buf][tid] = lreg;
  };

  float run = 0.0f;  // demand this half-lane's rows have put on `key` so far
  load_q(qs0);
  store_q(0);
  __syncthreads();
  for (int qs = qs0; qs < nqs; ++qs) {
    const int buf = (qs - qs0) & 1;
    if (qs + 1 < nqs) load_q(qs + 1);
    if (wave_live && 32 * qs + 31 >= kw0) {
      const bool diag = (32 * qs == kw0);
      const bool tail = (32 * qs + 32 > T);
      f32x16 sc = zero16();
      const __bf16 *qrow = &sQ[buf][l32 * kKRow];
#pragma unroll
      for (int c = 0; c < 4; ++c) sc = mfma32(lds_frag(qrow, c, h), kf[c], sc);
      if (32 * qs > kw0) {
        // demand committed before block qs: rows < 32 qs, both halves
        const float total = run + swap_halves(run);
        if (h == 0 && key < T) cin[(size_t)16 * qs * (qs - 1) + key] = total;
      }
      float part = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lq = *reinterpret_cast<const f32x4 *>(&sL[buf][8 * g + 4 * h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          float v = fast_exp2(__builtin_fmaf(sc[r], a.c2, -lq[i]));
          if (diag && l32 > acc_row(r, h)) v = 0.0f;
          if (tail && 32 * qs + acc_row(r, h) >= T) v = 0.0f;
          part += v;
        }
      }
      run += part;
    }
    if (qs + 1 < nqs) store_q(buf ^ 1);
    __syncthreads();
  }
  if (a.demand_out && wave_live) {
    const float total = run + swap_halves(run);
    if (h == 0 && key < T) a.demand_out[(size_t)bh * T + key] = total;
  }
}

hipError_t launch_rows_bf16(int mode, const FwdArgs &a, hipStream_t s) {
  const int nqb = (a.T + kBM - 1) / kBM;
  dim3 grid((unsigned)(nqb * a.BH)), block(256);
  switch (mode) {
    case kRowTempered: hipLaunchKernelGGL(rows_bf16_kernel<kRowTempered>, grid, block, 0, s, a, nqb); break;
    case kRowLse: hipLaunchKernelGGL(rows_bf16_kernel<kRowLse>, grid, block, 0, s, a, nqb); break;
    default: hipLaunchKernelGGL(rows_bf16_kernel<kRowShare>, grid, block, 0, s, a, nqb); break;
  }
  return hipGetLastError();
}

hipError_t launch_colsum_bf16(const FwdArgs &a, hipStream_t s) {
  const int nkb = (a.T + kCB - 1) / kCB;
  const int nqs = (a.T + 31) / 32;
  hipLaunchKernelGGL(colsum_bf16_kernel, dim3((unsigned)(nkb * a.BH)), dim3(256), 0, s, a, nkb, nqs);
  return hipGetLastError();
}

}  // namespace attn
