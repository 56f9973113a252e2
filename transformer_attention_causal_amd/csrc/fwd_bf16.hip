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
//    come from four 32x32x16 bf16 MFMAs over d = 64; a 64-key tile is two such
//    blocks, handled together.  Only the one tile holding a wave's diagonal
//    applies the causal mask.
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
//  * Rows past the end of the sequence get a log-sum-exp of +1e30, which makes
//    their bids exactly zero in passes 2a/2b without a per-element mask.
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
constexpr float kNoRow = 1e30f;            // log-sum-exp given to rows past the end

// Query index (within a wave's 32 rows) of accumulator element r in lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Load one 16-byte chunk of a [BH][T][64] bf16 tensor, zeros past the end.
__device__ __forceinline__ u32x4 load_row_chunk(const __bf16 *base, int row, int T, int chunk) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (row < T) z = *reinterpret_cast<const u32x4 *>(base + (size_t)row * kHeadDim + chunk * 8);
  return z;
}

// Load one 16-byte chunk of row min(row, T-1): rows past the end repeat the
// last row.  Used for tiles streamed inside loops: every such row is either
// causally masked or weighted by an exact zero, and the load being
// unconditional keeps the compiler from waiting on in-flight loads before it
// zero-fills a register.
__device__ __forceinline__ u32x4 load_row_clamped(const __bf16 *base, int row, int T, int chunk) {
  const int r = row < T ? row : T - 1;
  return *reinterpret_cast<const u32x4 *>(base + (size_t)r * kHeadDim + chunk * 8);
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

__device__ __forceinline__ bf16x8 pack8(const float *v) {
  return to_bf16x8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
}

// O^T[d][query] += V^T[d][keys of sub-tile t] * P^T[keys][query] for both
// 32-row halves of d.  pf0/pf1 hold keys 0..15 / 16..31 of the sub-tile in
// the accumulator-layout order.
__device__ __forceinline__ void pv_update(f32x16 &o0, f32x16 &o1, const __bf16 *vt_lds, int t,
                                          int l32, int h, const bf16x8 &pf0, const bf16x8 &pf1) {
  const __bf16 *v0 = vt_lds + l32 * kVRow + 32 * t;
  const __bf16 *v1 = vt_lds + (32 + l32) * kVRow + 32 * t;
  o0 = mfma32(lds_vfrag(v0, 0, h), pf0, o0);
  o1 = mfma32(lds_vfrag(v1, 0, h), pf0, o1);
  o0 = mfma32(lds_vfrag(v0, 1, h), pf1, o0);
  o1 = mfma32(lds_vfrag(v1, 1, h), pf1, o1);
}

// Per-wave state of the row kernels.
struct RowState {
  f32x16 o0, o1;   // O^T[d][query]: d in [0,32) and [32,64)
  float m_run;     // running max of the scaled logits (log2 units)
  float l_run;     // running sum of exp2(x - m_run) over this half's keys
  float rsum;      // share row sum over this half's keys (pass 2b)
};

// Tempered softmax / pass-1 update for one 64-key tile (S^T orientation).
template <int MODE, bool DIAG>
__device__ __forceinline__ void st_tile(RowState &st, const bf16x8 *qf, const __bf16 *kt_lds,
                                        const __bf16 *vt_lds, int kb, int qw0, int l32, int h,
                                        float c2) {
  f32x16 s[2] = {zero16(), zero16()};
  const __bf16 *krow0 = kt_lds + l32 * kKRow;
  const __bf16 *krow1 = kt_lds + (32 + l32) * kKRow;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    s[0] = mfma32(lds_frag(krow0, c, h), qf[c], s[0]);
    s[1] = mfma32(lds_frag(krow1, c, h), qf[c], s[1]);
  }
  // lane: query qw0 + l32; element (t, r): key kb + 32t + acc_row(r, h)
  const int qrel = qw0 + l32 - kb;   // keys with 32t + acc_row <= qrel are visible
  float tmax = -INFINITY;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = (!DIAG || 32 * t + acc_row(r, h) <= qrel) ? s[t][r] : -INFINITY;
      tmax = fmaxf(tmax, v);
    }
  }
  tmax = both_halves_max(tmax);
  const float tmax2 = tmax * c2;   // finite: every row sees at least its first key
  if (__ballot(tmax2 > st.m_run + kRescaleSlack) != 0ull) {
    const float m_new = fmaxf(st.m_run, tmax2);
    const float alpha = fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
    if constexpr (MODE == kRowTempered) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st.o0[r] *= alpha;
        st.o1[r] *= alpha;
      }
    }
    st.m_run = m_new;
  }
  const float mneg = -st.m_run;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e = fast_exp2(__builtin_fmaf(s[t][r], c2, mneg));
      if (DIAG && 32 * t + acc_row(r, h) > qrel) e = 0.0f;
      p[r] = e;
      st.l_run += e;
    }
    if constexpr (MODE == kRowTempered) pv_update(st.o0, st.o1, vt_lds, t, l32, h, pack8(p), pack8(p + 8));
  }
}

// Pass-2b update for one 64-key tile (S orientation), one 32-key sub-tile at
// a time.
template <bool DIAG>
__device__ __forceinline__ void share_tile(RowState &st, const bf16x8 *qf, const float *lseq,
                                           const bf16x8 *ident, const float *base,
                                           const __bf16 *kt_lds, const __bf16 *vt_lds, int kb,
                                           int qw0, int l32, int h, float c2) {
  const float hsel = h ? 1.0f : 0.0f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // lane: key kb + 32t + l32; element r: query qw0 + acc_row(r, h)
    const __bf16 *krow = kt_lds + (32 * t + l32) * kKRow;
    f32x16 s = zero16();
#pragma unroll
    for (int c = 0; c < 4; ++c) s = mfma32(qf[c], lds_frag(krow, c, h), s);
    const int krel = kb + 32 * t + l32 - qw0;   // visible to rows with acc_row >= krel
    float p[16], run[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e = fast_exp2(__builtin_fmaf(s[r], c2, -lseq[r]));
      if (DIAG && acc_row(r, h) < krel) e = 0.0f;
      p[r] = e;
      run[r] = e;
    }
    // inclusive prefix of the bids down the 32 rows of this block: in-lane
    // over each run of 4 consecutive rows, then across the two halves
    float acc_off = base[t];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      run[4 * g + 1] += run[4 * g];
      run[4 * g + 2] += run[4 * g + 1];
      run[4 * g + 3] += run[4 * g + 2];
      const HalfPair tot = halves(run[4 * g + 3]);   // rows 8g..8g+3 | 8g+4..8g+7
      const float off = __builtin_fmaf(tot.h0, hsel, acc_off);
      acc_off += tot.h0 + tot.h1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        run[r] = p[r] * fast_rcp(run[r] + off);   // the share
      }
    }
    // transpose the shares to S^T (lane = query) with an identity MFMA
    f32x16 sT = mfma32(pack8(run), ident[0], zero16());
    sT = mfma32(pack8(run + 8), ident[1], sT);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = sT[r];
      st.rsum += p[r];
    }
    pv_update(st.o0, st.o1, vt_lds, t, l32, h, pack8(p), pack8(p + 8));
  }
}

// Waves per SIMD each mode is compiled for (register budget 512/n per lane).
template <int MODE>
struct RowOccupancy {
  static constexpr int value = MODE == kRowLse ? 4 : 3;
};

template <int MODE>
__global__ void __launch_bounds__(256, RowOccupancy<MODE>::value) rows_bf16_kernel(FwdArgs a, int nqb) {
  constexpr bool kNeedV = (MODE != kRowLse);
  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * kKTile];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kNeedV ? 2 * kVTile : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // heaviest query blocks first; consecutive workgroups take different heads.
  // Workgroups go to the 8 XCDs round-robin, so with B*H a multiple of 8 each
  // XCD serves the same B*H/8 heads throughout and keeps their K/V in its L2.
  const int bh = blockIdx.x % a.BH;
  const int qb = nqb - 1 - blockIdx.x / a.BH;
  const int T = a.T;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * w;              // first row of this wave
  const bool wave_live = qw0 < T;
  const int kd = qw0 / kBN;                 // the tile holding this wave's diagonal
  const size_t head = (size_t)bh * T * kHeadDim;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;

  const int kend = min(q0 + kBM, T);        // keys [0, kend) are visible to some row
  const int nkt = (kend + kBN - 1) / kBN;

  // Q fragments: lane holds Q[qw0 + l32][16c + 8h .. +8) -- usable as the B
  // operand of S^T = K Q^T and as the A operand of S = Q K^T.
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, load_row_chunk(Q, qw0 + l32, T, 2 * c + h));

  // tile loaders: K as [key][d] rows; V transposed to [d][key] on the way in.
  u32x4 kreg[2], vreg[2];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      kreg[i] = load_row_clamped(K, key0 + (u >> 3), T, u & 7);
    }
    if constexpr (kNeedV) {
      const int kp = tid & 31, dc = tid >> 5;
      vreg[0] = load_row_clamped(V, key0 + 2 * kp, T, dc);
      vreg[1] = load_row_clamped(V, key0 + 2 * kp + 1, T, dc);
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
        const uint32_t even = __builtin_amdgcn_perm(a1, a0, 0x05040100u);  // d = 8dc + 2i
        const uint32_t odd = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // d = 8dc + 2i + 1
        *reinterpret_cast<uint32_t *>(vt + (8 * dc + 2 * i) * kVRow + 2 * kp) = even;
        *reinterpret_cast<uint32_t *>(vt + (8 * dc + 2 * i + 1) * kVRow + 2 * kp) = odd;
      }
    }
  };

  RowState st;
  st.o0 = zero16();
  st.o1 = zero16();
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
  st.rsum = 0.0f;

  float lseq[16];      // pass 2b: lse2 of this lane's 16 query rows (kNoRow past the end)
  bf16x8 ident[2];     // pass 2b: identity operand of the transpose
  const float *cin_blk = nullptr;
  float cin_next[2] = {0.0f, 0.0f};
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  if constexpr (MODE == kRowShare) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = qw0 + acc_row(r, h);
      lseq[r] = row < T ? a.lse2[(size_t)bh * T + row] : kNoRow;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = (acc_row(8 * c + j, h) == l32) ? 1.0f : 0.0f;
      ident[c] = pack8(e);
    }
    const int qs = qw0 >> 5;
    cin_blk = a.cin + (size_t)bh * cin_floats_per_head(T) + (size_t)16 * qs * (qs - 1);
  }
  // committed demand of this wave's block on keys kt*64 + 32t + l32 (0 on and
  // past the diagonal, where no earlier row of the sequence sees the key)
  auto load_cin = [&](int kt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = kt * kBN + 32 * t + l32;
      cin_next[t] = (wave_live && key < qw0) ? cin_blk[key] : 0.0f;
    }
  };

  // Wait here for the one-time loads (Q fragments, row LSEs).  Without this
  // the compiler cannot prove them complete on every path into the loop and
  // waits for all outstanding loads -- the tile prefetch included -- at their
  // first use in every iteration.
  __builtin_amdgcn_s_waitcnt(0);

  load_tile(0);
  store_tile(0);
  if constexpr (MODE == kRowShare) load_cin(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    float base[2];
    if constexpr (MODE == kRowShare) {
#pragma unroll
      for (int t = 0; t < 2; ++t) base[t] = fmaxf(cin_next[t] + a.eps, eps_floor);
    }
    if (kt + 1 < nkt) {
      load_tile(kt + 1);
      if constexpr (MODE == kRowShare) load_cin(kt + 1);
    }
    const __bf16 *kt_lds = sK + buf * kKTile;
    const __bf16 *vt_lds = sV + (kNeedV ? buf * kVTile : 0);
    const int kb = kt * kBN;
    if (wave_live && kt <= kd) {
      if constexpr (MODE == kRowShare) {
        if (kt < kd) share_tile<false>(st, qf, lseq, ident, base, kt_lds, vt_lds, kb, qw0, l32, h, a.c2);
        else share_tile<true>(st, qf, lseq, ident, base, kt_lds, vt_lds, kb, qw0, l32, h, a.c2);
      } else {
        if (kt < kd) st_tile<MODE, false>(st, qf, kt_lds, vt_lds, kb, qw0, l32, h, a.c2);
        else st_tile<MODE, true>(st, qf, kt_lds, vt_lds, kb, qw0, l32, h, a.c2);
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const int row = qw0 + l32;
  float denom;
  if constexpr (MODE == kRowShare) {
    denom = both_halves_sum(st.rsum);
  } else {
    denom = both_halves_sum(st.l_run);
    if (h == 0 && row < T) {
      const float lse2 = st.m_run + __builtin_log2f(denom);
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
        lo[0] = pack_bf16x2(st.o0[4 * g] * inv, st.o0[4 * g + 1] * inv);
        lo[1] = pack_bf16x2(st.o0[4 * g + 2] * inv, st.o0[4 * g + 3] * inv);
        hi[0] = pack_bf16x2(st.o1[4 * g] * inv, st.o1[4 * g + 1] * inv);
        hi[1] = pack_bf16x2(st.o1[4 * g + 2] * inv, st.o1[4 * g + 3] * inv);
        *reinterpret_cast<u32x2 *>(O + d0) = lo;
        *reinterpret_cast<u32x2 *>(O + 32 + d0) = hi;
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2a

constexpr int kCB = 128;  // keys per workgroup (4 waves x 32)
constexpr int kCQ = 64;   // query rows per LDS tile (two 32-row blocks)

__global__ void __launch_bounds__(256) colsum_bf16_kernel(FwdArgs a, int nkb, int nqs) {
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][kCQ * kKRow];
  __shared__ __attribute__((aligned(16))) float sL[2][kCQ];

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

  __builtin_amdgcn_s_waitcnt(0);             // K fragments: see the row kernels

  const int qt0 = (kb * kCB) / kCQ;          // first 64-row query tile
  const int nqt = (T + kCQ - 1) / kCQ;
  u32x4 qreg[2];
  float lreg = 0.0f;
  bool lvalid = false;
  auto load_q = [&](int qt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      qreg[i] = load_row_clamped(Q, qt * kCQ + (u >> 3), T, u & 7);
    }
    if (tid < kCQ) {
      const int row = qt * kCQ + tid;
      lvalid = row < T;
      lreg = L2[lvalid ? row : T - 1];
    }
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(&sQ[buf][(u >> 3) * kKRow + (u & 7) * 8]) = qreg[i];
    }
    if (tid < kCQ) sL[buf][tid] = lvalid ? lreg : kNoRow;   // rows past the end bid nothing
  };

  float run = 0.0f;  // demand this half-lane's rows have put on `key` so far
  load_q(qt0);
  store_q(0);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) load_q(qt + 1);
    if (wave_live) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int qs = 2 * qt + sb;              // 32-row block
        if (qs >= nqs || 32 * qs + 31 < kw0) continue;   // block entirely before the keys
        f32x16 sc = zero16();
        const __bf16 *qrow = &sQ[buf][(32 * sb + l32) * kKRow];
#pragma unroll
        for (int c = 0; c < 4; ++c) sc = mfma32(lds_frag(qrow, c, h), kf[c], sc);
        if (32 * qs > kw0) {
          // demand committed before block qs: rows < 32 qs, both halves
          const float total = both_halves_sum(run);
          if (h == 0 && key < T) cin[(size_t)16 * qs * (qs - 1) + key] = total;
        }
        const bool diag = (32 * qs == kw0);
        float part = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 lq = *reinterpret_cast<const f32x4 *>(&sL[buf][32 * sb + 8 * g + 4 * h]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            float v = fast_exp2(__builtin_fmaf(sc[r], a.c2, -lq[i]));
            if (diag && l32 > acc_row(r, h)) v = 0.0f;
            part += v;
          }
        }
        run += part;
      }
    }
    if (qt + 1 < nqt) store_q(buf ^ 1);
    __syncthreads();
  }
  if (a.demand_out && wave_live) {
    const float total = both_halves_sum(run);
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
