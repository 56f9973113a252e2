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
//    come from d/16 32x32x16 bf16 MFMAs (head dimension d = 64 or 128); a
//    64-key tile is two such blocks, handled together.  Only the one tile holding a wave's diagonal
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
#include "tiles.hpp"

#include <float.h>

namespace attn {

constexpr int kBM = 128;        // query rows per workgroup (row kernels)
constexpr float kSumLimit = 18446744073709551616.0f;   // 2^64: largest tile sum kept

// Per-wave state of the row kernels.
template <int D>
struct RowState {
  f32x16 o[Geom<D>::kOBlocks];   // O^T[d][query]: o[i] holds d in [32i, 32i+32)
  float m_run;     // running max of the scaled logits (log2 units)
  float l_run;     // fp32 row sum of exp2(x - m_run) over this half's keys (kernels
                   // that output the log-sum-exp)
  f32x4 lsum;      // row sum, on the matrix cores, of the bf16 weights fed to P@V
                   // (tempered: exp2(x - m_run), pass 2b: the shares), all elements
                   // equal: the output's normaliser, so that the weights' bf16 rounding
                   // enters numerator and denominator alike
};

// Bring the running max up to the tile's (masked) maximum and rescale what
// has been accumulated against the old one.
template <int MODE, bool FP32SUM, bool DIAG, int D>
__device__ __forceinline__ void st_rescale(RowState<D> &st, const f32x16 *s, int qrel, int h,
                                           float c2) {
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
  const float m_new = fmaxf(st.m_run, tmax * c2);   // finite: every row sees its first key
  const float alpha = fast_exp2(st.m_run - m_new);  // 0 while m_run is still -inf
  if constexpr (FP32SUM) st.l_run *= alpha;
  if constexpr (!FP32SUM || MODE == kRowTempered) st.lsum *= alpha;
  if constexpr (MODE == kRowTempered) {
#pragma unroll
    for (int i = 0; i < Geom<D>::kOBlocks; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[i][r] *= alpha;
  }
  st.m_run = m_new;
}

template <bool DIAG>
__device__ __forceinline__ void st_weights(const f32x16 *s, float m_run, int qrel, int h, float c2,
                                           float *p) {
  const float mneg = -m_run;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float e = fast_exp2(__builtin_fmaf(s[t][r], c2, mneg));
      if (DIAG && 32 * t + acc_row(r, h) > qrel) e = 0.0f;
      p[16 * t + r] = e;
    }
  }
}

// Tempered softmax / pass-1 update for one 64-key tile (S^T orientation).
// The running max m_run is lazy: the tile is weighted against the current
// m_run directly, and the tile max is only taken (and the tile weighted
// again) when a lane's tile sum leaves [0, 2^64].  Weights that large are
// still exact in fp32 and bf16; an overflow, or the first tile, where
// m_run = -inf, shows up there as inf or NaN.  The tile sum is the fp32 one
// (FP32SUM) or the matrix-core row sum of the bf16 weights, which the output
// normaliser accumulates anyway.
template <int MODE, bool FP32SUM, bool DIAG, int D, int VR>
__device__ __forceinline__ void st_tile(RowState<D> &st, const bf16x8 *qf, const bf16x8 &sel,
                                        const __bf16 *kt_lds, const __bf16 *v_lds, int kb,
                                        int qw0, int l32, int h, float c2) {
  f32x16 s[2] = {zero16(), zero16()};
  const __bf16 *krow0 = kt_lds + l32 * Geom<D>::kKRow;
  const __bf16 *krow1 = kt_lds + (32 + l32) * Geom<D>::kKRow;
#pragma unroll
  for (int c = 0; c < Geom<D>::kChunks; ++c) {
    s[0] = mfma32(lds_frag(krow0, c, h), qf[c], s[0]);
    s[1] = mfma32(lds_frag(krow1, c, h), qf[c], s[1]);
  }
  // lane: query qw0 + l32; element (t, r): key kb + 32t + acc_row(r, h)
  const int qrel = qw0 + l32 - kb;   // keys with 32t + acc_row <= qrel are visible
  if constexpr (FP32SUM) {
    float p[32];
    st_weights<DIAG>(s, st.m_run, qrel, h, c2, p);
    float ts = p[0];   // the weights are >= +0: the same bits as 0 + p[0] + ...
#pragma unroll
    for (int i = 1; i < 32; ++i) ts += p[i];
    if (__ballot(!(ts <= kSumLimit)) != 0ull) {
      st_rescale<MODE, FP32SUM, DIAG, D>(st, s, qrel, h, c2);
      st_weights<DIAG>(s, st.m_run, qrel, h, c2, p);
      ts = p[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) ts += p[i];
    }
    st.l_run += ts;
    if constexpr (MODE == kRowTempered) {
      // the output is normalised by the sum of the same bf16 weights (on the
      // matrix cores), the log-sum-exp by the fp32 sum
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 pf0 = pack8(p + 16 * t), pf1 = pack8(p + 16 * t + 8);
        st.lsum = mfma16(sel, pf0, st.lsum);
        st.lsum = mfma16(sel, pf1, st.lsum);
        pv_update_d<D, VR>(st.o, v_lds, t, pf0, pf1);
      }
    }
  } else {
    // the bf16 weights and their matrix-core row sum, the output's normaliser
    f32x4 tsum;
    bf16x8 pf[4];
    auto weigh = [&]() {
      const float mneg = -st.m_run;
      tsum = zero4();
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(__builtin_fmaf(s[t][r], c2, mneg));
          if (DIAG && 32 * t + acc_row(r, h) > qrel) e = 0.0f;
          p[r] = e;
        }
        pf[2 * t] = pack8(p);
        pf[2 * t + 1] = pack8(p + 8);
        tsum = mfma16(sel, pf[2 * t], tsum);
        tsum = mfma16(sel, pf[2 * t + 1], tsum);
      }
    };
    weigh();
    if (__ballot(!(tsum[0] <= kSumLimit)) != 0ull) {
      st_rescale<MODE, FP32SUM, DIAG, D>(st, s, qrel, h, c2);
      weigh();
    }
    st.lsum += tsum;
    if constexpr (MODE == kRowTempered) {
#pragma unroll
      for (int t = 0; t < 2; ++t) pv_update_d<D, VR>(st.o, v_lds, t, pf[2 * t], pf[2 * t + 1]);
    }
  }
}

// Pass-2b constant B operands, built once per wave.  Slot (h, e) of operand
// j carries query acc_row(8j + e, h) of the wave's block (the order in which
// a lane of the S layout holds its 16 queries); column n is query n.
struct ShareConsts {
  bf16x8 upre[2];   // inclusive prefix: 1 where the slot's query <= query n
  bf16x8 ident[2];  // transpose: 1 where the slot's query == query n
  bf16x8 bone;      // committed-demand slots: 1 in slots (0, 0..1), else 0
};

__device__ __forceinline__ ShareConsts share_consts(int l32, int h) {
  ShareConsts c;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float u[8], id[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qs = acc_row(8 * j + e, h);
      u[e] = qs <= l32 ? 1.0f : 0.0f;
      id[e] = qs == l32 ? 1.0f : 0.0f;
    }
    c.upre[j] = pack8(u);
    c.ident[j] = pack8(id);
  }
  const float one = h == 0 ? 1.0f : 0.0f;
  c.bone = to_bf16x8(one, one, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f);
  return c;
}

// Pass-2b update for one 64-key tile, one 32-key sub-tile at a time.
//  1. S = Q K^T with lane = key and the 16 queries in registers; bids
//     p = exp2(c2 s - lse2(query)) (zero above the diagonal), packed to bf16.
//  2. The bids, as the A operand (row = key, slot = query), are multiplied by
//     three constant B operands, transposing them to lane = query:
//       D = committed + eps + sum of the bids of the block's rows up to and
//           including the column's query (the inclusive column prefix;
//           committed + eps enters as its stored bf16 (hi, lo) pair);
//       P = the bids themselves.
//  3. share = P / D, the row sums, and share @ V on the matrix cores.
// lseq: the lse2 of the lane's 16 queries in accumulator order (registers),
// or with LDS_LSE the wave's 32 row values in row order (LDS).
template <bool DIAG, bool LDS_LSE = false>
__device__ __forceinline__ void share_bids(const f32x16 &s, const float *lseq, int krel, int h,
                                           float c2, bf16x8 &pa0, bf16x8 &pa1) {
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float l = LDS_LSE ? lseq[acc_row(r, h)] : lseq[r];
    float e = fast_exp2(__builtin_fmaf(s[r], c2, -l));
    if (DIAG && acc_row(r, h) < krel) e = 0.0f;
    p[r] = e;
  }
  pa0 = pack8(p);
  pa1 = pack8(p + 8);
}

// D (inclusive prefix + committed + eps) and P, both transposed to lane = query.
__device__ __forceinline__ void share_prefix(const bf16x8 &pa0, const bf16x8 &pa1, uint32_t base,
                                             const ShareConsts &sc, f32x16 &d, f32x16 &pt) {
  const u32x4 bw = {base, 0u, 0u, 0u};
  d = mfma32(pa0, sc.upre[0], zero16());
  pt = mfma32(pa0, sc.ident[0], zero16());
  d = mfma32(pa1, sc.upre[1], d);
  pt = mfma32(pa1, sc.ident[1], pt);
  d = mfma32(__builtin_bit_cast(bf16x8, bw), sc.bone, d);
}

__device__ __forceinline__ void share_values(const f32x16 &d, const f32x16 &pt, bf16x8 &sf0,
                                             bf16x8 &sf1) {
  float sh[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) sh[r] = pt[r] * fast_rcp(d[r]);
  sf0 = pack8(sh);
  sf1 = pack8(sh + 8);
}

template <bool DIAG, int D, int VR>
__device__ __forceinline__ void share_tile(RowState<D> &st, const bf16x8 *qf, const float *lseq,
                                           const ShareConsts &sc_, const bf16x8 &sel,
                                           const uint32_t *base,
                                           const __bf16 *kt_lds, const __bf16 *v_lds, int kb,
                                           int qw0, int l32, int h, float c2) {
  // The two 32-key sub-tiles are independent until share@V; their stages are
  // written staggered so that each sub-tile's matrix-core work overlaps the
  // other's vector work:
  //   scores 0,1 | bids 0 | prefix 0, bids 1 | prefix 1, shares 0 |
  //   P@V 0, shares 1 | P@V 1
  // sub-tile t, lane: key kb + 32t + l32; element r: query qw0 + acc_row(r, h)
  const __bf16 *krow0 = kt_lds + l32 * Geom<D>::kKRow;
  const __bf16 *krow1 = kt_lds + (32 + l32) * Geom<D>::kKRow;
  const int krel0 = kb + l32 - qw0;   // key visible to rows with acc_row >= krel
  if constexpr (D > 64) {
    // d = 128: one sub-tile after the other, so that only one sub-tile's
    // scores, prefix and shares are live at a time; the row LSEs are read
    // from LDS (lseq: the wave's 32 rows)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const __bf16 *krow = t == 0 ? krow0 : krow1;
      f32x16 sc = zero16();
#pragma unroll
      for (int c = 0; c < Geom<D>::kChunks; ++c) sc = mfma32(qf[c], lds_frag(krow, c, h), sc);
      bf16x8 pa0, pa1, sf0, sf1;
      share_bids<DIAG, true>(sc, lseq, krel0 + 32 * t, h, c2, pa0, pa1);
      f32x16 dd, pt;
      share_prefix(pa0, pa1, base[t], sc_, dd, pt);
      share_values(dd, pt, sf0, sf1);
      st.lsum = mfma16(sel, sf0, st.lsum);
      st.lsum = mfma16(sel, sf1, st.lsum);
      pv_update_d<D, VR>(st.o, v_lds, t, sf0, sf1);
    }
    return;
  }
  f32x16 s0 = zero16(), s1 = zero16();
#pragma unroll
  for (int c = 0; c < Geom<D>::kChunks; ++c) {
    s0 = mfma32(qf[c], lds_frag(krow0, c, h), s0);
    s1 = mfma32(qf[c], lds_frag(krow1, c, h), s1);
  }
  bf16x8 pa00, pa01, pa10, pa11;
  share_bids<DIAG>(s0, lseq, krel0, h, c2, pa00, pa01);
  // sub-tile t transposed, lane: query qw0 + l32; element r: key kb + 32t + acc_row(r, h)
  f32x16 d0, pt0, d1, pt1;
  share_prefix(pa00, pa01, base[0], sc_, d0, pt0);
  share_bids<DIAG>(s1, lseq, krel0 + 32, h, c2, pa10, pa11);
  share_prefix(pa10, pa11, base[1], sc_, d1, pt1);
  bf16x8 sf00, sf01, sf10, sf11;
  share_values(d0, pt0, sf00, sf01);
  st.lsum = mfma16(sel, sf00, st.lsum);
  st.lsum = mfma16(sel, sf01, st.lsum);
  pv_update_d<D, VR>(st.o, v_lds, 0, sf00, sf01);
  share_values(d1, pt1, sf10, sf11);
  st.lsum = mfma16(sel, sf10, st.lsum);
  st.lsum = mfma16(sel, sf11, st.lsum);
  pv_update_d<D, VR>(st.o, v_lds, 1, sf10, sf11);
}

// Waves per SIMD each mode is compiled for (register budget 512/n per lane).
template <int MODE, int D>
struct RowOccupancy {
  static constexpr int value =
      MODE == kRowLse ? (D > 64 ? 3 : 4) : (MODE == kRowShare || D > 64 ? 2 : 3);
};

// FP32SUM: row sums in fp32 on the vector ALUs (exact log-sum-exp output);
// otherwise on the matrix cores over the bf16 weights.
template <int MODE, bool FP32SUM, int D, bool SPLIT = false>
__global__ void __launch_bounds__(256, (RowOccupancy<MODE, D>::value))
    rows_bf16_kernel(FwdArgs a, int nqb) {
  using G = Geom<D>;
  constexpr bool kNeedV = (MODE != kRowLse);
  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * G::kKTile];
  // V tile row stride: P@V reads V only transposed, half a wave four rows
  // of 64 bytes per load, which is free of bank conflicts when the stride is
  // 64 or 192 bytes off a multiple of 256 (d + 32 elements).  That padding
  // is used where the registers allow it (the tempered kernel at d = 128,
  // where the conflicts cost most); elsewhere V has K's d + 8 and meets 2-way
  // conflicts.
  constexpr int kVR = (MODE == kRowTempered && D == 128) ? D + 32 : G::kKRow;
  constexpr int kVT = kBN * kVR;
  __shared__ __attribute__((aligned(16))) __bf16 sV[kNeedV ? 2 * kVT : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // heaviest query blocks first; consecutive workgroups take different heads.
  // Workgroups go to the 8 XCDs round-robin, so with B*H a multiple of 8 each
  // XCD serves the same B*H/8 heads throughout and keeps their K/V in its L2.
  // Rows are positions: query row r of Q is position P + r, and keys are
  // indexed from 0.  A whole prefill has P = 0; a later chunk starts at P > 0
  // and the blocks cover positions from vrow0 = P rounded down to kBM, the
  // positions before P standing for no row (no loads, no stores, no bids).
  // With a key split (SPLIT: dilution stages on small grids) workgroup b
  // takes range b / (nqb * BH) of its query block's key tiles.
  const int ks = SPLIT ? a.ksplit : 1;
  const int nitems = nqb * a.BH;
  const int split = SPLIT ? (int)blockIdx.x / nitems : 0;
  const int item = SPLIT ? (int)blockIdx.x % nitems : (int)blockIdx.x;
  const int bh = item % a.BH;
  const int qb = a.vrow0 / kBM + nqb - 1 - item / a.BH;
  const int T = a.T, Tq = a.Tq, P = T - Tq;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * w;              // first position of this wave
  const bool wave_live = qw0 < T && qw0 + 32 > P;
  const int kd = qw0 / kBN;                 // the tile holding this wave's diagonal
  const size_t qhead = (size_t)bh * Tq * D, khead = (size_t)bh * a.kstride * D;
  const float c2 = head_c2(a, bh);
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + qhead;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + khead;
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + khead;

  const int kend = min(q0 + kBM, T);        // keys [0, kend) are visible to some row
  const int nkt_all = (kend + kBN - 1) / kBN;
  const int kt0 = SPLIT ? split * nkt_all / ks : 0;                 // tiles [kt0, nkt)
  const int nkt = SPLIT ? (split + 1) * nkt_all / ks : nkt_all;

  // Q fragments: lane holds Q[qw0 + l32][16c + 8h .. +8) -- usable as the B
  // operand of S^T = K Q^T and as the A operand of S = Q K^T.
  bf16x8 qf[G::kChunks];
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c)
    qf[c] = __builtin_bit_cast(bf16x8, load_row_chunk<D>(Q, qw0 + l32 - P, Tq, 2 * c + h));

  // tile loaders: K and V as [key][d] rows (P@V reads V transposed from its
  // row-major tile).  Buffer loads with per-lane byte offsets fixed for the
  // whole loop; keys past the end of the sequence read as zeros.  Each
  // thread moves D/32 16-byte chunks of K and of V per tile.
  constexpr int kRowBytes = 2 * D, kRowChunks = D / 8;
  constexpr int kKL = D / 32;
  u32x4 kreg[kKL], vreg[kKL];
  auto load_tile = [&](int kt) {
    const int key0 = kt * kBN;                          // < T for every tile loaded
    const int bytes = (T - key0) * kRowBytes;
    const auto rk = make_rsrc(K + (size_t)key0 * D, bytes);
#pragma unroll
    for (int i = 0; i < kKL; ++i) kreg[i] = buf_load16(rk, 16u * (tid + 256 * i));
    if constexpr (kNeedV) {
      const auto rv = make_rsrc(V + (size_t)key0 * D, bytes);
#pragma unroll
      for (int i = 0; i < kKL; ++i) vreg[i] = buf_load16(rv, 16u * (tid + 256 * i));
    }
  };
  auto store_tile = [&](int buf) {
    __bf16 *k = sK + buf * G::kKTile;
    __bf16 *vv = sV + buf * kVT;
#pragma unroll
    for (int i = 0; i < kKL; ++i) {
      const int u = tid + 256 * i;
      const int row = u / kRowChunks, e = (u % kRowChunks) * 8, off = row * G::kKRow + e;
      *reinterpret_cast<u32x4 *>(k + off) = kreg[i];
      if constexpr (kNeedV)
        *reinterpret_cast<u32x4 *>(vv + (kVR == G::kKRow ? off : row * kVR + e)) = vreg[i];
    }
  };

  RowState<D> st;
#pragma unroll
  for (int i = 0; i < G::kOBlocks; ++i) st.o[i] = zero16();
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
  st.lsum = zero4();
  const bf16x8 sel = rowsum_selector(lane);

  // pass 2b: lse2 of this lane's 16 query rows (kNoRow for no row); at d = 128
  // the wave's 32 values sit in LDS instead
  constexpr bool kLdsLse = D > 64;
  float lseq[kLdsLse ? 1 : 16];
  __shared__ float sLse[MODE == kRowShare && kLdsLse ? kBM : 1];
  ShareConsts sc;      // pass 2b: constant operands of the prefix and transpose
  const uint32_t *cin_blk = nullptr;
  uint32_t cin_next[2] = {0u, 0u};
  // committed + eps of a key no earlier row sees (on and past the diagonal)
  const uint32_t eps_word = split2_bf16(fmaxf(a.eps, FLT_MIN));
  if constexpr (MODE == kRowShare) {
    if constexpr (kLdsLse) {
      const int lr = qw0 + l32 - P;
      if (h == 0) sLse[32 * w + l32] = (unsigned)lr < (unsigned)Tq ? a.lse2[(size_t)bh * Tq + lr] : kNoRow;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = qw0 + acc_row(r, h) - P;
        lseq[r] = (unsigned)lr < (unsigned)Tq ? a.lse2[(size_t)bh * Tq + lr] : kNoRow;
      }
    }
    sc = share_consts(l32, h);
    cin_blk = reinterpret_cast<const uint32_t *>(a.cin) + (size_t)bh * cin_floats_per_head(T, a.vrow0) +
              cin_block_offset(qw0 >> 5, a.vrow0);
  }
  // committed demand (+ eps, as a bf16 pair) of this wave's block on keys
  // kt*64 + 32t + l32; past the diagonal block no row of it sees the key, and
  // the table holds no entry for keys past the end
  const int cin_end = min(qw0 + 32, T);
  auto load_cin = [&](int kt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = kt * kBN + 32 * t + l32;
      cin_next[t] = (wave_live && key < cin_end) ? cin_blk[key] : eps_word;
    }
  };

  // Wait here for the one-time loads (Q fragments, row LSEs).  Without this
  // the compiler cannot prove them complete on every path into the loop and
  // waits for all outstanding loads -- the tile prefetch included -- at their
  // first use in every iteration.
  __builtin_amdgcn_s_waitcnt(0);

  if (!SPLIT || kt0 < nkt) {                 // an empty range loads nothing
    load_tile(kt0);
    store_tile(0);
    if constexpr (MODE == kRowShare) load_cin(kt0);
  }
  __syncthreads();

  for (int kt = kt0; kt < nkt; ++kt) {
    const int buf = (kt - kt0) & 1;
    uint32_t base[2];
    if constexpr (MODE == kRowShare) {
#pragma unroll
      for (int t = 0; t < 2; ++t) base[t] = cin_next[t];
    }
    if (kt + 1 < nkt) {
      load_tile(kt + 1);
      if constexpr (MODE == kRowShare) load_cin(kt + 1);
    }
    const __bf16 *kt_lds = sK + buf * G::kKTile;
    const __bf16 *v_lds = sV + (kNeedV ? buf * kVT : 0);
    const int kb = kt * kBN;
    if (wave_live && kt <= kd) {
      if constexpr (MODE == kRowShare) {
        const float *lsrc = kLdsLse ? sLse + 32 * w : lseq;
        if (kt < kd) share_tile<false, D, kVR>(st, qf, lsrc, sc, sel, base, kt_lds, v_lds, kb, qw0, l32, h, c2);
        else share_tile<true, D, kVR>(st, qf, lsrc, sc, sel, base, kt_lds, v_lds, kb, qw0, l32, h, c2);
      } else {
        if (kt < kd) st_tile<MODE, FP32SUM, false, D, kVR>(st, qf, sel, kt_lds, v_lds, kb, qw0, l32, h, c2);
        else st_tile<MODE, FP32SUM, true, D, kVR>(st, qf, sel, kt_lds, v_lds, kb, qw0, l32, h, c2);
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  const int lr = qw0 + l32 - P;               // this lane's query row
  const bool row_ok = (unsigned)lr < (unsigned)Tq;
  // log-sum-exp: the fp32 sum; output: the sum of its bf16 weights
  const float denom = FP32SUM ? both_halves_sum(st.l_run) : st.lsum[0];
  const float onorm = MODE == kRowTempered ? st.lsum[0] : denom;
  if constexpr (SPLIT) {
    // partial results of this key range: (max, sum) or the row sum, and the
    // unnormalised share @ V; a range past a wave's diagonal leaves (-inf, 0, 0)
    if (!row_ok) return;
    const size_t rec = ((size_t)bh * Tq + lr) * ks + split;
    if (h == 0) {
      a.part_ml[2 * rec] = st.m_run;
      a.part_ml[2 * rec + 1] = denom;
    }
    if constexpr (MODE == kRowShare) {
      float *po = a.part_o + rec * D;
#pragma unroll
      for (int i = 0; i < G::kOBlocks; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {st.o[i][4 * g], st.o[i][4 * g + 1], st.o[i][4 * g + 2], st.o[i][4 * g + 3]};
          *reinterpret_cast<f32x4 *>(po + 32 * i + 8 * g + 4 * h) = v;
        }
    }
    return;
  }
  if constexpr (MODE == kRowShare) {
    if (a.rowsum_out && h == 0 && row_ok) a.rowsum_out[(size_t)bh * Tq + lr] = denom;
  } else {
    if (h == 0 && row_ok) {
      const float lse2 = st.m_run + __builtin_log2f(denom);
      if (a.lse2) a.lse2[(size_t)bh * Tq + lr] = lse2;
      if (a.lse_nat) a.lse_nat[(size_t)bh * Tq + lr] = lse2 * kLn2;
    }
  }
  if constexpr (MODE != kRowLse) {
    if (row_ok) {
      const float inv = 1.0f / onorm;
      __bf16 *O = reinterpret_cast<__bf16 *>(a.out) + qhead + (size_t)lr * D;
#pragma unroll
      for (int i = 0; i < G::kOBlocks; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w;
          w[0] = pack_bf16x2(st.o[i][4 * g] * inv, st.o[i][4 * g + 1] * inv);
          w[1] = pack_bf16x2(st.o[i][4 * g + 2] * inv, st.o[i][4 * g + 3] * inv);
          *reinterpret_cast<u32x2 *>(O + 32 * i + 8 * g + 4 * h) = w;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- pass 2a

constexpr int kCB = 128;  // keys per workgroup (4 waves x 32)
constexpr int kCQ = 64;   // query rows per LDS tile (two 32-row blocks)

// Sum of the bids exp2(sc) down this lane's 16 query rows of a 32x32 block
// (S layout: lane = key); on the diagonal block rows before the key see
// nothing of it.
template <bool DIAG>
__device__ __forceinline__ float colsum_bids(const f32x16 &sc, int l32, int h) {
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float v = fast_exp2(sc[r]);
    if (DIAG && l32 > acc_row(r, h)) v = 0.0f;
    part += v;
  }
  return part;
}

template <int D>
__global__ void __launch_bounds__(256) colsum_bf16_kernel(FwdArgs a, int nkb, int nqs) {
  using G = Geom<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[2][kCQ * G::kKRow];
  __shared__ __attribute__((aligned(16))) float sL[2][kCQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  // Query tiles are walked by position (query row r of Q is position P + r);
  // positions before P, from vrow0 on, are no row and bid nothing.
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;          // longest column walks first
  const int T = a.T, Tq = a.Tq, P = T - Tq;
  const int kw0 = kb * kCB + 32 * w;          // first key of this wave
  const bool wave_live = kw0 < T;
  const int key = kw0 + l32;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + (size_t)bh * Tq * D;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + (size_t)bh * a.kstride * D;
  const float c2 = head_c2(a, bh);
  const float *L2 = a.lse2 + (size_t)bh * Tq;
  // committed demand + eps of each (32-row block, key), stored as a bf16 pair
  uint32_t *cin = reinterpret_cast<uint32_t *>(a.cin) + (size_t)bh * cin_floats_per_head(T, a.vrow0);
  const float eps_floor = fmaxf(a.eps, FLT_MIN);
  auto committed_word = [&](float total) { return split2_bf16(fmaxf(total + a.eps, eps_floor)); };

  bf16x8 kf[G::kChunks];
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c)
    kf[c] = __builtin_bit_cast(bf16x8, load_row_chunk<D>(K, key, T, 2 * c + h));
  // demand this half-lane's rows have put on `key` so far; the lower half
  // starts from the demand committed before position P
  float run = 0.0f;
  if (a.demand_in && h == 0 && key < T) run = a.demand_in[(size_t)bh * a.kstride + key];

  __builtin_amdgcn_s_waitcnt(0);             // K fragments: see the row kernels

  const int qt0 = max(kb * kCB, a.vrow0) / kCQ;   // first 64-row query tile
  const int nqt = (T + kCQ - 1) / kCQ;
  constexpr int kQL = D / 32, kRowChunks = D / 8;   // 16-byte Q loads per thread per tile
  u32x4 qreg[kQL];
  float lreg = 0.0f;
  bool lvalid = false;
  auto load_q = [&](int qt) {
    // rows lr0.. of Q; only a chunk's first tiles start before row 0 (lr0 < 0),
    // and their lanes for positions before P get an offset past the range
    const int lr0 = qt * kCQ - P, b0 = max(lr0, 0);   // b0 < Tq for every tile loaded
    const auto rq = make_rsrc(Q + (size_t)b0 * D, (Tq - b0) * (D * 2));
    const int sh = (lr0 - b0) * (D * 2);              // <= 0
#pragma unroll
    for (int i = 0; i < kQL; ++i) {
      const int off = 16 * (tid + 256 * i) + sh;
      qreg[i] = buf_load16(rq, off < 0 ? kNoOffset : (uint32_t)off);
    }
    if (tid < kCQ) {
      const int lr = lr0 + tid;
      lvalid = (unsigned)lr < (unsigned)Tq;
      lreg = L2[lvalid ? lr : 0];
    }
  };
  auto store_q = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kQL; ++i) {
      const int u = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(&sQ[buf][(u / kRowChunks) * G::kKRow + (u % kRowChunks) * 8]) = qreg[i];
    }
    if (tid < kCQ) sL[buf][tid] = lvalid ? -lreg : -kNoRow;   // no row: bids nothing
  };

  // Scores of the 32x32 block (rows 32 sb.. of Q buffer `buf`, this wave's
  // keys) in the S layout, as log2 of the bid: c2 s - lse2 of the query
  // (element r: query acc_row(r, h)).
  auto block_scores = [&](int buf, int sb) {
    f32x16 sc = zero16();
    const __bf16 *qrow = &sQ[buf][(32 * sb + l32) * G::kKRow];
#pragma unroll
    for (int c = 0; c < G::kChunks; ++c) {
      const bf16x8 qa = lds_frag(qrow, c, h);
      sc = mfma32(qa, kf[c], sc);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 nl = *reinterpret_cast<const f32x4 *>(&sL[buf][32 * sb + 8 * g + 4 * h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[4 * g + i] = __builtin_fmaf(sc[4 * g + i], c2, nl[i]);
    }
    return sc;
  };
  // demand committed before block qs (rows < 32 qs, both halves)
  auto commit = [&](int qs, float r) {
    const float total = both_halves_sum(r);
    if (h == 0 && key < T) cin[cin_block_offset(qs, a.vrow0) + key] = committed_word(total);
  };

  load_q(qt0);
  store_q(0);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt + 1 < nqt) load_q(qt + 1);
    if (wave_live) {
      const int qs0 = 2 * qt;
      if (32 * qs0 > kw0 && qs0 + 1 < nqs) {
        // both blocks below the diagonal block and inside the sequence: the
        // two independent MFMA chains interleave
        const f32x16 s0 = block_scores(buf, 0), s1 = block_scores(buf, 1);
        const float r0 = run;
        const float r1 = r0 + colsum_bids<false>(s0, l32, h);
        run = r1 + colsum_bids<false>(s1, l32, h);
        const float t0 = both_halves_sum(r0), t1 = both_halves_sum(r1);
        if (h == 0 && key < T) {
          cin[cin_block_offset(qs0, a.vrow0) + key] = committed_word(t0);
          cin[cin_block_offset(qs0 + 1, a.vrow0) + key] = committed_word(t1);
        }
      } else {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int qs = qs0 + sb;                  // 32-row block
          if (qs >= nqs || 32 * qs + 31 < kw0) continue;   // past the end, or before the keys
          const f32x16 sc = block_scores(buf, sb);
          commit(qs, run);
          run += (32 * qs == kw0) ? colsum_bids<true>(sc, l32, h) : colsum_bids<false>(sc, l32, h);
        }
      }
    }
    if (qt + 1 < nqt) store_q(buf ^ 1);
    __syncthreads();
  }
  if (a.demand_out && wave_live) {
    const float total = both_halves_sum(run);
    if (h == 0 && key < T) a.demand_out[(size_t)bh * a.kstride + key] = total;
  }
}

// Combine the key ranges of the dilution row stages, in range order.
// LSE stage: lse2 = M + log2 sum_s l_s 2^(m_s - M), one thread per row.
__global__ void __launch_bounds__(256) combine_lse_kernel(FwdArgs a) {
  const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= (size_t)a.BH * a.Tq) return;
  const int ks = a.ksplit;
  const float *ml = a.part_ml + row * ks * 2;
  float M = -INFINITY;
  for (int i = 0; i < ks; ++i) M = fmaxf(M, ml[2 * i]);
  float L = 0.0f;
  for (int i = 0; i < ks; ++i)
    if (ml[2 * i + 1] > 0.0f) L += ml[2 * i + 1] * fast_exp2(ml[2 * i] - M);
  const float lse2 = M + __builtin_log2f(L);
  if (a.lse2) a.lse2[row] = lse2;
  if (a.lse_nat) a.lse_nat[row] = lse2 * kLn2;
}

// Shares stage: out = sum_s o_s / sum_s r_s; one thread per (row, d).
template <int D>
__global__ void __launch_bounds__(256) combine_share_kernel(FwdArgs a) {
  const size_t row = (size_t)blockIdx.x * (256 / D) + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (row >= (size_t)a.BH * a.Tq) return;
  const int ks = a.ksplit;
  const float *ml = a.part_ml + row * ks * 2;
  const float *po = a.part_o + row * ks * D;
  float l = 0.0f, o = 0.0f;
  for (int i = 0; i < ks; ++i) {
    l += ml[2 * i + 1];
    o += po[(size_t)i * D + d];
  }
  reinterpret_cast<__bf16 *>(a.out)[row * D + d] = (__bf16)(o / l);
  if (a.rowsum_out && d == 0) a.rowsum_out[row] = l;
}

template <int D>
static void launch_rows_d(int mode, const FwdArgs &a, int nqb, hipStream_t s) {
  const int ks = mode == kRowTempered ? 1 : a.ksplit;
  dim3 grid((unsigned)(nqb * a.BH * ks)), block(256);
  if (ks > 1) {
    const size_t rows = (size_t)a.BH * a.Tq;
    if (mode == kRowLse) {
      hipLaunchKernelGGL((rows_bf16_kernel<kRowLse, true, D, true>), grid, block, 0, s, a, nqb);
      hipLaunchKernelGGL(combine_lse_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL((rows_bf16_kernel<kRowShare, false, D, true>), grid, block, 0, s, a, nqb);
      hipLaunchKernelGGL(combine_share_kernel<D>, dim3((unsigned)((rows * D + 255) / 256)), dim3(256),
                         0, s, a);
    }
    return;
  }
  switch (mode) {
    case kRowTempered:
      // an exact log-sum-exp output needs fp32 row sums
      if (a.lse2 || a.lse_nat)
        hipLaunchKernelGGL((rows_bf16_kernel<kRowTempered, true, D>), grid, block, 0, s, a, nqb);
      else
        hipLaunchKernelGGL((rows_bf16_kernel<kRowTempered, false, D>), grid, block, 0, s, a, nqb);
      break;
    case kRowLse:
      hipLaunchKernelGGL((rows_bf16_kernel<kRowLse, true, D>), grid, block, 0, s, a, nqb);
      break;
    default:
      hipLaunchKernelGGL((rows_bf16_kernel<kRowShare, false, D>), grid, block, 0, s, a, nqb);
      break;
  }
}

hipError_t launch_rows_bf16(int mode, const FwdArgs &a, hipStream_t s) {
  const int nqb = (a.T + kBM - 1) / kBM - a.vrow0 / kBM;   // blocks from position vrow0
  if (a.D == 128) launch_rows_d<128>(mode, a, nqb, s);
  else launch_rows_d<64>(mode, a, nqb, s);
  return hipGetLastError();
}

hipError_t launch_colsum_bf16(const FwdArgs &a, hipStream_t s) {
  const int nkb = (a.T + kCB - 1) / kCB;
  const int nqs = (a.T + 31) / 32;
  const dim3 grid((unsigned)(nkb * a.BH)), block(256);
  if (a.D == 128) hipLaunchKernelGGL(colsum_bf16_kernel<128>, grid, block, 0, s, a, nkb, nqs);
  else hipLaunchKernelGGL(colsum_bf16_kernel<64>, grid, block, 0, s, a, nkb, nqs);
  return hipGetLastError();
}

}  // namespace attn
