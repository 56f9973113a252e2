// bwd_bf16.hip -- bf16 backward kernels for gfx950 (exact gradients).
//
// "DilutionAttention v0.1.0 - results": the operator ("The operator") and
// the release's training kernels with exact gradients ("Everything behind
// these charts").  With p the bids, C the committed demand, D = C + p + eps,
// sigma = p / D, r_i = sum_j sigma_ij, a = sigma / r, o = a v and the
// incoming gradient dO, the chain rule gives (per head)
//   dV_j      = sum_i a_ij dO_i
//   dA_ij     = <dO_i, v_j>,  delta_i = <dO_i, o_i>
//   dsigma_ij = (dA_ij - delta_i) / r_i
//   g_ij      = dsigma_ij p_ij / D_ij^2
//   dp_ij     = dsigma_ij / D_ij - G_ij,   G_ij = sum_{i'' >= i} g_i''j
//               (every later row's committed demand contains p_ij)
//   dS_ij     = p_ij (dp_ij - rho_i),      rho_i = sum_j p_ij dp_ij
//   dQ_i = c sum_j dS_ij k_j,   dK_j = c sum_i dS_ij q_i,   c = tau / sqrt(d),
//   dL/dtau = sum_ij dS_ij <q_i, k_j> / sqrt(d) = sum_i <q_i, dQ_i / c> / sqrt(d)
// (the last form needs no division by tau, so it holds at tau = 0 too).
// Tempered attention is the same with a = p: dS_ij = p_ij (dA_ij - delta_i).
// With per-head multipliers (a learned temperature) c and tau are head bh's.
//
// Head dimension D = 64 or 128 (a template parameter of every kernel); at
// D = 128 the dQ and dK/dV kernels run one workgroup per CU, which doubles
// the registers per lane for the doubled operands and accumulators.  With
// one wave per SIMD only a wave's own instruction order can overlap its
// matrix-core and vector work, so at D = 128 the operands of the closing
// products are read into registers ahead of them, and the dilution dK/dV
// pass issues each block's closing products during the next block.
//
// Passes (dilution; tempered runs 1, 4, 4b and 3 only, dK/dV top-down):
//   1 bwd_prep_kernel   per row: log2-domain lse, 1/r, delta/r
//   2 colsum_bf16_kernel (the forward's) committed demand per 32-row block
//   3 bwd_dkdv_kernel   per 32 keys, walking 32-row blocks from the last one
//                       up: the sum of g over every later block (G's block
//                       part, carried in a register and stored for pass 4),
//                       dV, dK' = sum_i p_ij dp_ij q_i (fp32 workspace), and
//                       per row its 128 keys' part of rho_i = sum_j p_ij dp_ij
//   4 bwd_dq_kernel     per 32 query rows: rho_i from those parts, then
//                       dQ_i = c sum_j p_ij (dp_ij - rho_i) k_j and <q_i, dQ_i / c>
//   4b bwd_dtau_kernel  (when dL/dtau is asked for) per head: the rows' sum
//   5 bwd_dkrho_kernel  per 32 keys: dK_j = c (dK'_j - sum_i p_ij rho_i q_i)
// Splitting dK_j = c sum_i p_ij (dp_ij - rho_i) q_i at rho lets the dK/dV
// pass run before rho is known (rho needs every key of a row, and dp needs
// G, the column sums that pass carries), so one column pass over all pairs
// does G, dK/dV and the parts of rho.
// Both in-block scans (the column prefix inside D and the column suffix
// inside G) are matrix-core products against constant triangular operands,
// as in the forward shares pass.
// The closing products (dK^T += Q^T dS, dV^T += dO^T a, dQ^T += K^T dS^T and
// the rho pass's Q^T (p rho)) need Q, dO and K dim-major.  They read them
// straight from the row-major LDS blocks with the transposing LDS load
// (ds_read_b64_tr_b16), so each block is read from memory once, with
// coalesced 16-byte loads, and stored to LDS once.
#include "attn_common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

#include <float.h>

namespace attn {

constexpr int kColKeys = 128;   // keys per workgroup in the column kernels (4 waves x 32)
constexpr float kInvDMax = 18446744073709551616.0f;   // 2^64: clamp on 1/D (eps = 0 only)
constexpr float kNoClampEps = 1.0842021724855044e-19f;   // 2^-63

// 1/D.  D >= eps (the committed demand and the bids are non-negative, and
// committed + eps is stored to 2^-17 relative), so for eps >= 2^-63 the
// reciprocal stays below 2^64: the clamp that keeps eps = 0 finite is then
// left out (CLAMP = false), with the same bits.
template <bool CLAMP>
__device__ __forceinline__ float inv_denominator(float d) {
  const float r = fast_rcp(d);
  return CLAMP ? fminf(r, kInvDMax) : r;
}

// The multiplier of head bh (1 when the scales carry a scalar tau).
__device__ __forceinline__ float head_tau(const BwdArgs &a, int bh) {
  return a.tau_bh ? a.tau_bh[bh] : 1.0f;
}

__device__ __forceinline__ bf16x8 word_operand(uint32_t w) {
  const u32x4 u = {w, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, u);
}

// ------------------------------------------------------------------ prep

// Eight lanes per row: delta = <dO_i, o_i> from 16-byte loads (D/64 per
// lane), then the per-row scalars the other passes read.
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdArgs a, int dilution) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid >> 3;
  const int dc = (int)(gid & 7);
  const bool live = row < (size_t)a.BH * a.T;
  float acc = 0.0f;
  if (live) {
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
      const size_t off = row * D + 64 * j + 8 * dc;
      const u32x4 ov = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const __bf16 *>(a.o) + off);
      const u32x4 gv =
          *reinterpret_cast<const u32x4 *>(reinterpret_cast<const __bf16 *>(a.dout) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = ov[i], y = gv[i];
        acc = __builtin_fmaf(bf16_lo(x), bf16_lo(y), acc);
        acc = __builtin_fmaf(bf16_hi(x), bf16_hi(y), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 8);
  acc += __shfl_xor(acc, 2, 8);
  acc += __shfl_xor(acc, 4, 8);
  if (live && dc == 0) {
    a.lse2[row] = a.lse[row] * kLog2e;
    if (dilution) {
      const float ir = 1.0f / a.rowsum[row];
      a.invr[row] = ir;
      a.dri[row] = acc * ir;
    } else {
      a.invr[row] = 1.0f;
      a.dri[row] = acc;
    }
  }
}

// ------------------------------------------------------- column kernels
//
// A workgroup owns 128 keys (wave w the 32 keys [kw0, kw0 + 32), K and V rows
// held in registers as B operands) and walks the 32-row query blocks that
// see them.  Scores of a block are in the S layout (lane = key, element r =
// query acc_row(r, h)).  The column scans take the packed bids / gradient
// terms as the B operand against constant A operands (lane = output row m):

struct ScanConsts {
  bf16x8 le[2];    // inclusive prefix: 1 where the slot's query <= m
  bf16x8 ge[2];    // inclusive suffix: 1 where the slot's query >= m
  bf16x8 ones;     // slots (0, 0) and (0, 1): adds a per-key bf16 (hi, lo) pair
  bf16x8 ident[2]; // B operand: 1 where the slot's query == n; with packed
                   // S-layout values as the A operand (m = key, slots = queries)
                   // it moves them to lane = query
};

__device__ __forceinline__ ScanConsts scan_consts(int l32, int h) {
  ScanConsts c;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float le[8], ge[8], id[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qs = acc_row(8 * j + e, h);
      le[e] = qs <= l32 ? 1.0f : 0.0f;
      ge[e] = qs >= l32 ? 1.0f : 0.0f;
      id[e] = qs == l32 ? 1.0f : 0.0f;
    }
    c.le[j] = pack8(le);
    c.ge[j] = pack8(ge);
    c.ident[j] = pack8(id);
  }
  const float one = h == 0 ? 1.0f : 0.0f;
  c.ones = to_bf16x8(one, one, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f);
  return c;
}

// Per-block LDS staging of the dK/dV kernel: Q and dO rows of one 32-row
// block (DualRows layout: the A operands of S = Q K^T and dA = dO V^T, read
// transposed for the closing products), and the per-row scalars.
template <int D>
struct ColBlock {
  __bf16 q[32 * DualRows<D>::kRow];
  __bf16 g[32 * DualRows<D>::kRow];
  float lse2[32], invr[32], dri[32];
};

// Bids of a block in the S layout; on the diagonal block rows before the key
// see nothing of it.
template <bool DIAG>
__device__ __forceinline__ void col_bids(const f32x16 &s, const float *lq, float c2, int l32,
                                         int h, float *p) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float e = fast_exp2(__builtin_fmaf(s[r], c2, -lq[r]));
    if (DIAG && acc_row(r, h) < l32) e = 0.0f;
    p[r] = e;
  }
}

// Per-row scalars of the block in the S-layout register order.
__device__ __forceinline__ void col_rowvals(const float *src, int h, float *dst) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(src + 8 * g + 4 * h);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[4 * g + i] = v[i];
  }
}

// The block's S = Q K^T and dA = dO V^T for this wave's keys.
template <int D>
__device__ __forceinline__ void col_scores(const ColBlock<D> &b, const bf16x8 *kf,
                                           const bf16x8 *vf, int l32, int h, f32x16 &s,
                                           f32x16 &da) {
  s = zero16();
  da = zero16();
#pragma unroll
  for (int c = 0; c < Geom<D>::kChunks; ++c) {
    s = mfma32(lds_frag_swz<D>(b.q, l32, c, h), kf[c], s);
    da = mfma32(lds_frag_swz<D>(b.g, l32, c, h), vf[c], da);
  }
}

// Pass 3: dK and dV for this wave's keys.  The transposed Q and dO blocks
// (dim-major) are the A operands of dK^T += Q^T dS and dV^T += dO^T a; the
// packed dS and a (S layout) are their B operands.  Dilution takes p dp in
// place of dS (rho enters in pass 5) and, walking bottom-up, carries in
// `running` each half-lane's sum of g over the blocks below; `gin_word`
// returns that sum over both halves (bf16 pair) for the dQ pass, and
// `rho_part` the block's rows' sums of the packed p dp over this wave's 32
// keys (lane l32: row l32 of the block).

template <bool DIL, bool DIAG, bool CLAMP, int D>
__device__ __forceinline__ void dkdv_block(const ColBlock<D> &b,
                                           const bf16x8 *kf, const bf16x8 *vf,
                                           const ScanConsts &sc, uint32_t cin_word,
                                           float &running, uint32_t &gin_word, float &rho_part,
                                           float c2, int l32, int h, f32x16 *dkt, f32x16 *dvt) {
  f32x16 s, da;
  col_scores(b, kf, vf, l32, h, s, da);
  // The tempered form reads the transposed Q and dO fragments of the closing
  // dK/dV products into registers right after the score products, so that
  // their LDS latency passes behind the vector work instead of before each
  // product; the dilution form at d = 64 has no registers to spare for them.
  constexpr bool kAhead = !DIL;
  bf16x8 qtf[Geom<D>::kOBlocks][2], gtf[Geom<D>::kOBlocks][2];
  auto read_ahead = [&]() {
#pragma unroll
    for (int u = 0; u < Geom<D>::kOBlocks; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        qtf[u][j] = lds_tr_frag_swz<D>(b.q, 16 * j, 32 * u);
        gtf[u][j] = lds_tr_frag_swz<D>(b.g, 16 * j, 32 * u);
      }
    __builtin_amdgcn_sched_barrier(0);   // keep the reads where they are issued
  };
  if constexpr (kAhead) read_ahead();
  float ds[16], aw[16];
  if constexpr (DIL) {
    // written out stage by stage so each per-row array and temporary dies
    // as soon as it is used
    float lq[16];
    col_rowvals(b.lse2, h, lq);
    float p[16];
    col_bids<DIAG>(s, lq, c2, l32, h, p);
    f32x16 d = mfma32(sc.le[0], pack8(p), zero16());
    d = mfma32(sc.le[1], pack8(p + 8), d);
    d = mfma32(sc.ones, word_operand(cin_word), d);
    float invd[16], sg[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      invd[r] = inv_denominator<CLAMP>(d[r]);
      sg[r] = p[r] * invd[r];
    }
    float iq[16];
    col_rowvals(b.invr, h, iq);
#pragma unroll
    for (int r = 0; r < 16; ++r) aw[r] = sg[r] * iq[r];
    float rq[16];
    col_rowvals(b.dri, h, rq);
    float dsg[16], g[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dsg[r] = __builtin_fmaf(da[r], iq[r], -rq[r]);
      g[r] = dsg[r] * sg[r] * invd[r];
    }
    // G = gradient terms of the later blocks + inclusive suffix in this one
    gin_word = split2_bf16(both_halves_sum(running));
    f32x16 G = mfma32(sc.ge[0], pack8(g), zero16());
    G = mfma32(sc.ge[1], pack8(g + 8), G);
    G = mfma32(sc.ones, word_operand(gin_word), G);
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) part += g[r];
    running += part;
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = p[r] * __builtin_fmaf(dsg[r], invd[r], -G[r]);
  } else {
    float lq[16], rq[16];
    col_rowvals(b.lse2, h, lq);
    col_rowvals(b.dri, h, rq);
    col_bids<DIAG>(s, lq, c2, l32, h, aw);
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = aw[r] * (da[r] - rq[r]);
  }
  const bf16x8 sf[2] = {pack8(ds), pack8(ds + 8)};
  const bf16x8 af[2] = {pack8(aw), pack8(aw + 8)};
  if constexpr (DIL) {
    // the packed p dp moved to lane = row (keys in the elements), summed
    f32x16 rt = mfma32(sf[0], sc.ident[0], zero16());
    rt = mfma32(sf[1], sc.ident[1], rt);
    float part = rt[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) part += rt[r];
    rho_part = both_halves_sum(part);
  }
#pragma unroll
  for (int u = 0; u < Geom<D>::kOBlocks; ++u) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (kAhead) {
        dkt[u] = mfma32(qtf[u][j], sf[j], dkt[u]);
        dvt[u] = mfma32(gtf[u][j], af[j], dvt[u]);
      } else {
        dkt[u] = mfma32(lds_tr_frag_swz<D>(b.q, 16 * j, 32 * u), sf[j], dkt[u]);
        dvt[u] = mfma32(lds_tr_frag_swz<D>(b.g, 16 * j, 32 * u), af[j], dvt[u]);
      }
    }
  }
}

// The dilution form of pass 3 at d = 128, software-pipelined across blocks.
// At one wave per SIMD a wave's matrix-core and vector work overlap only
// where its own instruction stream interleaves them, and a block's closing
// dK/dV products depend on the whole vector chain before them.  So block n's
// closing products (operands qtf / gtf and the packed sf / af, carried in
// registers) are issued during block n + 1, one beside each element step of
// that block's vector chain, and block n + 1's fragments are read after them.
// Each accumulator still receives its products block by block in the same
// order, so the sums are the same bits.  The caller issues the last block's
// products after the loop (dkdv_tail); before the first block the carried
// operands are zero, and the products add +0.
template <int D>
struct DkdvCarry {
  bf16x8 qtf[Geom<D>::kOBlocks][2], gtf[Geom<D>::kOBlocks][2];   // transposed Q / dO fragments
  bf16x8 sf[2], af[2];   // packed dS (dilution: p dp) and a of the block
};

// Product i (0 .. 4 kOBlocks - 1) of the carried block's closing products.
template <int D>
__device__ __forceinline__ void dkdv_tail_step(const DkdvCarry<D> &cr, int i, f32x16 *dkt,
                                               f32x16 *dvt) {
  const int u = i >> 2, j = (i >> 1) & 1;
  if (i & 1) dvt[u] = mfma32(cr.gtf[u][j], cr.af[j], dvt[u]);
  else dkt[u] = mfma32(cr.qtf[u][j], cr.sf[j], dkt[u]);
}

template <int D>
__device__ __forceinline__ void dkdv_tail(const DkdvCarry<D> &cr, f32x16 *dkt, f32x16 *dvt) {
#pragma unroll
  for (int i = 0; i < 4 * Geom<D>::kOBlocks; ++i) dkdv_tail_step<D>(cr, i, dkt, dvt);
}

template <bool DIAG, bool CLAMP, int D>
__device__ __forceinline__ void dkdv_block_pipelined(const ColBlock<D> &b,
                                                     const bf16x8 *kf, const bf16x8 *vf,
                                                     const ScanConsts &sc, uint32_t cin_word,
                                                     float &running, uint32_t &gin_word,
                                                     float &rho_part, float c2, int l32, int h,
                                                     DkdvCarry<D> &cr, f32x16 *dkt, f32x16 *dvt) {
  static_assert(4 * Geom<D>::kOBlocks == 16, "one carried product per element step");
  f32x16 s, da;
  col_scores(b, kf, vf, l32, h, s, da);
  float lq[16];
  col_rowvals(b.lse2, h, lq);
  float p[16];
  col_bids<DIAG>(s, lq, c2, l32, h, p);
  float iq[16], rq[16];
  col_rowvals(b.invr, h, iq);
  col_rowvals(b.dri, h, rq);
  f32x16 d = mfma32(sc.le[0], pack8(p), zero16());
  d = mfma32(sc.le[1], pack8(p + 8), d);
  d = mfma32(sc.ones, word_operand(cin_word), d);
  // the carried block's closing products, one beside each element step
  float invd[16], dsg[16], g[16], aw[16];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    dkdv_tail_step<D>(cr, r, dkt, dvt);
    invd[r] = inv_denominator<CLAMP>(d[r]);
    const float sg = p[r] * invd[r];
    aw[r] = sg * iq[r];
    dsg[r] = __builtin_fmaf(da[r], iq[r], -rq[r]);
    g[r] = dsg[r] * sg * invd[r];
    __builtin_amdgcn_sched_barrier(0);
  }
  // this block's fragments, into the registers the carried products have read
#pragma unroll
  for (int u = 0; u < Geom<D>::kOBlocks; ++u)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      cr.qtf[u][j] = lds_tr_frag_swz<D>(b.q, 16 * j, 32 * u);
      cr.gtf[u][j] = lds_tr_frag_swz<D>(b.g, 16 * j, 32 * u);
    }
  // G = gradient terms of the later blocks + inclusive suffix in this one
  gin_word = split2_bf16(both_halves_sum(running));
  f32x16 G = mfma32(sc.ge[0], pack8(g), zero16());
  G = mfma32(sc.ge[1], pack8(g + 8), G);
  G = mfma32(sc.ones, word_operand(gin_word), G);
  float part = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) part += g[r];
  running += part;
  float ds[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) ds[r] = p[r] * __builtin_fmaf(dsg[r], invd[r], -G[r]);
  cr.sf[0] = pack8(ds);
  cr.sf[1] = pack8(ds + 8);
  cr.af[0] = pack8(aw);
  cr.af[1] = pack8(aw + 8);
  // the packed p dp moved to lane = row (keys in the elements), summed
  f32x16 rt = mfma32(cr.sf[0], sc.ident[0], zero16());
  rt = mfma32(cr.sf[1], sc.ident[1], rt);
  float rsum = rt[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) rsum += rt[r];
  rho_part = both_halves_sum(rsum);
}

// Waves per SIMD the dQ and dK/dV kernels are built for: two at d = 64; one
// at d = 128, whose operand fragments and accumulators need twice the registers.
template <int D>
struct BwdOccupancy {
  static constexpr int value = D > 64 ? 1 : 2;
};

template <bool DIL, int D, bool CLAMP>
__global__ void __launch_bounds__(256, (BwdOccupancy<D>::value)) bwd_dkdv_kernel(BwdArgs a,
                                                                                 int nqs) {
  constexpr int kKR = Geom<D>::kKRow, kCh = Geom<D>::kChunks, kOB = Geom<D>::kOBlocks;
  constexpr int kRowChunks = D / 8;   // 16-byte chunks per row
  constexpr int kBlkLoads = 32 * kRowChunks / 256;   // per thread, per tensor
  __shared__ __attribute__((aligned(16))) ColBlock<D> sb[2];
  // dilution: this workgroup's K and V rows (the B operands of S and dA) sit
  // in LDS and are read per block, which keeps the kernel within two waves'
  // registers per SIMD without spills; the tempered form keeps them in registers
  __shared__ __attribute__((aligned(16))) __bf16 sKV[DIL ? 2 : 1][DIL ? kColKeys * kKR : 8];
  // dilution: per block, each wave's sums of p dp over its keys (row l32),
  // added over the four waves one iteration later (double buffered)
  __shared__ float sRho[DIL ? 2 : 1][4][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;
  const float tb = head_tau(a, bh), c2 = a.c2 * tb, cs = a.c * tb;
  const int T = a.T;
  const int kw0 = kb * kColKeys + 32 * w;
  const bool wave_live = kw0 < T;
  const int key = kw0 + l32;
  const size_t head = (size_t)bh * T * D;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;
  const __bf16 *G = reinterpret_cast<const __bf16 *>(a.dout) + head;
  const float *L2 = a.lse2 + (size_t)bh * T;
  const float *IR = a.invr + (size_t)bh * T;
  const float *DR = a.dri + (size_t)bh * T;
  const uint32_t *cin = nullptr;
  uint32_t *gin = nullptr;
  if constexpr (DIL) {
    cin = reinterpret_cast<const uint32_t *>(a.cin) + (size_t)bh * cin_floats_per_head(T, 0);
    gin = reinterpret_cast<uint32_t *>(a.gin) + (size_t)bh * gin_floats_per_head(T);
  }
  const uint32_t eps_word = split2_bf16(fmaxf(a.eps, FLT_MIN));

  bf16x8 kf[kCh], vf[kCh];
  const __bf16 *krow = nullptr, *vrow = nullptr;
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const u32x4 kc = load_row_chunk<D>(K, key, T, 2 * c + h);
    const u32x4 vc = load_row_chunk<D>(V, key, T, 2 * c + h);
    if constexpr (DIL) {
      *reinterpret_cast<u32x4 *>(&sKV[0][(32 * w + l32) * kKR + 16 * c + 8 * h]) = kc;
      *reinterpret_cast<u32x4 *>(&sKV[1][(32 * w + l32) * kKR + 16 * c + 8 * h]) = vc;
    } else {
      kf[c] = __builtin_bit_cast(bf16x8, kc);
      vf[c] = __builtin_bit_cast(bf16x8, vc);
    }
  }
  if constexpr (DIL) {
    krow = &sKV[0][(32 * w + l32) * kKR];
    vrow = &sKV[1][(32 * w + l32) * kKR];
  }
  const ScanConsts sc = scan_consts(l32, h);
  f32x16 dkt[kOB], dvt[kOB];
#pragma unroll
  for (int u = 0; u < kOB; ++u) dkt[u] = dvt[u] = zero16();
  // dilution at d = 128: each block's closing products are issued during the next one
  constexpr bool kPipe = DIL && D > 64;
  DkdvCarry<D> carry;
  if constexpr (kPipe) {
    const bf16x8 z = to_bf16x8(0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int u = 0; u < kOB; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) carry.qtf[u][j] = carry.gtf[u][j] = z;
    carry.sf[0] = carry.sf[1] = carry.af[0] = carry.af[1] = z;
  }
  __builtin_amdgcn_s_waitcnt(0);

  const int qs_lo = (kb * kColKeys) / 32;
  // loaders: chunk u = tid + 256 i of the Q and dO blocks is row
  // u / kRowChunks, chunk u % kRowChunks.  The closing products read the
  // blocks transposed straight from these row-major copies.
  u32x4 qreg[kBlkLoads], greg[kBlkLoads];
  float lreg = 0.0f, ireg = 0.0f, rreg = 0.0f;
  auto load_block = [&](int qs) {
    const int row0 = 32 * qs;
    const int bytes = (T - row0) * (D * 2);
    const auto rq = make_rsrc(Q + (size_t)row0 * D, bytes);
    const auto rg = make_rsrc(G + (size_t)row0 * D, bytes);
#pragma unroll
    for (int i = 0; i < kBlkLoads; ++i) {
      const int u = tid + 256 * i;
      qreg[i] = buf_load16(rq, 16u * u);
      greg[i] = buf_load16(rg, 16u * u);
    }
    if (tid < 32) {
      const int row = row0 + tid;
      const bool ok = row < T;
      const int rr = ok ? row : T - 1;
      lreg = ok ? L2[rr] : kNoRow;
      ireg = ok ? IR[rr] : 0.0f;
      rreg = ok ? DR[rr] : 0.0f;
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kBlkLoads; ++i) {
      const int u = tid + 256 * i;
      const int off = swz_off<D>(u / kRowChunks, (u % kRowChunks) * 8);
      *reinterpret_cast<u32x4 *>(&sb[buf].q[off]) = qreg[i];
      *reinterpret_cast<u32x4 *>(&sb[buf].g[off]) = greg[i];
    }
    if (tid < 32) {
      sb[buf].lse2[tid] = lreg;
      sb[buf].invr[tid] = ireg;
      sb[buf].dri[tid] = rreg;
    }
  };

  // blocks qs_lo .. nqs - 1, dilution from the last one up (G's carried
  // part is a sum over the rows below), tempered from the first one down
  const int nblk = nqs - qs_lo;
  auto block_at = [&](int n) { return DIL ? nqs - 1 - n : qs_lo + n; };
  float running = 0.0f;   // dilution: sum of g over this half-lane's rows below
  // dilution: this workgroup's part of rho for the rows of block qs, written
  // as [bh][kb][row]
  float *rhop = DIL ? a.rhop + ((size_t)bh * ((T + kColKeys - 1) / kColKeys) + kb) * T : nullptr;
  auto flush_rho = [&](int qs, int buf) {
    if (DIL && w == 0 && h == 0) {
      const int row = 32 * qs + l32;
      if (row < T) rhop[row] = ((sRho[buf][0][l32] + sRho[buf][1][l32]) + sRho[buf][2][l32]) +
                               sRho[buf][3][l32];
    }
  };
  // dilution: the committed demand (+ eps) of block qs on this lane's key,
  // loaded with the block's rows one iteration ahead: a load issued inside
  // the iteration would make its wait drain the next block's loads as well
  uint32_t cw_next = 0u;
  auto load_cin = [&](int qs) {
    if constexpr (DIL)
      cw_next = (wave_live && key < 32 * qs) ? cin[cin_block_offset(qs, 0) + key] : eps_word;
  };
  load_block(block_at(0));
  load_cin(block_at(0));
  store_block(0);
  __syncthreads();
  for (int n = 0; n < nblk; ++n) {
    const int qs = block_at(n);
    const int buf = n & 1;
    const uint32_t cw_cur = cw_next;
    if (n + 1 < nblk) {
      load_block(block_at(n + 1));
      load_cin(block_at(n + 1));
    }
    if (n > 0) flush_rho(block_at(n - 1), buf ^ 1);
    float rho_part = 0.0f;   // waves whose keys block qs does not see add 0
    if (wave_live && 32 * qs + 31 >= kw0) {
      uint32_t cw = cw_cur, gw = 0u;
      if constexpr (DIL) {
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
          kf[c] = lds_frag(krow, c, h);
          vf[c] = lds_frag(vrow, c, h);
        }
      }
      if constexpr (kPipe) {
        if (32 * qs == kw0)
          dkdv_block_pipelined<true, CLAMP>(sb[buf], kf, vf, sc, cw, running, gw,
                                            rho_part, c2, l32, h, carry, dkt, dvt);
        else
          dkdv_block_pipelined<false, CLAMP>(sb[buf], kf, vf, sc, cw, running, gw,
                                             rho_part, c2, l32, h, carry, dkt, dvt);
      } else {
        if (32 * qs == kw0)
          dkdv_block<DIL, true, CLAMP>(sb[buf], kf, vf, sc, cw, running, gw, rho_part, c2,
                                       l32, h, dkt, dvt);
        else
          dkdv_block<DIL, false, CLAMP>(sb[buf], kf, vf, sc, cw, running, gw, rho_part,
                                        c2, l32, h, dkt, dvt);
      }
      // the wave's keys are all below 32 (qs + 1): block qs keeps an entry for each
      if (DIL && h == 0 && key < T) gin[(size_t)16 * qs * (qs + 1) + key] = gw;
    }
    if (DIL && h == 0) sRho[buf][w][l32] = rho_part;
    if (n + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }
  if (nblk > 0) flush_rho(block_at(nblk - 1), (nblk - 1) & 1);
  if constexpr (kPipe) dkdv_tail<D>(carry, dkt, dvt);   // the last block's closing products
  if (!wave_live || key >= T) return;
  // lane: key; element (u, r): dim 32u + acc_row(r, h)
  __bf16 *dK = reinterpret_cast<__bf16 *>(a.dk) + head + (size_t)key * D;
  __bf16 *dV = reinterpret_cast<__bf16 *>(a.dv) + head + (size_t)key * D;
  float *dKp = DIL ? a.dkp + head + (size_t)key * D : nullptr;
#pragma unroll
  for (int u = 0; u < kOB; ++u) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * u + 8 * g + 4 * h;
      u32x2 vv;
      vv[0] = pack_bf16x2(dvt[u][4 * g], dvt[u][4 * g + 1]);
      vv[1] = pack_bf16x2(dvt[u][4 * g + 2], dvt[u][4 * g + 3]);
      *reinterpret_cast<u32x2 *>(dV + d0) = vv;
      if constexpr (DIL) {
        const f32x4 kp = {dkt[u][4 * g], dkt[u][4 * g + 1], dkt[u][4 * g + 2], dkt[u][4 * g + 3]};
        *reinterpret_cast<f32x4 *>(dKp + d0) = kp;
      } else {
        u32x2 kk;
        kk[0] = pack_bf16x2(dkt[u][4 * g] * cs, dkt[u][4 * g + 1] * cs);
        kk[1] = pack_bf16x2(dkt[u][4 * g + 2] * cs, dkt[u][4 * g + 3] * cs);
        *reinterpret_cast<u32x2 *>(dK + d0) = kk;
      }
    }
  }
}

// Pass 6 (dilution): dK_j = c (dK'_j - Y_j), Y_j = sum_i p_ij rho_i q_i, with
// dK' from pass 3 (fp32 workspace) and rho from pass 5.  A workgroup owns 128
// keys (wave w 32 of them, the key row in registers as the B operand of
// S = Q K^T) and walks the 32-row blocks that see them, two per barrier; per
// block the bids are recomputed (S layout), scaled by their rows' rho,
// packed and accumulated as Y^T += Q^T (p rho), with Q^T read transposed
// from the block's row-major Q rows.
template <int D>
struct RhoBlock {
  __bf16 q[32 * DualRows<D>::kRow];   // Q rows (A operand of S; read transposed for Y^T)
  float lse2[32], rho[32];
};

template <int D>
__global__ void __launch_bounds__(256, 2) bwd_dkrho_kernel(BwdArgs a, int nqs) {
  constexpr int kKR = Geom<D>::kKRow, kCh = Geom<D>::kChunks, kOB = Geom<D>::kOBlocks;
  constexpr int kRowChunks = D / 8;                  // 16-byte chunks per row
  constexpr int kRowLoads = 64 * kRowChunks / 256;   // row-major chunks per thread and stage
  __shared__ __attribute__((aligned(16))) RhoBlock<D> sb[2][2];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;
  const float tb = head_tau(a, bh), c2 = a.c2 * tb, cs = a.c * tb;
  const int T = a.T;
  const int kw0 = kb * kColKeys + 32 * w;
  const bool wave_live = kw0 < T;
  const int key = kw0 + l32;
  const size_t head = (size_t)bh * T * D;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const float *L2 = a.lse2 + (size_t)bh * T;
  const float *RH = a.rho + (size_t)bh * T;

  bf16x8 kf[kCh];
#pragma unroll
  for (int c = 0; c < kCh; ++c) kf[c] = __builtin_bit_cast(bf16x8, load_row_chunk<D>(K, key, T, 2 * c + h));
  f32x16 yt[kOB];
#pragma unroll
  for (int u = 0; u < kOB; ++u) yt[u] = zero16();
  __builtin_amdgcn_s_waitcnt(0);

  // a stage is the 64 rows of blocks (2P, 2P + 1).  Loaders: chunk
  // u = tid + 256 i is row u / kRowChunks, chunk u % kRowChunks
  u32x4 qreg[kRowLoads];
  float lreg = 0.0f, hreg = 0.0f;
  auto load_stage = [&](int P) {              // 64 P < T for every stage loaded
    const int row0 = 64 * P;
    const auto rq = make_rsrc(Q + (size_t)row0 * D, (T - row0) * (D * 2));
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i) qreg[i] = buf_load16(rq, 16u * (tid + 256 * i));
    if (tid < 64) {
      const int row = row0 + tid;
      const bool ok = row < T;
      const int rr = ok ? row : T - 1;
      lreg = ok ? L2[rr] : kNoRow;
      hreg = ok ? RH[rr] : 0.0f;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kRowLoads; ++i) {
      const int u = tid + 256 * i, row = u / kRowChunks;
      *reinterpret_cast<u32x4 *>(&sb[buf][row >> 5].q[swz_off<D>(row & 31, (u % kRowChunks) * 8)]) =
          qreg[i];
    }
    if (tid < 64) {
      sb[buf][tid >> 5].lse2[tid & 31] = lreg;
      sb[buf][tid >> 5].rho[tid & 31] = hreg;
    }
  };

  // qs_lo = 4 kb is even: stages p_lo .. p_hi cover blocks qs_lo .. nqs - 1
  const int p_lo = 2 * kb, p_hi = (nqs - 1) / 2;
  load_stage(p_lo);
  store_stage(0);
  __syncthreads();
  for (int P = p_lo; P <= p_hi; ++P) {
    const int buf = (P - p_lo) & 1;
    if (P < p_hi) load_stage(P + 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qs = 2 * P + i;
      if (qs < nqs && wave_live && 32 * qs + 31 >= kw0) {
        const RhoBlock<D> &b = sb[buf][i];
        f32x16 sc = zero16();
#pragma unroll
        for (int c = 0; c < kCh; ++c) sc = mfma32(lds_frag_swz<D>(b.q, l32, c, h), kf[c], sc);
        float lq[16], pq[16], wv[16];
        col_rowvals(b.lse2, h, lq);
        col_rowvals(b.rho, h, pq);
        if (32 * qs == kw0) col_bids<true>(sc, lq, c2, l32, h, wv);
        else col_bids<false>(sc, lq, c2, l32, h, wv);
#pragma unroll
        for (int r = 0; r < 16; ++r) wv[r] *= pq[r];
        const bf16x8 wf[2] = {pack8(wv), pack8(wv + 8)};
#pragma unroll
        for (int u = 0; u < kOB; ++u)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            yt[u] = mfma32(lds_tr_frag_swz<D>(b.q, 16 * j, 32 * u), wf[j], yt[u]);
      }
    }
    if (P < p_hi) store_stage(buf ^ 1);
    __syncthreads();
  }
  if (!wave_live || key >= T) return;
  // lane: key; element (u, r): dim 32u + acc_row(r, h)
  __bf16 *dK = reinterpret_cast<__bf16 *>(a.dk) + head + (size_t)key * D;
  const float *dKp = a.dkp + head + (size_t)key * D;
#pragma unroll
  for (int u = 0; u < kOB; ++u) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * u + 8 * g + 4 * h;
      const f32x4 kp4 = *reinterpret_cast<const f32x4 *>(dKp + d0);
      u32x2 kk;
      kk[0] = pack_bf16x2((kp4[0] - yt[u][4 * g]) * cs, (kp4[1] - yt[u][4 * g + 1]) * cs);
      kk[1] = pack_bf16x2((kp4[2] - yt[u][4 * g + 2]) * cs, (kp4[3] - yt[u][4 * g + 3]) * cs);
      *reinterpret_cast<u32x2 *>(dK + d0) = kk;
    }
  }
}

// --------------------------------------------------------------- dQ rows
//
// A workgroup owns 128 query rows (wave w the 32 rows [qw0, qw0 + 32)) and
// streams 64-key tiles of K and V (row-major) through LDS; K also serves,
// read transposed, as the A operand of dQ^T += K^T dS^T.  Scores are taken as S^T
// (lane = query, element r = key acc_row(r, h)), so the per-row scalars are
// per lane; the column scans need the bids and g with queries in the
// operand slots, so those are moved to the S layout by identity products.

struct DqConsts {
  bf16x8 upre[2];   // B operands, slot (h, e) of operand j = query acc_row(8j+e, h):
  bf16x8 usuf[2];   //   inclusive prefix (<= n), inclusive suffix (>= n)
  bf16x8 ident[2];  //   and identity (== n); keys in place of queries for the
  bf16x8 bone;      //   S^T -> S transpose.  bone: slots (0, 0..1) on h = 0.
};

__device__ __forceinline__ DqConsts dq_consts(int l32, int h) {
  DqConsts c;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float u[8], v[8], id[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int qs = acc_row(8 * j + e, h);
      u[e] = qs <= l32 ? 1.0f : 0.0f;
      v[e] = qs >= l32 ? 1.0f : 0.0f;
      id[e] = qs == l32 ? 1.0f : 0.0f;
    }
    c.upre[j] = pack8(u);
    c.usuf[j] = pack8(v);
    c.ident[j] = pack8(id);
  }
  const float one = h == 0 ? 1.0f : 0.0f;
  c.bone = to_bf16x8(one, one, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f);
  return c;
}

template <int D>
struct DqState {
  f32x16 x[Geom<D>::kOBlocks];   // X^T[d][query] = sum_j dS_ij k_j; x[u] holds d in
                                 // [32u, 32u + 32)
};

template <bool DIL, bool DIAG, bool CLAMP, int D>
__device__ __forceinline__ void dq_subtile(DqState<D> &st, const bf16x8 *qf, const bf16x8 *gf,
                                           const DqConsts &dc,
                                           const __bf16 *kt_lds, const __bf16 *vt_lds,
                                           int t, uint32_t cin_word,
                                           uint32_t gin_word, float lse2, float invr, float dri,
                                           float rho, int qrel, int l32, int h, float c2) {
  // S^T and dA^T for keys 32t.. of the tile (lane = query)
  const __bf16 *vrow = vt_lds + (32 * t + l32) * Geom<D>::kKRow;
  f32x16 s = zero16(), da = zero16();
#pragma unroll
  for (int c = 0; c < Geom<D>::kChunks; ++c) {
    s = mfma32(lds_frag_swz<D>(kt_lds, 32 * t + l32, c, h), qf[c], s);
    da = mfma32(lds_frag(vrow, c, h), gf[c], da);
  }
  // The K^T fragments of the closing dQ products, read transposed from the
  // row-major K tile and ahead of the products as in the dK/dV pass
  // (dilution: once the in-block prefix is formed; tempered: right away).
  constexpr bool kAhead = D > 64 || !DIL;
  bf16x8 kta[Geom<D>::kOBlocks][2];
  auto kt_frag = [&](int i, int c) {
    return lds_tr_frag_swz<D>(kt_lds, 32 * t + 16 * c, 32 * i);
  };
  auto read_ahead = [&]() {
#pragma unroll
    for (int i = 0; i < Geom<D>::kOBlocks; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) kta[i][c] = kt_frag(i, c);
    __builtin_amdgcn_sched_barrier(0);   // keep the reads where they are issued
  };
  // dQ^T += K^T dS^T for the sub-tile's keys (e0, e1: the packed dS^T)
  auto update = [&](const bf16x8 &e0, const bf16x8 &e1) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < Geom<D>::kOBlocks; ++i) {
        if constexpr (kAhead) st.x[i] = mfma32(kta[i][c], c == 0 ? e0 : e1, st.x[i]);
        else st.x[i] = mfma32(kt_frag(i, c), c == 0 ? e0 : e1, st.x[i]);
      }
  };
  if constexpr (kAhead && !DIL) read_ahead();
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float e = fast_exp2(__builtin_fmaf(s[r], c2, -lse2));
    if (DIAG && 32 * t + acc_row(r, h) > qrel) e = 0.0f;
    p[r] = e;
  }
  const bf16x8 pt0 = pack8(p), pt1 = pack8(p + 8);
  if constexpr (DIL) {
    // the bids with queries in the slots (S layout), then D^T
    f32x16 ps = mfma32(pt0, dc.ident[0], zero16());
    ps = mfma32(pt1, dc.ident[1], ps);
    float pv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pv[r] = ps[r];
    const bf16x8 pa0 = pack8(pv), pa1 = pack8(pv + 8);
    f32x16 d = mfma32(pa0, dc.upre[0], zero16());
    d = mfma32(pa1, dc.upre[1], d);
    d = mfma32(word_operand(cin_word), dc.bone, d);
    if constexpr (kAhead) read_ahead();
    float invd[16], dsg[16], g[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      invd[r] = inv_denominator<CLAMP>(d[r]);
      const float sg = p[r] * invd[r];
      dsg[r] = __builtin_fmaf(da[r], invr, -dri);
      g[r] = dsg[r] * sg * invd[r];
    }
    // G^T: g to the S layout, then the inclusive suffix plus later blocks
    f32x16 gs = mfma32(pack8(g), dc.ident[0], zero16());
    gs = mfma32(pack8(g + 8), dc.ident[1], gs);
    float gv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) gv[r] = gs[r];
    f32x16 G = mfma32(pack8(gv), dc.usuf[0], zero16());
    G = mfma32(pack8(gv + 8), dc.usuf[1], G);
    G = mfma32(word_operand(gin_word), dc.bone, G);
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = p[r] * (__builtin_fmaf(dsg[r], invd[r], -G[r]) - rho);
    update(pack8(e), pack8(e + 8));
  } else {
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = p[r] * (da[r] - dri);
    update(pack8(ds), pack8(ds + 8));
  }
}

template <bool DIL, int D, bool CLAMP>
__global__ void __launch_bounds__(256, (BwdOccupancy<D>::value)) bwd_dq_kernel(BwdArgs a,
                                                                               int nqb) {
  constexpr int kKR = Geom<D>::kKRow, kKT = Geom<D>::kKTile;
  constexpr int kCh = Geom<D>::kChunks, kOB = Geom<D>::kOBlocks;
  constexpr int kRowChunks = D / 8;                     // 16-byte chunks per row
  constexpr int kTileLoads = kBN * kRowChunks / 256;    // per thread, per tensor
  constexpr int kKTs = kBN * DualRows<D>::kRow;   // the K tile, read both ways
  __shared__ __attribute__((aligned(16))) __bf16 sK[2 * kKTs];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2 * kKT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int bh = blockIdx.x % a.BH;
  const int qb = nqb - 1 - blockIdx.x / a.BH;   // heaviest query blocks first
  const float tb = head_tau(a, bh), c2 = a.c2 * tb, cs = a.c * tb;
  const int T = a.T;
  const int q0 = qb * 128;
  const int qw0 = q0 + 32 * w;
  const bool wave_live = qw0 < T;
  const int kd = qw0 / kBN;
  const size_t head = (size_t)bh * T * D;
  const __bf16 *Q = reinterpret_cast<const __bf16 *>(a.q) + head;
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.k) + head;
  const __bf16 *V = reinterpret_cast<const __bf16 *>(a.v) + head;
  const __bf16 *G = reinterpret_cast<const __bf16 *>(a.dout) + head;
  const int kend = min(q0 + 128, T);
  const int nkt = (kend + kBN - 1) / kBN;
  const int row = qw0 + l32;
  const bool row_ok = row < T;

  bf16x8 qf[kCh], gf[kCh];
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    qf[c] = __builtin_bit_cast(bf16x8, load_row_chunk<D>(Q, row, T, 2 * c + h));
    gf[c] = __builtin_bit_cast(bf16x8, load_row_chunk<D>(G, row, T, 2 * c + h));
  }
  const size_t ridx = (size_t)bh * T + (row_ok ? row : T - 1);
  const float lse2 = row_ok ? a.lse2[ridx] : kNoRow;
  const float invr = row_ok ? a.invr[ridx] : 0.0f;
  const float dri = row_ok ? a.dri[ridx] : 0.0f;
  const DqConsts dc = dq_consts(l32, h);
  const uint32_t eps_word = split2_bf16(fmaxf(a.eps, FLT_MIN));
  const uint32_t *cin_blk = nullptr, *gin_blk = nullptr;
  const int qsb = qw0 >> 5;   // this wave's 32-row block
  if constexpr (DIL) {
    cin_blk = reinterpret_cast<const uint32_t *>(a.cin) + (size_t)bh * cin_floats_per_head(T, 0) +
              cin_block_offset(qsb, 0);
    gin_blk = reinterpret_cast<const uint32_t *>(a.gin) + (size_t)bh * gin_floats_per_head(T) +
              (size_t)16 * qsb * (qsb + 1);
  }

  // loaders: chunk u = tid + 256 i of the K and V tiles is key u / kRowChunks,
  // chunk u % kRowChunks.  The closing products read K transposed straight
  // from its row-major tile.
  u32x4 kreg[kTileLoads], vreg[kTileLoads];
  auto load_tile = [&](int kt) {   // kt < nkt, so its first key is < T
    const int key0 = kt * kBN;
    const int bytes = (T - key0) * (D * 2);
    const auto rk = make_rsrc(K + (size_t)key0 * D, bytes);
    const auto rv = make_rsrc(V + (size_t)key0 * D, bytes);
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i) {
      kreg[i] = buf_load16(rk, 16u * (tid + 256 * i));
      vreg[i] = buf_load16(rv, 16u * (tid + 256 * i));
    }
  };
  auto store_tile = [&](int buf) {
    __bf16 *k = sK + buf * kKTs;
    __bf16 *v = sV + buf * kKT;
#pragma unroll
    for (int i = 0; i < kTileLoads; ++i) {
      const int u = tid + 256 * i;
      const int row = u / kRowChunks, e = (u % kRowChunks) * 8;
      *reinterpret_cast<u32x4 *>(k + swz_off<D>(row, e)) = kreg[i];
      *reinterpret_cast<u32x4 *>(v + row * kKR + e) = vreg[i];
    }
  };
  // committed demand (+eps) and later blocks' g sums of this wave's block on
  // keys kt*64 + 32t + l32
  uint32_t cw_next[2] = {0u, 0u}, gw_next[2] = {0u, 0u};
  auto load_words = [&](int kt) {
    if constexpr (DIL) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key = kt * kBN + 32 * t + l32;
        cw_next[t] = (wave_live && key < qw0) ? cin_blk[key] : eps_word;
        // keys past the end are masked, but their sums enter the scans: zero
        gw_next[t] = (wave_live && key < qw0 + 32 && key < T) ? gin_blk[key] : 0u;
      }
    }
  };

  DqState<D> st;
#pragma unroll
  for (int u = 0; u < kOB; ++u) st.x[u] = zero16();
  // dilution: rho_i = sum_j p_ij dp_ij from the dK/dV pass's parts (one per
  // 128-key workgroup up to the row's own, added in a fixed order: even parts
  // on the lower half-wave, odd ones on the upper), kept for the dK pass
  float rho = 0.0f;
  if constexpr (DIL) {
    if (row_ok) {
      const int nkb = (T + kColKeys - 1) / kColKeys;
      const float *rp = a.rhop + (size_t)bh * nkb * T + row;
      for (int kb = h; kb <= row / kColKeys; kb += 2) rho += rp[(size_t)kb * T];
    }
    rho = both_halves_sum(rho);
    if (row_ok && h == 0) a.rho[ridx] = rho;
  }
  __builtin_amdgcn_s_waitcnt(0);

  load_tile(0);
  store_tile(0);
  load_words(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    const uint32_t cw[2] = {cw_next[0], cw_next[1]}, gw[2] = {gw_next[0], gw_next[1]};
    if (kt + 1 < nkt) {
      load_tile(kt + 1);
      load_words(kt + 1);
    }
    if (wave_live && kt <= kd) {
      const __bf16 *kl = sK + buf * kKTs, *vl = sV + buf * kKT;
      const int qrel = qw0 + l32 - kt * kBN;
      // one sub-tile at a time: the per-sub-tile temporaries would not fit
      // twice beside the accumulators
#pragma unroll 1
      for (int t = 0; t < 2; ++t) {
        if (kt < kd)
          dq_subtile<DIL, false, CLAMP, D>(st, qf, gf, dc, kl, vl, t, cw[t], gw[t], lse2,
                                           invr, dri, rho, qrel, l32, h, c2);
        else
          dq_subtile<DIL, true, CLAMP, D>(st, qf, gf, dc, kl, vl, t, cw[t], gw[t], lse2,
                                          invr, dri, rho, qrel, l32, h, c2);
      }
    }
    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (!wave_live || !row_ok) return;
  __bf16 *dQ = reinterpret_cast<__bf16 *>(a.dq) + head + (size_t)row * D;
  // lane: query; element (block u, r): dim 32u + acc_row(r, h).  With u_i =
  // dQ_i / c, <q_i, u_i> = sum_j dS_ij <q_i, k_j>: this row's share of dL/dtau.
  const __bf16 *Qr = Q + (size_t)row * D;
  float tq = 0.0f;
#pragma unroll
  for (int u = 0; u < kOB; ++u) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * u + 8 * g + 4 * h;
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = st.x[u][4 * g + i];
      if (a.dtau) {
        const u32x2 qw = *reinterpret_cast<const u32x2 *>(Qr + d0);
        tq = __builtin_fmaf(bf16_lo(qw[0]), x[0], tq);
        tq = __builtin_fmaf(bf16_hi(qw[0]), x[1], tq);
        tq = __builtin_fmaf(bf16_lo(qw[1]), x[2], tq);
        tq = __builtin_fmaf(bf16_hi(qw[1]), x[3], tq);
      }
      u32x2 o2;
      o2[0] = pack_bf16x2(x[0] * cs, x[1] * cs);
      o2[1] = pack_bf16x2(x[2] * cs, x[3] * cs);
      *reinterpret_cast<u32x2 *>(dQ + d0) = o2;
    }
  }
  if (a.dtau) {
    tq = both_halves_sum(tq);
    if (h == 0) a.trow[ridx] = tq;
  }
}

// dL/dtau of each head: the rows' <q_i, u_i> (in tslices partial sums) summed
// in a fixed order (strided per thread, then a tree over the workgroup),
// times 1/sqrt(d).
__global__ void __launch_bounds__(256) bwd_dtau_kernel(BwdArgs a) {
  __shared__ float red[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  float acc = 0.0f;
  for (int sl = 0; sl < a.tslices; ++sl) {
    const float *tr = a.trow + ((size_t)sl * a.BH + bh) * a.T;
    for (int i = tid; i < a.T; i += 256) acc += tr[i];
  }
  red[tid] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.dtau[bh] = red[0] * a.rsd;
}

hipError_t launch_dtau(const BwdArgs &a, hipStream_t s) {
  if (!a.dtau) return hipSuccess;
  hipLaunchKernelGGL(bwd_dtau_kernel, dim3((unsigned)a.BH), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CLAMP>
hipError_t launch_bwd_d(int mode, const BwdArgs &a, hipStream_t s) {
  const bool dil = mode == 1;
  const size_t rows = (size_t)a.BH * a.T;
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0,
                     s, a, dil ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nqs = (a.T + 31) / 32;
  const int nkb = (a.T + kColKeys - 1) / kColKeys;
  const int nqb = (a.T + 127) / 128;
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
    if (!a.cin_given) e = launch_colsum_bf16(f, s);
    if (e != hipSuccess) return e;
    // dV, dK', the parts of rho and the later blocks' g sums (read by the dQ pass)
    hipLaunchKernelGGL((bwd_dkdv_kernel<true, D, CLAMP>), dim3((unsigned)(nkb * a.BH)), dim3(256),
                       0, s, a, nqs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<true, D, CLAMP>), dim3((unsigned)(nqb * a.BH)), dim3(256), 0,
                       s, a, nqb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dtau(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkrho_kernel<D>), dim3((unsigned)(nkb * a.BH)), dim3(256), 0, s, a,
                       nqs);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<false, D, false>), dim3((unsigned)(nqb * a.BH)), dim3(256),
                       0, s, a, nqb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_dtau(a, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<false, D, false>), dim3((unsigned)(nkb * a.BH)), dim3(256),
                       0, s, a, nqs);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16(int mode, const BwdArgs &a, hipStream_t s) {
  // the 1/D clamp matters only for dilution with eps below 2^-63 (eps = 0)
  const bool clamp = mode == 1 && !(a.eps >= kNoClampEps);
  switch (a.D) {
    case 64: return clamp ? launch_bwd_d<64, true>(mode, a, s) : launch_bwd_d<64, false>(mode, a, s);
    case 128:
      return clamp ? launch_bwd_d<128, true>(mode, a, s) : launch_bwd_d<128, false>(mode, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
