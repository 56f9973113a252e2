// launch.hpp -- host-side launchers of the attention kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kHeadDim = 64;  // default head dimension of the row-load helpers

// Row-major passes over the causal score matrix (one workgroup per query
// block).  lse2 is the log2-domain log-sum-exp of each row.
enum RowMode { kRowTempered = 0, kRowLse = 1, kRowShare = 2 };

struct FwdArgs {
  const void *q, *k, *v;
  void *out;
  float *lse2;          // [BH*Tq] workspace (dilution) or NULL
  float *lse_nat;       // [BH*Tq] optional natural-log output
  float *cin;           // committed demand per 32-row query block (dilution); the
                        // bf16 path stores each entry as a bf16 (hi, lo) pair of
                        // committed + eps in the same 32 bits
  const float *demand_in;  // [BH*kstride] demand committed before the first query
                           // row (dilution), or NULL for none
  float *demand_out;    // [BH*kstride] optional final column totals (dilution);
                        // may be demand_in itself
  float *rowsum_out;    // [BH*Tq] optional row sums of the shares (dilution)
  int BH;
  int T;                // keys 0..T-1; query row r sits at position T - Tq + r
  int Tq;               // query rows per head (Q, out and the per-row arrays)
  int kstride;          // rows per head of K, V and the demand arrays (>= T)
  int vrow0;            // first position the row kernels cover: T - Tq rounded
                        // down to a multiple of 128 (0 for a whole prefill)
  int D;                // head dimension: 64 (both storage types) or 128 (bf16)
  int ksplit;           // dilution row stages: key-tile ranges per query block
                        // (1: none; >1: partials in part_ml / part_o, then a
                        // combine pass)
  float *part_ml;       // [BH*Tq*ksplit*2] per-range (max, sum) / row sum
  float *part_o;        // [BH*Tq*ksplit*D] per-range unnormalised share @ V
  const float *tau_bh;  // [BH] per-(batch, head) multipliers, or NULL
  float c2;             // tau / sqrt(d) * log2(e); with tau_bh: log2(e) / sqrt(d),
                        // and head bh uses tau_bh[bh] * c2
  float eps;
};

// The logit scale (log2 units) of head bh.
__device__ __forceinline__ float head_c2(const FwdArgs &a, int bh) {
  return a.tau_bh ? a.tau_bh[bh] * a.c2 : a.c2;
}

// First position the row kernels cover for keys 0..T-1 and Tq query rows at
// positions T-Tq..T-1: the first row's position rounded down to the largest
// query block (128 rows).
__host__ __device__ inline int first_block_row(int T, int Tq) { return ((T - Tq) / 128) * 128; }

// Key-tile ranges per query block for the bf16 dilution row stages: grids of
// fewer than 512 workgroups (a chunk of a prefill, few heads) leave CUs with a
// single wave per SIMD, so each query block's keys are split over up to 8
// workgroups whose partial results a combine pass adds in a fixed order.
__host__ __device__ inline int row_ksplit(int BH, int T, int Tq, int dtype_bf16) {
  if (!dtype_bf16) return 1;
  const int vrow0 = first_block_row(T, Tq);
  const long items = (long)((T + 127) / 128 - vrow0 / 128) * BH;
  if (items >= 512) return 1;
  int ks = (int)((1024 + items - 1) / items);
  const int tiles = (T + 63) / 64;
  if (ks > tiles) ks = tiles;
  return ks > 8 ? 8 : (ks < 1 ? 1 : ks);
}

// Committed-demand storage: 32-row query block qs keeps one entry per key
// j < 32*(qs+1) -- the demand its rows inherit from every earlier row,
// including rows before a prefill chunk -- at offset cin_block_offset(qs)
// inside its head's region.  Blocks start at qs0 = vrow0/32.
__host__ __device__ inline size_t cin_block_offset(int qs, int vrow0) {
  const size_t b = (size_t)qs, b0 = (size_t)(vrow0 / 32);
  return 16 * b * (b + 1) - 16 * b0 * (b0 + 1);
}
__host__ __device__ inline size_t cin_floats_per_head(int T, int vrow0) {
  return cin_block_offset((T + 31) / 32, vrow0);
}

hipError_t launch_rows_bf16(int mode, const FwdArgs &a, hipStream_t s);
hipError_t launch_colsum_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_rows_f32(int mode, const FwdArgs &a, hipStream_t s);
hipError_t launch_colsum_f32(const FwdArgs &a, hipStream_t s);

// Suffix sums of the committed-demand gradient terms: query sub-block qs keeps
// one entry per key j < 32*(qs+1), at offset 16*qs*(qs+1) in its head's region.
__host__ __device__ inline size_t gin_floats_per_head(int T) {
  const size_t n = ((size_t)T + 31) / 32;
  return 16 * n * (n + 1);
}

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;       // [BH*T] natural-log log-sum-exp of each row (forward)
  const float *rowsum;    // [BH*T] dilution: row sums of the shares (forward)
  void *dq, *dk, *dv;
  float *lse2;            // [BH*T] workspace: log2-domain log-sum-exp
  float *invr;            // [BH*T] workspace: 1 / rowsum (dilution)
  float *dri;             // [BH*T] workspace: <dO_i, o_i> / rowsum (tempered: <dO_i, o_i>)
  float *rho;             // [BH*T] workspace: sum_j p_ij dp_ij (dilution)
  float *cin;             // committed demand per (32-row block, key): bf16 path
                          // committed + eps as bf16 pairs, fp32 path fp32
  float *gin;             // later blocks' share-gradient sums per (block, key): bf16
                          // pairs (bf16 path) or fp32
  void *pk;               // [BH*T*D] workspace, fp32 path: sum_j p_ij k_j (dilution)
  float *dkp;             // [BH*T*D] workspace, fp32 (bf16 dilution): sum_i p_ij dp_ij q_i
  float *rhop;            // [BH][ceil(T/128)][T] workspace (bf16 dilution): per row, each
                          // 128-key block's part of rho
  const float *tau_bh;    // [BH] per-head multipliers, or NULL (then c2, c carry tau)
  float *dtau;            // [BH] output: dL/dtau per head, or NULL
  float *trow;            // [tslices][BH*T] workspace: <q_i, dQ_i / c> per row (for
                          // dtau), in tslices partial sums over slices of d
  int tslices;            // partial sums per row (1: every dq kernel covers all of d)
  int cin_given;          // 1: cin is the forward's committed-demand table (read as is)
  int BH, T, D;           // D: head dimension, 64 or 128
  float c2;               // tau / sqrt(d) * log2(e)  (with tau_bh: log2(e) / sqrt(d))
  float c;                // tau / sqrt(d)            (with tau_bh: 1 / sqrt(d))
  float rsd;              // 1 / sqrt(d)
  float eps;
};

hipError_t launch_bwd_bf16(int mode, const BwdArgs &a, hipStream_t s);
hipError_t launch_bwd_f32(int mode, const BwdArgs &a, hipStream_t s);

struct DecodeArgs {
  const void *q, *kc, *vc;
  float *demand;
  void *out;
  const int32_t *kv_len;
  const float *tau_sh;   // [S*H] per-(sequence, head) multipliers, or NULL
  int S, H, Lcap, splits, chunk;
  int D;                 // head dimension: 64 or 128
  float c2, eps;         // c2: tau / sqrt(d) * log2(e), or log2(e) / sqrt(d) with tau_sh
  float *scores;   // [S*H*Lcap]
  float *part_ml;  // [S*H*splits*2]  (max, sum) in log2 domain
  float *part_o;   // [S*H*splits*(D+1)]
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);

// Rotary position embedding of `rows` rows per head (rope.hip): row t of head
// bh is read at x[(bh * in_stride + t) * D] and written at
// y[(bh * out_stride + t) * D], turned at position pos0 + t by freq[m] per
// dimension pair (2m, 2m+1).
struct RopeArgs {
  const void *x;
  void *y;
  int BH, rows, D;
  size_t in_stride, out_stride;
  const float *freq;     // [D/2]
  long pos0;
};
hipError_t launch_rope(const RopeArgs &a, int bf16, hipStream_t s);

// Record a HIP error as the text attn_strerror(ATTN_EHIP) reports; returns ATTN_EHIP.
int record_hip_error(hipError_t e);

// attn_fwd's host-side argument checks (everything but the workspace and the
// device): ATTN_OK or the status attn_fwd would return for these arguments.
int validate_fwd(const void *q, const void *k, const void *v, const void *out, int B, int H, int T,
                 int d, float tau, int mode, float eps, int dtype);

}  // namespace attn
