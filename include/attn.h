/*
 * attn.h -- C ABI of the MI355X (gfx950) reshaped-softmax causal attention
 * library (libattn.so).
 *
 * Two reshapings of causal softmax attention are provided:
 *
 *  ATTN_TEMPERED  o_i = sum_{j<=i} softmax_j(tau * <q_i,k_j> / sqrt(d)) v_j.
 *                 The multiplier tau sharpens (tau > 1) or flattens the bids:
 *                 Focal Attention ("Learning to Focus", sec. 2.1, eq.
 *                 focal-const) divides the logits by t < 1, i.e. tau = 1/t;
 *                 YaRN ("YaRN > Attention Temperature Scaling") multiplies the
 *                 scores by sqrt(t) with t = 0.1 ln s + 1 (see attn_yarn_tau).
 *
 *  ATTN_DILUTION  DilutionAttention v0.1.0, section "The operator":
 *                   p         = causal_softmax(tau * q k^T / sqrt(d))   (bids)
 *                   committed = exclusive cumulative sum of p down each key
 *                               column (demand from earlier queries)
 *                   share     = p / (committed + p + eps)
 *                   A         = share / rowsum(share);  out = A @ v
 *                 The page writes the plain 1/sqrt(d) scale, i.e. tau = 1.
 *
 * attn_decode is the cached-decode form of dilution (same page: the ordinary
 * key/value cache plus one running demand total per key and head).
 *
 * Conventions for every entry point
 *  - Device pointers are plain HIP device addresses owned by the caller; the
 *    library never allocates, frees or retains them.  Calls are asynchronous:
 *    all work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *    stream) and the call returns once it is enqueued.  Errors raised while
 *    kernels run surface at the caller's next synchronisation on that stream.
 *  - Tensors are dense and row-major: [B,H,T,d] for the forward pass,
 *    [S,H,Lcap,d] for the decode caches, with d innermost.  All device
 *    pointers must be 16-byte aligned.
 *  - Arithmetic: products on bf16 matrix cores with fp32 accumulation for
 *    ATTN_BF16 storage; exponentials, scans, reciprocals and row sums in fp32.
 *    ATTN_F32 storage runs an fp32-only path (no bf16 rounding anywhere).
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders, bit-identical output for identical inputs.
 *  - Return value: ATTN_OK or a negative attn_status.  Nothing is enqueued
 *    when a call returns an error (except ATTN_EHIP, which reports a failed
 *    launch).  The library never aborts or throws across this boundary.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,     /* bad argument: null/misaligned pointer, size <= 0, tau/eps out of range */
  ATTN_ENOTSUP = -2,    /* valid but unsupported: head dim, fp32 decode, not gfx950 */
  ATTN_EWORKSPACE = -3, /* workspace missing or smaller than *_workspace_bytes() */
  ATTN_EHIP = -4,       /* a HIP runtime call or kernel launch failed */
  ATTN_ESCRATCH = -5    /* attn_fwd_noalloc: the shape needs more workspace than
                           the library's fixed scratch array holds */
} attn_status;

/* Size of the fixed device scratch array behind attn_fwd_noalloc. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum { ATTN_TEMPERED = 0, ATTN_DILUTION = 1 } attn_mode;
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Bytes of device workspace attn_fwd needs for this shape (0 for
 * ATTN_TEMPERED).  Dilution keeps the fp32 log-sum-exp of every query row
 * (B*H*T floats) and the demand committed before every 32-row query block on
 * each key up to the block's end (B*H*16*n*(n+1) floats, n = ceil(T/32)).
 * Returns 0 for an invalid shape. */
size_t attn_fwd_workspace_bytes(int B, int H, int T, int d, int mode, int dtype);

/* Causal attention forward pass (both modes; see top of file).
 *   q, k, v    [B,H,T,d] device arrays of `dtype` (inputs, not modified)
 *   out        [B,H,T,d] device array of `dtype` (output; may not alias q/k/v)
 *   B, H, T    batch, heads, sequence length (each >= 1; T < 16777216 and
 *              T * d * element size < 2^31: the kernels address one head's
 *              rows with 32-bit byte offsets -- for bf16 T < 2^24 at d = 64
 *              and T < 2^23 at d = 128, for fp32 half of that; B * H * T
 *              <= 2^32 rows in all; else ATTN_EINVAL)
 *   d          head dimension: 64 or 128 (else ATTN_ENOTSUP)
 *   tau        logit multiplier, finite and >= 0 (tau = 0 gives uniform bids)
 *   mode       ATTN_TEMPERED or ATTN_DILUTION
 *   eps        share-denominator constant (dilution), finite and >= 0
 *   dtype      ATTN_F32 or ATTN_BF16
 *   workspace  device scratch of >= attn_fwd_workspace_bytes(...) bytes (may
 *              be NULL when that is 0); contents on entry are ignored.  It is
 *              written, so it may not overlap q, k, v, out or any optional
 *              output (else ATTN_EINVAL)
 *   hip_stream hipStream_t to enqueue on (NULL: default stream) */
int attn_fwd(const void *q, const void *k, const void *v, void *out, int B, int H, int T, int d,
             float tau, int mode, float eps, int dtype, void *workspace, size_t workspace_bytes,
             void *hip_stream);

/* attn_fwd with three optional fp32 outputs (NULL to skip any):
 *   lse_out    [B,H,T]  natural-log log-sum-exp of each query row's tempered
 *              logits, log sum_{j<=i} exp(tau <q_i,k_j>/sqrt(d))
 *   demand_out [B,H,T]  dilution only: each key's final column total
 *              sum_i p_ij -- the running demand a cached decode continues
 *              from (DilutionAttention v0.1.0, cached decoding).
 *   rowsum_out [B,H,T]  dilution only: each row's sum of shares, the
 *              renormaliser of A ("The operator"); attn_bwd needs it.
 * demand_out and rowsum_out must be NULL in ATTN_TEMPERED mode (else
 * ATTN_EINVAL).  The outputs may not alias each other or any tensor. */
int attn_fwd_ex(const void *q, const void *k, const void *v, void *out, int B, int H, int T,
                int d, float tau, int mode, float eps, int dtype, void *workspace,
                size_t workspace_bytes, float *lse_out, float *demand_out, float *rowsum_out,
                void *hip_stream);

/* attn_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments are attn_fwd's without the workspace: the dilution workspace is
 * a fixed array of ATTN_NOALLOC_SCRATCH_BYTES (128 MiB) inside the library,
 * one per GPU, held from the time the library's code is loaded on that GPU
 * until the process ends.  The call allocates, frees and clears nothing.
 * Limit: shapes whose attn_fwd_workspace_bytes(...) exceeds that size (for
 * dilution, about B*H*T*T/16 bytes: B*H = 16 heads at T = 8192 fit) return
 * ATTN_ESCRATCH with nothing enqueued; ATTN_TEMPERED needs no workspace and
 * has no limit beyond attn_fwd's.  Every call on one GPU shares that GPU's
 * array and leaves its contents behind: calls on one GPU whose executions
 * overlap (other streams, other host threads) race on it and must be
 * ordered by the caller.  No kernel needs the array cleared between calls.
 * Results are bit for bit those of attn_fwd with a workspace of its own. */
int attn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int B, int H, int T,
                     int d, float tau, int mode, float eps, int dtype, void *hip_stream);

/* Bytes of device workspace attn_bwd and attn_bwd_ex need: five fp32 values
 * per query row, and for dilution the committed
 * demand and the later rows' gradient sums per (32-row query block, key):
 * B*H*16*n*(n+1) 32-bit values each, n = ceil(T/32), plus a [B,H,T,d] fp32
 * array and, for ATTN_BF16, B*H*ceil(T/128)*T fp32 values.  0 for an
 * unsupported shape, mode, head dimension or dtype. */
size_t attn_bwd_workspace_bytes(int B, int H, int T, int d, int mode, int dtype);

/* Exact gradients of either operator (DilutionAttention v0.1.0: the release's
 * kernels train with exact gradients; "The operator" defines what is
 * differentiated).  For the loss L with dL/dout = dout:
 *   q, k, v, out, dout  [B,H,T,d] device arrays of `dtype`: the forward's
 *                       inputs, its output, and the incoming gradient
 *   lse                 [B,H,T] fp32: the forward's lse_out (natural log)
 *   rowsum              [B,H,T] fp32: the forward's rowsum_out (dilution;
 *                       ignored and may be NULL for ATTN_TEMPERED)
 *   dq, dk, dv          [B,H,T,d] outputs of `dtype`, overwritten; may not
 *                       alias each other or any input
 *   B, H, T, d, tau, mode, eps  as passed to the forward
 *   dtype               ATTN_BF16 (matrix-core kernels) or ATTN_F32
 *                       (vector-ALU kernels in full single precision), each
 *                       at d = 64 or 128; else ATTN_ENOTSUP
 *   workspace           device scratch of >= attn_bwd_workspace_bytes(...)
 *                       bytes; contents on entry are ignored.  It is
 *                       written, so it may not overlap any other argument
 *                       (else ATTN_EINVAL)
 * Deterministic: fixed reduction orders, no atomics.  attn_bwd is
 * attn_bwd_ex with tau_bh = dtau_out = fwd_workspace = NULL. */
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
             const float *lse, const float *rowsum, void *dq, void *dk, void *dv, int B, int H,
             int T, int d, float tau, int mode, float eps, int dtype, void *workspace,
             size_t workspace_bytes, void *hip_stream);

/* attn_bwd with per-head multipliers and the gradient with respect to them
 * ("Learning to Focus", sec. 2.2: the temperature is learned, so training
 * needs dL/dtau), and optionally the dilution forward's own workspace.
 * Arguments as attn_bwd, and:
 *   tau_bh    [B,H] fp32 device array or NULL: head (b,h)'s multiplier, as
 *             given to attn_prefill (which produces the matching lse and
 *             rowsum through lse_out/rowsum_out); tau is then ignored.
 *             Values finite and >= 0, read on the device and not checked.
 *   dtau_out  [B,H] fp32 device array or NULL: receives, per head,
 *             dL/dtau_bh = sum_ij dS_ij <q_i, k_j> / sqrt(d) with dS the
 *             gradient of the logits (for a scalar tau shared by all heads,
 *             dL/dtau is the sum over heads).  It is formed as
 *             sum_i <q_i, dQ_i / c> / sqrt(d) with fp32 row terms, so it is
 *             defined at tau = 0 too.  May not overlap any other argument.
 *   fwd_workspace, fwd_workspace_bytes
 *             NULL and 0, or (ATTN_DILUTION; ignored for ATTN_TEMPERED) the
 *             workspace of the forward that produced `out`, `lse` and
 *             `rowsum` from these q, k, v (attn_fwd / attn_fwd_ex, the three
 *             stage calls, or attn_prefill of the whole sequence with
 *             Tq = Tk = T and no carried demand), with the same B, H, T, d,
 *             tau or tau_bh, eps and dtype, and not written since.  Read
 *             only: its committed-demand table is used as is instead of
 *             being recomputed (one pass over all pairs fewer).  The caller
 *             vouches for it as for lse and rowsum; nothing on the device
 *             checks it.  fwd_workspace_bytes must be >=
 *             attn_fwd_workspace_bytes(B,H,T,d,ATTN_DILUTION,dtype) and the
 *             pointer 16-byte aligned (else ATTN_EWORKSPACE); it may not
 *             overlap dq, dk, dv, dtau_out or `workspace` (else ATTN_EINVAL).
 * tau_bh may not overlap dq, dk, dv or dtau_out. */
int attn_bwd_ex(const void *q, const void *k, const void *v, const void *out, const void *dout,
                const float *lse, const float *rowsum, void *dq, void *dk, void *dv, int B,
                int H, int T, int d, float tau, const float *tau_bh, int mode, float eps,
                int dtype, float *dtau_out, const void *fwd_workspace,
                size_t fwd_workspace_bytes, void *workspace, size_t workspace_bytes,
                void *hip_stream);

/* The dilution forward pass, one stage per call (attn_fwd with ATTN_DILUTION
 * runs exactly these three in order on one stream).  All three take the same
 * shape, tau, dtype and workspace (>= attn_fwd_workspace_bytes(...,
 * ATTN_DILUTION, dtype), overlapping no argument, as for attn_fwd); a stage
 * reads what the previous stage left in the workspace, so they must be
 * enqueued in order on one stream.
 *
 * attn_dilution_lse        stage 1: log-sum-exp of each query row's logits,
 *                          the normaliser of the causal softmax bids ("The
 *                          operator").  lse_out: optional [B,H,T] fp32
 *                          natural-log copy.
 * attn_dilution_committed  stage 2: for every 32-row query block and every
 *                          earlier key, the demand committed by all earlier
 *                          rows -- the exclusive cumulative sum of the bids
 *                          down each key column ("The operator", committed),
 *                          taken block by block.  It stores committed +
 *                          eps, so stage 3 must be given the same eps.
 *                          demand_out: optional [B,H,T] fp32 final column
 *                          totals.
 * attn_dilution_shares     stage 3: shares p / (committed + p + eps) with the
 *                          prefix finished inside each block, then out = A @ v
 *                          with A the row-renormalised shares ("The operator",
 *                          share and A). */
int attn_dilution_lse(const void *q, const void *k, int B, int H, int T, int d, float tau,
                      int dtype, void *workspace, size_t workspace_bytes, float *lse_out,
                      void *hip_stream);
int attn_dilution_committed(const void *q, const void *k, int B, int H, int T, int d, float tau,
                            float eps, int dtype, void *workspace, size_t workspace_bytes,
                            float *demand_out, void *hip_stream);
int attn_dilution_shares(const void *q, const void *k, const void *v, void *out, int B, int H,
                         int T, int d, float tau, float eps, int dtype, void *workspace,
                         size_t workspace_bytes, void *hip_stream);

/* Bytes of device workspace attn_prefill needs for Tq query rows over Tk keys
 * (0 for ATTN_TEMPERED, or for an invalid shape): the fp32 log-sum-exp of
 * each query row and the committed demand of each 32-row query block from
 * position P = Tk - Tq rounded down to 128 onwards. */
size_t attn_prefill_workspace_bytes(int B, int H, int Tq, int Tk, int d, int mode, int dtype);

/* One chunk of a prefill over cached keys, either operator: the Tq new query
 * rows are the positions P = Tk-Tq .. Tk-1, and the row at position i sees
 * keys 0..i.  Dilution continues from the demand the rows before P committed
 * (DilutionAttention v0.1.0: cached decoding keeps one running demand total
 * per key and head; "The operator" then runs unchanged with committed_ij =
 * demand_in_j + the bids of this chunk's rows above i).  A whole prefill is
 * Tq = Tk with no demand; a one-row chunk is one decode step with the new
 * key visible.
 *   q          [B,H,Tq,d] of `dtype`: the chunk's queries
 *   kcache, vcache  [B,H,Lcap,d] of `dtype`: keys/values 0..Tk-1 (the caller
 *              has written the chunk's own keys/values at P..Tk-1); rows
 *              Tk..Lcap-1 are not read
 *   out        [B,H,Tq,d] of `dtype` (may not alias q or the caches)
 *   B, H       >= 1;  1 <= Tq <= Tk <= Lcap < 16777216, and Lcap * d *
 *              element size < 2^31 (as T for attn_fwd)
 *   d, tau, mode, eps, dtype  as for attn_fwd
 *   tau_bh     [B,H] fp32 device array or NULL: when given, head (b,h) uses
 *              the multiplier tau_bh[b*H+h] in place of tau -- the per-
 *              sequence temperature a learned-temperature layer produces
 *              ("Learning to Focus", sec. 2.2: tau_learned = clip(mean(X w),
 *              tau_min, tau_max) replaces sqrt(d), i.e. a multiplier
 *              sqrt(d)/tau_learned).  Values must be finite and >= 0; they
 *              are read on the device and not checked.
 *   demand_in  [B,H,Lcap] fp32 (dilution): each key's demand from the rows
 *              before P (the new keys' entries are normally 0), or NULL for
 *              none; entries >= Tk are not read
 *   demand_out [B,H,Lcap] fp32 (dilution), optional: demand_in + the column
 *              totals of this chunk's bids on keys < Tk (entries >= Tk are
 *              not written).  May be demand_in itself (updated in place);
 *              otherwise no overlap with it.
 *   lse_out    [B,H,Tq] fp32, optional: natural-log log-sum-exp per row
 *   rowsum_out [B,H,Tq] fp32 (dilution), optional: each row's sum of shares,
 *              the renormaliser of A (with lse_out, what attn_bwd_ex needs)
 *   workspace  >= attn_prefill_workspace_bytes(B,H,Tq,Tk,d,mode,dtype) bytes
 * demand_in, demand_out and rowsum_out must be NULL for ATTN_TEMPERED (else
 * ATTN_EINVAL).  Outputs may not alias each other or any tensor argument. */
int attn_prefill(const void *q, const void *kcache, const void *vcache, void *out, int B, int H,
                 int Tq, int Tk, int Lcap, int d, float tau, const float *tau_bh, int mode,
                 float eps, int dtype, const float *demand_in, float *demand_out, float *lse_out,
                 float *rowsum_out, void *workspace, size_t workspace_bytes, void *hip_stream);

/* Bytes of device workspace attn_prefill_rope needs: the rotated query rows
 * [B,H,Tq,d] and rotated keys [B,H,Lcap,d] in `dtype`, then (ATTN_DILUTION)
 * attn_prefill_workspace_bytes(B,H,Tq,Tk,d,mode,dtype).  0 for an invalid
 * shape, mode, head dimension or dtype. */
size_t attn_prefill_rope_workspace_bytes(int B, int H, int Tq, int Tk, int Lcap, int d, int mode,
                                         int dtype);

/* attn_prefill with rotary position embedding applied to Q and K first
 * ("YaRN > Attention Temperature Scaling", code cell In[16]: each token's
 * query and key are rotated at its position with the per-pair frequencies
 * times YaRN's gamma, then the scores are taken and multiplied by sqrt(t) --
 * here the multiplier tau or tau_bh).  Arguments as attn_prefill, with the
 * cache holding the keys BEFORE rotation, and:
 *   rope_freq  [d/2] fp32 device array: the frequency of dimension pair
 *              (2m, 2m+1), YaRN's per-pair gamma already applied by the
 *              caller (the page leaves gamma's helpers undefined); not
 *              checked on the host (NULL: ATTN_EINVAL)
 *   pos0       position of key 0 (>= 0, pos0 + Tk < 2^31): key j sits at
 *              pos0 + j and the chunk's query row r at pos0 + Tk - Tq + r
 * Row x at position n has pair m turned counter-clockwise by the angle
 * n * rope_freq[m]: (a, b) -> (a cos - b sin, a sin + b cos).  The angle is
 * reduced in double precision; the rotated rows are rounded once to `dtype`
 * in the workspace, and the attention kernels read them from there.
 * Scores then depend on the distance between positions only, so pos0 moves
 * nothing but rounding.  workspace: >= attn_prefill_rope_workspace_bytes(...)
 * bytes (needed in both modes), not overlapping any argument. */
int attn_prefill_rope(const void *q, const void *kcache, const void *vcache, void *out, int B,
                      int H, int Tq, int Tk, int Lcap, int d, float tau, const float *tau_bh,
                      int mode, float eps, int dtype, const float *rope_freq, int pos0,
                      const float *demand_in, float *demand_out, float *lse_out,
                      float *rowsum_out, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/* Bytes of device workspace attn_decode needs (per-(sequence,head,split)
 * partial maxima, sums and weighted values plus one fp32 score per cached
 * key). */
size_t attn_decode_workspace_bytes(int S, int H, int Lcap, int d);

/* One cached-decode step of dilution attention for S sequences at once.
 *   q        [S,H,d] bf16: this step's query per (sequence, head)
 *   kcache   [S,H,Lcap,d] bf16, vcache [S,H,Lcap,d] bf16: cached keys/values
 *   demand   [S,H,Lcap] fp32, READ-MODIFY-WRITE: on entry the demand each key
 *            has received from earlier queries; on return demand_j += p_j,
 *            where p is this step's softmax bid.  The output uses the demand
 *            as it stood on entry: share_j = p_j / (demand_j + p_j + eps).
 *   out      [S,H,d] bf16: sum_j share_j v_j / sum_j share_j
 *   kv_len   device int32 [S], visible keys per sequence (1..Lcap), or NULL
 *            for Lcap everywhere.  To decode with the new token's own key, the
 *            caller writes its k/v at index kv_len-1 and zeroes its demand.
 *            A kv_len outside [1, Lcap] is clamped to that range on device.
 *   d        64 or 128
 *   tau, eps as for attn_fwd; dtype must be ATTN_BF16 (else ATTN_ENOTSUP).
 *   workspace >= attn_decode_workspace_bytes(S,H,Lcap,d) bytes; it is written,
 *            so it may not overlap any other argument (else ATTN_EINVAL).
 * Consecutive steps must be ordered on one stream (each reads the demand the
 * previous one wrote). */
int attn_decode(const void *q, const void *kcache, const void *vcache, float *demand, void *out,
                int S, int H, int Lcap, const int32_t *kv_len, int d, float tau, float eps,
                int dtype, void *workspace, size_t workspace_bytes, void *hip_stream);

/* attn_decode with a per-(sequence, head) multiplier: tau_sh is an [S,H] fp32
 * device array (or NULL for `tau` everywhere); (s,h) uses tau_sh[s*H+h] in
 * place of tau, as attn_prefill's tau_bh (values finite and >= 0, not
 * checked). */
int attn_decode_ex(const void *q, const void *kcache, const void *vcache, float *demand, void *out,
                   int S, int H, int Lcap, const int32_t *kv_len, int d, float tau,
                   const float *tau_sh, float eps, int dtype, void *workspace,
                   size_t workspace_bytes, void *hip_stream);

/* YaRN attention temperature ("YaRN > Attention Temperature Scaling"):
 * returns sqrt(t) with t = 0.1 ln(s) + 1, the multiplier for extension
 * factor s >= 1; NaN for s < 1 or NaN. */
double attn_yarn_tau(double s);

/* Static description of a status code (never NULL). For ATTN_EHIP it names
 * the last HIP error the library saw. */
const char *attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
