/*
 * oracle.c -- plain fp64 CPU oracle for reshaped-softmax causal attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The HIP product path
 * shares no code, header, table or helper with it.
 *
 * Every quantity is computed straight from its definition, one query row at a
 * time (the dilution passes hold up to 64 rows' bids at once, each share and
 * sum still formed for one row), in double precision.  Inputs arrive as
 * fp64, fp32 or raw bf16 bits and are widened exactly to double before any
 * arithmetic.
 *
 * Sources (cited by page title and section):
 *   [FOCAL]  "Learning to Focus: Focal Attention for Selective and Scalable
 *            Transformers" (arXiv 2511.06818), sec. 2 (softmax, eqs. 1-2) and
 *            sec. 2.1 (scaled dot-product attention, eq. focal-const).
 *   [YARN]   "YaRN > Attention Temperature Scaling" (Brenndoerfer), the
 *            temperature formula t = 0.1 ln s + 1 and the sqrt(t) score
 *            multiplier (code cells In[14] and In[16]).
 *   [DIL]    "DilutionAttention v0.1.0 - results", section "The operator":
 *            the four-line definition (bids, committed, share, A/out) and the
 *            sentence on cached decoding; section "Everything behind these
 *            charts" (the release's kernels carry exact gradients).
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes):
 *   - tau multiplies the already scaled logits: s = tau * <q,k> / sqrt(d)
 *     ([YARN] In[16] multiplies the scores by sqrt(t) after the 1/sqrt(d)).
 *   - causal means key j visible to query i iff j <= i.
 *   - committed(i,j) sums the bids p(i',j) of all earlier queries i' < i
 *     down key column j ("demand from earlier queries", [DIL]).
 *   - eps appears only in the share denominator; a zero bid gets a zero
 *     share (so eps = 0 never yields 0/0).
 *   - the decode step uses the demand as it stood before the step, then
 *     adds this query's bids to it (the bid, not the share).
 *
 * Parity of every function here is pinned by the CPU tests against closed
 * forms, brute force on tiny inputs, a library attention routine and the
 * pages' invariants; none of them is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

/* Exact widening of one stored element to double. */
static double widen(const void *base, int dtype, size_t idx) {
  if (dtype == OR_F64) return ((const double *)base)[idx];
  if (dtype == OR_F32) return (double)((const float *)base)[idx];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Copy n consecutive stored elements starting at idx into a double buffer. */
static void widen_block(double *dst, const void *base, int dtype, size_t idx, size_t n) {
  for (size_t e = 0; e < n; ++e) dst[e] = widen(base, dtype, idx + e);
}

static double dot(const double *a, const double *b, int d) {
  double acc = 0.0;
  for (int e = 0; e < d; ++e) acc += a[e] * b[e];
  return acc;
}

/* [YARN]: t = 0.1 ln(s) + 1 and the score multiplier sqrt(t). */
double oracle_yarn_t(double s) { return 0.1 * log(s) + 1.0; }
double oracle_yarn_tau(double s) { return sqrt(oracle_yarn_t(s)); }

static int nthreads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

#define MAX_PARTS 256
/* rows shorter than this are summed by one thread (fork/join costs more) */
#define PAR_MIN_ROW 256
/* query rows the dilution passes take together (inner parallelism) */
#define ROW_BATCH 64

/*
 * Causal softmax bids of one query row ([FOCAL] eq. 1 applied to the logits
 * of eq. focal-const, restricted to the visible keys j <= i):
 *   s_j = c <q_i, k_j>,  c = tau / sqrt(d)
 *   lse = log sum_j exp(s_j)   (computed around the row maximum)
 *   p_j = exp(s_j - lse)
 * Writes p[0..i] and returns lse.
 */
static double causal_bids(const double *qi, const double *K, int i, int d, double c,
                          double *p, int inner_parallel) {
  /* Work is split into fixed contiguous ranges of j, and the per-range maxima
     and sums are combined in range order, so the result does not depend on
     thread timing. */
  int parts = (inner_parallel && i + 1 >= PAR_MIN_ROW) ? nthreads() : 1;
  if (parts > MAX_PARTS) parts = MAX_PARTS;
  double pm[MAX_PARTS], pz[MAX_PARTS];
  double lse = 0.0;
#pragma omp parallel num_threads(parts) if (parts > 1)
  {
    int t = 0, n = 1;
#ifdef _OPENMP
    t = omp_get_thread_num();
    n = omp_get_num_threads();
#endif
    const long lo = (long)(i + 1) * t / n, hi = (long)(i + 1) * (t + 1) / n;
    double m = -INFINITY;
    for (long j = lo; j < hi; ++j) {
      p[j] = c * dot(qi, K + (size_t)j * d, d);
      if (p[j] > m) m = p[j];
    }
    pm[t] = m;
#pragma omp barrier
    double M = -INFINITY;
    for (int u = 0; u < n; ++u)
      if (pm[u] > M) M = pm[u];
    double z = 0.0;
    for (long j = lo; j < hi; ++j) z += exp(p[j] - M);
    pz[t] = z;
#pragma omp barrier
    double Z = 0.0;
    for (int u = 0; u < n; ++u) Z += pz[u];
    const double l = M + log(Z);
    for (long j = lo; j < hi; ++j) p[j] = exp(p[j] - l);
    if (t == 0) lse = l;
  }
  return lse;
}

/*
 * Tempered causal attention ([FOCAL] eq. focal-const with tau = 1/t, and the
 * [YARN] multiplier tau = sqrt(t)):  o_i = sum_{j<=i} p_ij v_j.
 *
 * q,k,v: [B,H,T,d] in dtype; out: [B,H,T,d] fp64; lse (optional): [B,H,T].
 * rows/nrows (optional): only these query rows are computed (others of out
 * and lse are left untouched); rows == NULL computes all rows.
 */
int oracle_tempered_fwd(const void *q, const void *k, const void *v, int dtype, double *out,
                        double *lse, int B, int H, int T, int d, double tau, const int *rows,
                        int nrows) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0) return -1;
  const double c = tau / sqrt((double)d);
  const int nr = rows ? nrows : T;
  double *Kh = malloc(sizeof(double) * (size_t)T * d);
  double *Vh = malloc(sizeof(double) * (size_t)T * d);
  if (!Kh || !Vh) { free(Kh); free(Vh); return -2; }
  for (int bh = 0; bh < B * H; ++bh) {
    const size_t base = (size_t)bh * T * d;
    widen_block(Kh, k, dtype, base, (size_t)T * d);
    widen_block(Vh, v, dtype, base, (size_t)T * d);
    int failed = 0;
#pragma omp parallel
    {
      double *p = malloc(sizeof(double) * (size_t)T);
      double *qi = malloc(sizeof(double) * (size_t)d);
      double *acc = malloc(sizeof(double) * (size_t)d);
      if (!p || !qi || !acc) {
#pragma omp atomic write
        failed = 1;
      } else {
#pragma omp for schedule(dynamic, 8)
        for (int r = 0; r < nr; ++r) {
          const int i = rows ? rows[r] : r;
          if (i < 0 || i >= T) continue;
          widen_block(qi, q, dtype, base + (size_t)i * d, d);
          const double l = causal_bids(qi, Kh, i, d, c, p, 0);
          for (int e = 0; e < d; ++e) acc[e] = 0.0;
          for (int j = 0; j <= i; ++j)
            for (int e = 0; e < d; ++e) acc[e] += p[j] * Vh[(size_t)j * d + e];
          for (int e = 0; e < d; ++e) out[base + (size_t)i * d + e] = acc[e];
          if (lse) lse[(size_t)bh * T + i] = l;
        }
      }
      free(p); free(qi); free(acc);
    }
    if (failed) { free(Kh); free(Vh); return -2; }
  }
  free(Kh); free(Vh);
  return 0;
}

/*
 * One dilution head, rows in increasing order ([DIL] "The operator"):
 *   p        = causal softmax bids of row i
 *   committed_ij = D_j = sum_{i'<i} p_i'j   (running column total, i.e. the
 *                                           exclusive cumulative sum down key
 *                                           column j)
 *   share_ij = p_ij / (committed_ij + p_ij + eps)   (0 where p_ij = 0)
 *   A_ij     = share_ij / sum_j share_ij ;  o_i = sum_j A_ij v_j
 * then D_j += p_ij before the next row.
 * The query rows are the positions P..T-1 (P = 0 for a whole prefill; a
 * later chunk of a prefill starts at P > 0 over the same keys 0..T-1).  Qh,
 * Oh, lse_h and want are indexed by i - P.  want[i - P] != 0 selects the rows
 * whose output is formed (all rows still add their bids to D).  D (length T)
 * enters as the demand already committed before row P -- zero for a plain
 * prefill, the earlier chunks' column totals otherwise -- and leaves as the
 * final column totals.  pbuf and sbuf hold the bids and shares of
 * ROW_BATCH rows (of one row without inner parallelism), T values each.
 */
static void dilution_head(const double *Qh, const double *Kh, const double *Vh, int P, int T,
                          int d, double c, double eps, const unsigned char *want, double *Oh,
                          double *lse_h, double *D, double *pbuf, double *sbuf, int inner_parallel) {
  /* ROW_BATCH rows at a time (one without inner parallelism): first the
     batch's bids, row by row; then the shares, key by key with the rows in
     order, each row's share of key j formed against the demand the rows
     before it committed, after which its own bid joins D_j; last each row's
     sums over its keys in increasing j.  Every value is the expression of
     the definition above for one (row, key) pair; the batch only lets the
     rows share each pass over K and V. */
  const int R = inner_parallel ? ROW_BATCH : 1;
  for (int i0 = P; i0 < T; i0 += R) {
    const int i1 = i0 + R < T ? i0 + R : T;
#pragma omp parallel for if (inner_parallel) schedule(dynamic, 1)
    for (int i = i0; i < i1; ++i) {
      const int li = i - P;
      double *p = pbuf + (size_t)(i - i0) * T;
      const double l = causal_bids(Qh + (size_t)li * d, Kh, i, d, c, p, 0);
      if (lse_h) lse_h[li] = l;
    }
#pragma omp parallel for if (inner_parallel) schedule(static)
    for (int j = 0; j < i1; ++j) {
      for (int i = j > i0 ? j : i0; i < i1; ++i) {
        const double *p = pbuf + (size_t)(i - i0) * T;
        sbuf[(size_t)(i - i0) * T + j] = p[j] > 0.0 ? p[j] / (D[j] + p[j] + eps) : 0.0;
        D[j] += p[j];
      }
    }
#pragma omp parallel for if (inner_parallel) schedule(dynamic, 1)
    for (int i = i0; i < i1; ++i) {
      const int li = i - P;
      if (want && !want[li]) continue;
      const double *sh = sbuf + (size_t)(i - i0) * T;
      double r = 0.0;
      double acc[512];
      for (int e = 0; e < d; ++e) acc[e] = 0.0;
      for (int j = 0; j <= i; ++j) {
        const double share = sh[j];
        if (share > 0.0) {
          r += share;
          for (int e = 0; e < d; ++e) acc[e] += share * Vh[(size_t)j * d + e];
        }
      }
      for (int e = 0; e < d; ++e) Oh[(size_t)li * d + e] = acc[e] / r;
    }
  }
}

/* Widen one head's inputs and run dilution_head on it (0 on success). */
static int dilution_one_head(const void *q, const void *k, const void *v, int dtype, double *out,
                             double *lse, double *demand, int B, int H, int T, int d, double c,
                             double eps, const unsigned char *want, int bh, int inner_parallel) {
  if (bh < 0 || bh >= B * H) return 0;
  const size_t base = (size_t)bh * T * d;
  double *Qh = malloc(sizeof(double) * (size_t)T * d);
  double *Kh = malloc(sizeof(double) * (size_t)T * d);
  double *Vh = malloc(sizeof(double) * (size_t)T * d);
  double *D = calloc((size_t)T, sizeof(double));
  const size_t rows = inner_parallel ? ROW_BATCH : 1;
  double *p = malloc(sizeof(double) * rows * (size_t)T);
  double *sh = malloc(sizeof(double) * rows * (size_t)T);
  int rc = 0;
  if (!Qh || !Kh || !Vh || !D || !p || !sh) {
    rc = -2;
  } else {
    widen_block(Qh, q, dtype, base, (size_t)T * d);
    widen_block(Kh, k, dtype, base, (size_t)T * d);
    widen_block(Vh, v, dtype, base, (size_t)T * d);
    dilution_head(Qh, Kh, Vh, 0, T, d, c, eps, want, out + base,
                  lse ? lse + (size_t)bh * T : NULL, D, p, sh, inner_parallel);
    if (demand) memcpy(demand + (size_t)bh * T, D, sizeof(double) * (size_t)T);
  }
  free(Qh); free(Kh); free(Vh); free(D); free(p); free(sh);
  return rc;
}

/*
 * Dilution attention forward ([DIL] "The operator").
 * q,k,v: [B,H,T,d] in dtype.  out: [B,H,T,d] fp64 (rows not selected are left
 * untouched).  lse (optional): [B,H,T].  demand (optional): [B,H,T] fp64,
 * receives the final column totals sum_i p_ij.  rows/nrows: optional subset of
 * query rows whose output is formed; heads/nheads: optional subset of the
 * flattened (b*H+h) heads to process (others untouched).
 */
int oracle_dilution_fwd(const void *q, const void *k, const void *v, int dtype, double *out,
                        double *lse, double *demand, int B, int H, int T, int d, double tau,
                        double eps, const int *rows, int nrows, const int *heads, int nheads) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || d > 512) return -1;
  const double c = tau / sqrt((double)d);
  unsigned char *want = NULL;
  if (rows) {
    want = calloc((size_t)T, 1);
    if (!want) return -2;
    for (int r = 0; r < nrows; ++r)
      if (rows[r] >= 0 && rows[r] < T) want[rows[r]] = 1;
  }
  const int nh = heads ? nheads : B * H;
  /* Heads are independent: with enough of them each thread takes whole heads;
     otherwise heads run one after another and each row's sums are split
     across the threads. */
  const int outer = nh >= nthreads();
  int failed = 0;
  if (outer) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int hi = 0; hi < nh; ++hi)
      if (dilution_one_head(q, k, v, dtype, out, lse, demand, B, H, T, d, c, eps, want,
                            heads ? heads[hi] : hi, 0) != 0) {
#pragma omp atomic write
        failed = 1;
      }
  } else {
    for (int hi = 0; hi < nh; ++hi)
      if (dilution_one_head(q, k, v, dtype, out, lse, demand, B, H, T, d, c, eps, want,
                            heads ? heads[hi] : hi, 1) != 0)
        failed = 1;
  }
  free(want);
  return failed ? -2 : 0;
}

/*
 * A later chunk of a prefill, either operator.  The keys 0..Tk-1 of each
 * (b, h) sit in caches with room for Lcap rows per head; the chunk's Tq query
 * rows are the positions P = Tk-Tq .. Tk-1, and row i sees keys j <= i.
 *   tempered: o_i = sum_{j<=i} p_ij v_j                 ([FOCAL] eq. focal-const)
 *   dilution: committed_ij = Din_j + sum_{P<=i'<i} p_i'j  ([DIL] "The operator",
 *             with the demand the cached-decoding sentence keeps per key and
 *             head standing in for the rows before P), then the shares and
 *             the renormalised weights as for a whole prefill.
 * q: [B,H,Tq,d]; kc, vc: [B,H,Lcap,d]; out: [B,H,Tq,d] fp64; lse (optional):
 * [B,H,Tq]; demand (dilution, optional): [B,H,Lcap] fp64, in: Din (zero where
 * NULL), out: Din + the chunk's column totals on keys < Tk (others untouched).
 * mode: 0 tempered, 1 dilution.
 */
int oracle_prefill(const void *q, const void *kc, const void *vc, int dtype, double *out,
                   double *lse, double *demand, int B, int H, int Tq, int Tk, int Lcap, int d,
                   double tau, double eps, int mode) {
  if (B <= 0 || H <= 0 || Tq <= 0 || Tk < Tq || Lcap < Tk || d <= 0 || d > 512) return -1;
  const double c = tau / sqrt((double)d);
  const int P = Tk - Tq;
  /* Heads are independent: with enough of them each thread takes whole heads;
     otherwise heads run one after another and each row's sums are split
     across the threads (the same arithmetic, partial sums added in a fixed
     order), as in oracle_dilution_fwd. */
  const int inner = B * H < nthreads();
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) if (!inner)
  for (int bh = 0; bh < B * H; ++bh) {
    const size_t qbase = (size_t)bh * Tq * d, kbase = (size_t)bh * Lcap * d;
    double *Qh = malloc(sizeof(double) * (size_t)Tq * d);
    double *Kh = malloc(sizeof(double) * (size_t)Tk * d);
    double *Vh = malloc(sizeof(double) * (size_t)Tk * d);
    double *D = calloc((size_t)Tk, sizeof(double));
    const size_t rows = (mode == 1 && inner) ? ROW_BATCH : 1;
    double *p = malloc(sizeof(double) * rows * (size_t)Tk);
    double *sh = mode == 1 ? malloc(sizeof(double) * rows * (size_t)Tk) : NULL;
    if (!Qh || !Kh || !Vh || !D || !p || (mode == 1 && !sh)) {
#pragma omp atomic write
      failed = 1;
    } else {
      widen_block(Qh, q, dtype, qbase, (size_t)Tq * d);
      widen_block(Kh, kc, dtype, kbase, (size_t)Tk * d);
      widen_block(Vh, vc, dtype, kbase, (size_t)Tk * d);
      double *lse_h = lse ? lse + (size_t)bh * Tq : NULL;
      if (mode == 1) {
        if (demand) memcpy(D, demand + (size_t)bh * Lcap, sizeof(double) * (size_t)Tk);
        dilution_head(Qh, Kh, Vh, P, Tk, d, c, eps, NULL, out + qbase, lse_h, D, p, sh, inner);
        if (demand) memcpy(demand + (size_t)bh * Lcap, D, sizeof(double) * (size_t)Tk);
      } else {
        for (int i = P; i < Tk; ++i) {
          const double l = causal_bids(Qh + (size_t)(i - P) * d, Kh, i, d, c, p, inner);
          double *o = out + qbase + (size_t)(i - P) * d;
          for (int e = 0; e < d; ++e) o[e] = 0.0;
          for (int j = 0; j <= i; ++j)
            for (int e = 0; e < d; ++e) o[e] += p[j] * Vh[(size_t)j * d + e];
          if (lse_h) lse_h[i - P] = l;
        }
      }
    }
    free(Qh); free(Kh); free(Vh); free(D); free(p); free(sh);
  }
  return failed ? -2 : 0;
}

/* One (sequence, head) of a decode step; 0 on success. */
static int decode_one_pair(const void *q, const void *kc, const void *vc, int dtype, double *D,
                           double *out, int H, int Lcap, int d, const int *kv_len, double c,
                           double eps, int sh, int inner_parallel) {
  const int s = sh / H;
  const int L = kv_len ? kv_len[s] : Lcap;
  if (L <= 0 || L > Lcap || d > 512) return -1;
  double *Kh = malloc(sizeof(double) * (size_t)L * d);
  double *Vh = malloc(sizeof(double) * (size_t)L * d);
  double *p = malloc(sizeof(double) * (size_t)L);
  double qv[512];
  int rc = 0;
  if (!Kh || !Vh || !p) {
    rc = -2;
  } else {
    widen_block(qv, q, dtype, (size_t)sh * d, d);
    widen_block(Kh, kc, dtype, (size_t)sh * Lcap * d, (size_t)L * d);
    widen_block(Vh, vc, dtype, (size_t)sh * Lcap * d, (size_t)L * d);
    /* the new query sees every cached key: its bids are the causal bids of a
       row whose last visible key is L-1 */
    causal_bids(qv, Kh, L - 1, d, c, p, inner_parallel);
    double *Dh = D + (size_t)sh * Lcap;
    double r = 0.0, acc[512];
    for (int e = 0; e < d; ++e) acc[e] = 0.0;
    for (int j = 0; j < L; ++j) {
      if (p[j] > 0.0) {
        const double share = p[j] / (Dh[j] + p[j] + eps);
        r += share;
        for (int e = 0; e < d; ++e) acc[e] += share * Vh[(size_t)j * d + e];
      }
    }
    for (int e = 0; e < d; ++e) out[(size_t)sh * d + e] = acc[e] / r;
    for (int j = 0; j < L; ++j) Dh[j] += p[j];
  }
  free(Kh); free(Vh); free(p);
  return rc;
}

/*
 * One cached-decode step of dilution attention ([DIL], the sentence on cached
 * decoding: the ordinary key/value cache plus one running demand total per
 * key and head).  For each selected (sequence, head) with L visible keys:
 *   s_j = c <q, k_j>, p = softmax(s) over j < L,
 *   share_j = p_j / (D_j + p_j + eps) (0 where p_j = 0),
 *   o = sum_j share_j v_j / sum_j share_j,
 *   then D_j += p_j in place.
 * q: [S,H,d]; kc,vc: [S,H,Lcap,d] (all in dtype); D: [S,H,Lcap] fp64 in/out;
 * out: [S,H,d] fp64; kv_len: [S] or NULL (all Lcap); pairs/npairs: optional
 * subset of flattened (s*H+h) indices to process.
 */
int oracle_dilution_decode_step(const void *q, const void *kc, const void *vc, int dtype,
                                double *D, double *out, int S, int H, int Lcap, int d,
                                const int *kv_len, double tau, double eps, const int *pairs,
                                int npairs) {
  if (S <= 0 || H <= 0 || Lcap <= 0 || d <= 0) return -1;
  const double c = tau / sqrt((double)d);
  const int np = pairs ? npairs : S * H;
  const int outer = np >= nthreads();
  int failed = 0;
  if (outer) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int pi = 0; pi < np; ++pi) {
      const int sh = pairs ? pairs[pi] : pi;
      if (sh < 0 || sh >= S * H) continue;
      if (decode_one_pair(q, kc, vc, dtype, D, out, H, Lcap, d, kv_len, c, eps, sh, 0) != 0) {
#pragma omp atomic write
        failed = 1;
      }
    }
  } else {
    for (int pi = 0; pi < np; ++pi) {
      const int sh = pairs ? pairs[pi] : pi;
      if (sh < 0 || sh >= S * H) continue;
      if (decode_one_pair(q, kc, vc, dtype, D, out, H, Lcap, d, kv_len, c, eps, sh, 1) != 0)
        failed = 1;
    }
  }
  return failed ? -2 : 0;
}

/*
 * Exact gradients of both operators ([DIL] "Everything behind these charts":
 * the kernels train with exact gradients), by the chain rule through the
 * forward definitions above, one head at a time with every (i, j) matrix
 * materialised.  For dilution, with p the bids, C the committed demand,
 * D = C + p + eps, sigma = p / D, r_i = sum_j sigma_ij, a = sigma / r and
 * o_i = sum_j a_ij v_j, given dO:
 *   dV_j      = sum_i a_ij dO_i
 *   dA_ij     = <dO_i, v_j>,            delta_i = sum_j a_ij dA_ij
 *   dsigma_ij = (dA_ij - delta_i) / r_i
 *   sigma depends on p_ij directly and through D_ij, and C_i''j of every
 *   later row i'' > i contains p_ij, so with g_ij = dsigma_ij p_ij / D_ij^2
 *   dp_ij     = dsigma_ij / D_ij - sum_{i'' >= i} g_i''j
 *   (entries with p_ij = 0 -- masked or underflowed -- carry no gradient)
 *   dS_ij     = p_ij (dp_ij - sum_j' p_ij' dp_ij')     (softmax)
 *   dQ_i = c sum_j dS_ij k_j,  dK_j = c sum_i dS_ij q_i,  c = tau / sqrt(d).
 * Tempered is the same with a = p, so dp_ij = dA_ij.
 *
 * With logits tau <q_i, k_j> / sqrt(d) the multiplier's own gradient is
 *   dL/dtau = sum_ij dS_ij <q_i, k_j> / sqrt(d)
 * (the per-head temperature a learned-temperature layer feeds in, [FOCAL]
 * sec. 2.2 eq. learn-temp).
 *
 * q,k,v,dout: [B,H,T,d] in dtype; dq,dk,dv: [B,H,T,d] fp64.  rsum (optional,
 * dilution): [B,H,T] fp64, the row sums r_i.  dtau (optional): [B,H] fp64.
 * tau_bh (optional): [B,H] per-head multipliers in place of tau.  mode: 0
 * tempered, 1 dilution.
 */
static int bwd_one_head(const void *q, const void *k, const void *v, const void *dout, int dtype,
                        double *dq, double *dk, double *dv, double *rsum, double *dtau, int T,
                        int d, double c, double eps, int mode, int bh) {
  const size_t base = (size_t)bh * T * d, TT = (size_t)T * T;
  double *Q = malloc(sizeof(double) * (size_t)T * d), *K = malloc(sizeof(double) * (size_t)T * d);
  double *V = malloc(sizeof(double) * (size_t)T * d), *dO = malloc(sizeof(double) * (size_t)T * d);
  double *P = calloc(TT, sizeof(double)), *Dn = calloc(TT, sizeof(double));
  double *A = calloc(TT, sizeof(double)), *dP = calloc(TT, sizeof(double));
  double *r = calloc((size_t)T, sizeof(double)), *col = calloc((size_t)T, sizeof(double));
  int rc = 0;
  if (!Q || !K || !V || !dO || !P || !Dn || !A || !dP || !r || !col) {
    rc = -2;
    goto done;
  }
  widen_block(Q, q, dtype, base, (size_t)T * d);
  widen_block(K, k, dtype, base, (size_t)T * d);
  widen_block(V, v, dtype, base, (size_t)T * d);
  widen_block(dO, dout, dtype, base, (size_t)T * d);
  /* forward: bids, committed demand, shares, weights A */
  for (int i = 0; i < T; ++i) causal_bids(Q + (size_t)i * d, K, i, d, c, P + (size_t)i * T, 0);
  for (int i = 0; i < T; ++i) {
    double *Pi = P + (size_t)i * T, *Ai = A + (size_t)i * T, *Di = Dn + (size_t)i * T;
    if (mode == 0) {
      for (int j = 0; j <= i; ++j) Ai[j] = Pi[j];
      continue;
    }
    for (int j = 0; j <= i; ++j) {
      Di[j] = col[j] + Pi[j] + eps;          /* col[j] = committed C_ij */
      Ai[j] = Pi[j] > 0.0 ? Pi[j] / Di[j] : 0.0;
      r[i] += Ai[j];
    }
    for (int j = 0; j <= i; ++j) Ai[j] /= r[i];
    for (int j = 0; j <= i; ++j) col[j] += Pi[j];
  }
  if (rsum && mode == 1) memcpy(rsum + (size_t)bh * T, r, sizeof(double) * (size_t)T);
  /* dA and the gradient with respect to the bids */
  for (int i = 0; i < T; ++i) {
    const double *Ai = A + (size_t)i * T;
    double *dPi = dP + (size_t)i * T;
    double delta = 0.0;
    for (int j = 0; j <= i; ++j) {
      dPi[j] = dot(dO + (size_t)i * d, V + (size_t)j * d, d);   /* dA_ij for now */
      delta += Ai[j] * dPi[j];
    }
    if (mode == 1)
      for (int j = 0; j <= i; ++j) dPi[j] = (dPi[j] - delta) / r[i];   /* dsigma_ij */
  }
  if (mode == 1) {
    /* dp_ij = dsigma_ij / D_ij - (inclusive suffix sum of g down column j) */
    for (int j = 0; j < T; ++j) col[j] = 0.0;
    for (int i = T - 1; i >= 0; --i) {
      const double *Pi = P + (size_t)i * T, *Di = Dn + (size_t)i * T;
      double *dPi = dP + (size_t)i * T;
      for (int j = 0; j <= i; ++j) {
        if (Pi[j] > 0.0) {
          col[j] += dPi[j] * Pi[j] / (Di[j] * Di[j]);
          dPi[j] = dPi[j] / Di[j] - col[j];
        } else {
          dPi[j] = 0.0;
        }
      }
    }
  }
  /* softmax: dS = p (dp - sum_j p dp), kept in dP */
  for (int i = 0; i < T; ++i) {
    const double *Pi = P + (size_t)i * T;
    double *dPi = dP + (size_t)i * T;
    double rho = 0.0;
    for (int j = 0; j <= i; ++j) rho += Pi[j] * dPi[j];
    for (int j = 0; j <= i; ++j) dPi[j] = Pi[j] * (dPi[j] - rho);
  }
  /* the multiplier: logits are tau <q_i, k_j> / sqrt(d), so
     dL/dtau = sum_ij dS_ij <q_i, k_j> / sqrt(d) */
  if (dtau) {
    double acc = 0.0;
    for (int i = 0; i < T; ++i)
      for (int j = 0; j <= i; ++j)
        acc += dP[(size_t)i * T + j] * dot(Q + (size_t)i * d, K + (size_t)j * d, d);
    dtau[bh] = acc / sqrt((double)d);
  }
  for (int i = 0; i < T; ++i) {
    const double *Si = dP + (size_t)i * T;
    double *dqi = dq + base + (size_t)i * d;
    for (int e = 0; e < d; ++e) dqi[e] = 0.0;
    for (int j = 0; j <= i; ++j)
      for (int e = 0; e < d; ++e) dqi[e] += c * Si[j] * K[(size_t)j * d + e];
  }
  for (int j = 0; j < T; ++j) {
    double *dkj = dk + base + (size_t)j * d, *dvj = dv + base + (size_t)j * d;
    for (int e = 0; e < d; ++e) dkj[e] = dvj[e] = 0.0;
    for (int i = j; i < T; ++i) {
      const double s = dP[(size_t)i * T + j], a = A[(size_t)i * T + j];
      for (int e = 0; e < d; ++e) {
        dkj[e] += c * s * Q[(size_t)i * d + e];
        dvj[e] += a * dO[(size_t)i * d + e];
      }
    }
  }
done:
  free(Q); free(K); free(V); free(dO); free(P); free(Dn); free(A); free(dP); free(r); free(col);
  return rc;
}

int oracle_attn_bwd(const void *q, const void *k, const void *v, const void *dout, int dtype,
                    double *dq, double *dk, double *dv, double *rsum, double *dtau, int B, int H,
                    int T, int d, double tau, const double *tau_bh, double eps, int mode) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || (mode != 0 && mode != 1)) return -1;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh)
    if (bwd_one_head(q, k, v, dout, dtype, dq, dk, dv, rsum, dtau, T, d,
                     (tau_bh ? tau_bh[bh] : tau) / sqrt((double)d), eps, mode, bh) != 0) {
#pragma omp atomic write
      failed = 1;
    }
  return failed ? -2 : 0;
}

/*
 * Rotary position embedding, applied to Q and K before the scores ([YARN]
 * code cell In[16]: apply_yarn_rope rotates each token's query and key at its
 * position with the per-pair frequencies times YaRN's gamma, then the scores
 * are Q_rot K_rot^T / sqrt(d) times sqrt(t)).  The page leaves apply_rope,
 * the pair layout and gamma undefined; read here as: the caller passes the
 * frequencies with gamma already applied, dimension pair m is (2m, 2m+1), and
 * the pair turns counter-clockwise by the angle
 *   theta = (pos0 + t) * freq[m]
 * for row t:  (x, y) -> (x cos theta - y sin theta, x sin theta + y cos theta).
 * x: [B,H,T,d] in dtype; out: [B,H,T,d] fp64; freq: [d/2] fp64; d even.
 */
/*
 * x rounded to the nearest bfloat16 value (8 significant bits, the exponent
 * range of binary32), ties to the even significand.  Used where a method
 * stores an intermediate row in bf16.  Finite inputs within binary32's normal
 * range only (the rows rotated here); others are returned unchanged.
 */
static double round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  const double m = frexp(x, &e);          /* x = m 2^e, 0.5 <= |m| < 1 */
  if (e < -125 || e > 128) return x;
  const double scaled = ldexp(m, 8);      /* 8 significant bits left of the point */
  double r = floor(scaled);
  const double frac = scaled - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  return ldexp(r, e - 8);
}

int oracle_rope(const void *x, int dtype, double *out, int B, int H, int T, int d,
                const double *freq, long pos0, int round_to_bf16) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0 || (d & 1)) return -1;
  const long rows = (long)B * H * T;
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const long t = r % T;
    for (int m = 0; m < d / 2; ++m) {
      const double theta = (double)(pos0 + t) * freq[m];
      const double c = cos(theta), sn = sin(theta);
      const double a = widen(x, dtype, (size_t)r * d + 2 * m);
      const double b = widen(x, dtype, (size_t)r * d + 2 * m + 1);
      out[(size_t)r * d + 2 * m] = a * c - b * sn;
      out[(size_t)r * d + 2 * m + 1] = a * sn + b * c;
    }
    if (round_to_bf16)
      for (int e = 0; e < d; ++e) out[(size_t)r * d + e] = round_bf16(out[(size_t)r * d + e]);
  }
  return 0;
}

int oracle_num_threads(void) { return nthreads(); }
