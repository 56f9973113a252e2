// decode.hip -- cached-decode step of dilution attention for gfx950.
//
// "DilutionAttention v0.1.0 - results", "The operator": cached decoding needs
// the ordinary key/value cache plus one running demand total per key and
// head.  For one new query per (sequence, head) over L cached keys:
//   s_j = tau <q,k_j> / sqrt(d),  p = softmax(s),
//   share_j = p_j / (D_j + p_j + eps),  out = sum_j share_j v_j / sum_j share_j,
//   then D_j += p_j in place (the bid, not the share).
//
// The step streams K once and V once, so it is bound by HBM bandwidth.  For
// caches of up to 32768 keys one workgroup per (sequence, head) does the whole
// step with the scores in LDS (dec_fused).  Longer caches split the keys of a
// (sequence, head) into chunks, one workgroup each:
//   dec_scores   : s_j (kept in fp32 scratch) and a partial (max, sum exp)
//   dec_share_v  : global log-sum-exp from the partials, p_j, share_j, the
//                  in-place demand update, and partial (sum share v, sum share)
//   dec_combine  : out = sum of partial numerators / sum of partial row sums
// Loads are 16 bytes per lane; d/8 lanes cover one key row (128 bytes at
// d = 64, 256 at d = 128), so one wave instruction reads 1 KB of consecutive
// rows, fully coalesced, and d/8 such loads bring 64 keys per wave.  The
// caches are read exactly once per step, so they stream with non-temporal
// loads (measured on MI355X: ~7.1 TB/s against ~6.3 TB/s for ordinary loads).
#include "attn_common.hpp"
#include "launch.hpp"

#include <float.h>

namespace attn {

constexpr int kDecThreads = 256;

__device__ __forceinline__ int visible_keys(const int32_t *kv_len, int s, int Lcap) {
  if (!kv_len) return Lcap;
  const int L = kv_len[s];
  return L < 1 ? 1 : (L > Lcap ? Lcap : L);
}

// <k, q> over one lane's 8 dimensions with packed bf16 dot products (fp32
// accumulation).  Each 32-bit word is copied to a scalar before the bit cast:
// a bit cast applied directly to a vector element was lowered as element 0.
__device__ __forceinline__ float dot8_bf16(const u32x4 &kw, const u32x4 &qw) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t kx = kw[i], qx = qw[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kx),
                                          __builtin_bit_cast(bf16x2_t, qx), acc, false);
  }
  return acc;
}

// Lane geometry for head dimension D: kLanes lanes (one 16-byte chunk each)
// per key row, kRows rows per wave instruction.
template <int D>
struct DecGeom {
  static constexpr int kLanes = D / 8;
  static constexpr int kRows = 64 / kLanes;
};

template <int D>
__global__ void __launch_bounds__(kDecThreads) dec_scores(DecodeArgs a) {
  using G = DecGeom<D>;
  __shared__ float sm[kDecThreads / 64], sl[kDecThreads / 64];
  const int split = blockIdx.x % a.splits;
  const int sh = blockIdx.x / a.splits;
  const int seq = sh / a.H;
  const int L = visible_keys(a.kv_len, seq, a.Lcap);
  const int c0 = split * a.chunk, c1 = min(c0 + a.chunk, L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane / G::kLanes, dc = lane % G::kLanes;
  const float c2 = a.tau_sh ? a.tau_sh[sh] * a.c2 : a.c2;

  const u32x4 qw = *reinterpret_cast<const u32x4 *>(
      reinterpret_cast<const __bf16 *>(a.q) + (size_t)sh * D + 8 * dc);
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.kc) + (size_t)sh * a.Lcap * D;
  float *S = a.scores + (size_t)sh * a.Lcap;
  float m = -INFINITY, l = 0.0f;

  // Each wave-iteration covers 64 consecutive keys: load u brings keys
  // base + kRows u + slot (kLanes lanes each).  After the dot products every
  // lane keeps the score of key base + kRows dc + slot, so the 64 lanes hold
  // 64 distinct keys.
  constexpr int kU = G::kLanes;            // loads in flight per lane
  constexpr int kWaveKeys = G::kRows * kU;  // = 64
  for (int base = c0 + w * kWaveKeys; base < c1; base += (kDecThreads / 64) * kWaveKeys) {
    u32x4 kw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = base + G::kRows * u + slot;
      kw[u] = (j < c1) ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4 *>(K + (size_t)j * D + 8 * dc))
                       : u32x4{0u, 0u, 0u, 0u};
    }
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float s = dot8_bf16(kw[u], qw);
#pragma unroll
      for (int off = 1; off < G::kLanes; off <<= 1) s += __shfl_xor(s, off, G::kLanes);
      mine = (dc == u) ? s : mine;
    }
    const int j = base + G::kRows * dc + slot;
    if (j < c1) {
      const float x = mine * c2;   // log2-domain logit
      S[j] = x;
      const float m_new = fmaxf(m, x);
      l = l * fast_exp2(m - m_new) + fast_exp2(x - m_new);
      m = m_new;
    }
  }
  // combine (m, l) over the wave, then over the waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
    const float mn = fmaxf(m, mo);
    l = (mn == -INFINITY) ? 0.0f : l * fast_exp2(m - mn) + lo * fast_exp2(mo - mn);
    m = mn;
  }
  if (lane == 0) { sm[w] = m; sl[w] = l; }
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY, Ls = 0.0f;
    for (int i = 0; i < kDecThreads / 64; ++i) {
      const float mn = fmaxf(M, sm[i]);
      Ls = (mn == -INFINITY) ? 0.0f : Ls * fast_exp2(M - mn) + sl[i] * fast_exp2(sm[i] - mn);
      M = mn;
    }
    a.part_ml[2 * ((size_t)sh * a.splits + split)] = M;
    a.part_ml[2 * ((size_t)sh * a.splits + split) + 1] = Ls;
  }
}

template <int D>
__global__ void __launch_bounds__(kDecThreads) dec_share_v(DecodeArgs a) {
  using G = DecGeom<D>;
  __shared__ float sShare[kDecThreads / 64][64];
  __shared__ float sO[kDecThreads / 64][D + 1];
  const int split = blockIdx.x % a.splits;
  const int sh = blockIdx.x / a.splits;
  const int seq = sh / a.H;
  const int L = visible_keys(a.kv_len, seq, a.Lcap);
  const int c0 = split * a.chunk, c1 = min(c0 + a.chunk, L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane / G::kLanes, dc = lane % G::kLanes;

  // log-sum-exp of this query's scores over all chunks (fixed order)
  float M = -INFINITY, Ls = 0.0f;
  for (int i = 0; i < a.splits; ++i) {
    const float mi = a.part_ml[2 * ((size_t)sh * a.splits + i)];
    const float li = a.part_ml[2 * ((size_t)sh * a.splits + i) + 1];
    const float mn = fmaxf(M, mi);
    Ls = (mn == -INFINITY) ? 0.0f : Ls * fast_exp2(M - mn) + li * fast_exp2(mi - mn);
    M = mn;
  }
  const float lse2 = M + __builtin_log2f(Ls);
  const float eps_floor = fmaxf(a.eps, FLT_MIN);

  const __bf16 *Vc = reinterpret_cast<const __bf16 *>(a.vc) + (size_t)sh * a.Lcap * D;
  const float *S = a.scores + (size_t)sh * a.Lcap;
  float *Dm = a.demand + (size_t)sh * a.Lcap;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float rsum = 0.0f;

  for (int base = c0 + 64 * w; base < c1; base += 64 * (kDecThreads / 64)) {
    // one key per lane: bid, share and the demand update
    const int j = base + lane;
    float share = 0.0f;
    if (j < c1) {
      const float p = fast_exp2(S[j] - lse2);
      const float dj = Dm[j];
      share = p * fast_rcp(fmaxf(dj + p + a.eps, eps_floor));
      Dm[j] = dj + p;
    }
    rsum += share;
    sShare[w][lane] = share;
    // kLanes lanes per key row for the values
    u32x4 vw[G::kLanes];
#pragma unroll
    for (int u = 0; u < G::kLanes; ++u) {
      const int jj = base + G::kRows * u + slot;
      vw[u] = (jj < c1) ? __builtin_nontemporal_load(
                              reinterpret_cast<const u32x4 *>(Vc + (size_t)jj * D + 8 * dc))
                        : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < G::kLanes; ++u) {
      const float sj = sShare[w][G::kRows * u + slot];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(sj, bf16_lo(vw[u][i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(sj, bf16_hi(vw[u][i]), acc[2 * i + 1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // reduce over the key slots of the wave (lanes with equal dc), then waves
#pragma unroll
  for (int off = G::kLanes; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) rsum += __shfl_xor(rsum, off, 64);
  if (lane < G::kLanes) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sO[w][8 * dc + e] = acc[e];
  }
  if (lane == 0) sO[w][D] = rsum;
  __syncthreads();
  if (tid <= D) {
    float v = 0.0f;
    for (int i = 0; i < kDecThreads / 64; ++i) v += sO[i][tid];
    a.part_o[((size_t)sh * a.splits + split) * (D + 1) + tid] = v;
  }
}

// One thread per output element; 128 threads cover 128/D (sequence, head) pairs.
template <int D>
__global__ void __launch_bounds__(128) dec_combine(DecodeArgs a) {
  const int sh = blockIdx.x * (128 / D) + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (sh >= a.S * a.H) return;
  float num = 0.0f, den = 0.0f;
  for (int i = 0; i < a.splits; ++i) {
    const float *po = a.part_o + ((size_t)sh * a.splits + i) * (D + 1);
    num += po[d];
    den += po[D];
  }
  reinterpret_cast<__bf16 *>(a.out)[(size_t)sh * D + d] = (__bf16)(num / den);
}

// ------------------------------------------------------------ fused form
//
// Caches of up to kFusedKeys keys: one workgroup per (sequence, head) keeps
// every score in LDS, so K and V are each streamed once and
// nothing else touches HBM but the demand.  Three phases, separated by
// workgroup barriers: scores (and their maximum) from K; the log-sum-exp from
// the scores in LDS; then bids, shares, the demand update and share @ V from
// V.  Reductions run in a fixed order.

constexpr int kFusedKeys = 32768;

// 16 waves at d = 64; 8 at d = 128, whose 16 loads in flight per lane need
// the larger register budget.  Either way 128 KB of loads are in flight per
// workgroup.
template <int D>
struct FusedGeom {
  static constexpr int kThreads = D > 64 ? 512 : 1024;
  static constexpr int kWaves = kThreads / 64;
};

template <int D>
__global__ void __launch_bounds__(FusedGeom<D>::kThreads) dec_fused(DecodeArgs a) {
  using G = DecGeom<D>;
  constexpr int kFusedThreads = FusedGeom<D>::kThreads, kFusedWaves = FusedGeom<D>::kWaves;
  __shared__ float sS[kFusedKeys];
  __shared__ float sRed[kFusedWaves];
  __shared__ float sShare[kFusedWaves][64];
  const int sh = blockIdx.x;
  const int seq = sh / a.H;
  const int L = visible_keys(a.kv_len, seq, a.Lcap);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int slot = lane / G::kLanes, dc = lane % G::kLanes;
  const float c2 = a.tau_sh ? a.tau_sh[sh] * a.c2 : a.c2;
  const u32x4 qw = *reinterpret_cast<const u32x4 *>(
      reinterpret_cast<const __bf16 *>(a.q) + (size_t)sh * D + 8 * dc);
  const __bf16 *K = reinterpret_cast<const __bf16 *>(a.kc) + (size_t)sh * a.Lcap * D;
  const __bf16 *Vc = reinterpret_cast<const __bf16 *>(a.vc) + (size_t)sh * a.Lcap * D;
  float *Dm = a.demand + (size_t)sh * a.Lcap;
  constexpr int kU = G::kLanes;
  constexpr int kStride = 64 * kFusedWaves;   // keys per workgroup iteration

  // phase 1: scores (log2 domain) into LDS and their maximum
  float m = -INFINITY;
  for (int base = 64 * w; base < L; base += kStride) {
    u32x4 kw[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = base + G::kRows * u + slot;
      kw[u] = (j < L) ? __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4 *>(K + (size_t)j * D + 8 * dc))
                      : u32x4{0u, 0u, 0u, 0u};
    }
    float mine = 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float sc = dot8_bf16(kw[u], qw);
#pragma unroll
      for (int off = 1; off < G::kLanes; off <<= 1) sc += __shfl_xor(sc, off, G::kLanes);
      mine = (dc == u) ? sc : mine;
    }
    const int j = base + G::kRows * dc + slot;
    if (j < L) {
      const float x = mine * c2;
      sS[j] = x;
      m = fmaxf(m, x);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) sRed[w] = m;
  __syncthreads();
  float M = sRed[0];
#pragma unroll
  for (int i = 1; i < kFusedWaves; ++i) M = fmaxf(M, sRed[i]);
  __syncthreads();   // every wave has read sRed before it is reused

  // phase 2: sum of exp2(s - M) over the scores in LDS
  float l = 0.0f;
  for (int j = tid; j < L; j += kFusedThreads) l += fast_exp2(sS[j] - M);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
  if (lane == 0) sRed[w] = l;
  __syncthreads();
  float Ls = 0.0f;
#pragma unroll
  for (int i = 0; i < kFusedWaves; ++i) Ls += sRed[i];
  const float lse2 = M + __builtin_log2f(Ls);
  const float eps_floor = fmaxf(a.eps, FLT_MIN);

  // phase 3: bids, shares and the demand update (one lane per key), then
  // share @ V with kLanes lanes per value row
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float rsum = 0.0f;
  for (int base = 64 * w; base < L; base += kStride) {
    const int j = base + lane;
    float share = 0.0f;
    if (j < L) {
      const float p = fast_exp2(sS[j] - lse2);
      const float dj = Dm[j];
      share = p * fast_rcp(fmaxf(dj + p + a.eps, eps_floor));
      Dm[j] = dj + p;
    }
    rsum += share;
    sShare[w][lane] = share;
    u32x4 vw[G::kLanes];
#pragma unroll
    for (int u = 0; u < G::kLanes; ++u) {
      const int jj = base + G::kRows * u + slot;
      vw[u] = (jj < L) ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4 *>(Vc + (size_t)jj * D + 8 * dc))
                       : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < G::kLanes; ++u) {
      const float sj = sShare[w][G::kRows * u + slot];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(sj, bf16_lo(vw[u][i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(sj, bf16_hi(vw[u][i]), acc[2 * i + 1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int off = G::kLanes; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) rsum += __shfl_xor(rsum, off, 64);
  __syncthreads();   // the scores are no longer needed: sS holds the partials
  float *sO = sS;    // [kFusedWaves][D + 1]
  if (lane < G::kLanes) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sO[w * (D + 1) + 8 * dc + e] = acc[e];
  }
  if (lane == 0) sO[w * (D + 1) + D] = rsum;
  __syncthreads();
  if (tid < D) {
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int i = 0; i < kFusedWaves; ++i) {
      num += sO[i * (D + 1) + tid];
      den += sO[i * (D + 1) + D];
    }
    reinterpret_cast<__bf16 *>(a.out)[(size_t)sh * D + tid] = (__bf16)(num / den);
  }
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t s) {
  if (a.Lcap <= kFusedKeys) {
    hipLaunchKernelGGL(dec_fused<D>, dim3((unsigned)(a.S * a.H)), dim3(FusedGeom<D>::kThreads), 0,
                       s, a);
    return hipGetLastError();
  }
  const unsigned nwg = (unsigned)(a.S * a.H * a.splits);
  hipLaunchKernelGGL(dec_scores<D>, dim3(nwg), dim3(kDecThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dec_share_v<D>, dim3(nwg), dim3(kDecThreads), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int kPer = 128 / D;
  hipLaunchKernelGGL(dec_combine<D>, dim3((unsigned)((a.S * a.H + kPer - 1) / kPer)), dim3(128), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  return a.D == 128 ? launch_decode_d<128>(a, s) : launch_decode_d<64>(a, s);
}

}  // namespace attn
