// Router: logits = X W_g (+ offset), scores, top-k and gates.
//
// LLM Internals 14.2.1 steps 2-3 and the AI Knowledge Map "MoE" router steps:
// a linear scoring layer, an fp32 softmax over all E experts (or DeepSeek-V3's
// per-cell sigmoid affinity with a selection-only bias, eq. 16 as restated in
// LLM Internals 14.2.3), hard top-k, then renormalisation inside the chosen
// set.  The study note's pitfalls section fixes the router softmax to fp32.
#include "common.h"
#include "kernels.h"

namespace moe {

// --------------------------------------------------------------------------
// Logits GEMM: part[z][t][e] = sum_{i in slice z} X[t][i] * Wg[e][i].
// One wave owns a 16-token x 16-expert MFMA block and walks its d-slice,
// reading both operands straight from global memory (each lane pulls 16 B of
// a row; Wg stays in L2).  The four waves of a block cover wpt = min(4,
// ceil(E/16)) expert blocks of 4/wpt token groups, so small E still keeps
// every wave busy; split-K slices add parallelism.
template <typename T>
__global__ __launch_bounds__(256) void k_router_logits(
    const T* __restrict__ X, const T* __restrict__ Wg, float* __restrict__ part,
    int T_, int d, int E, int dchunk, int wpt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.y * 16 * wpt + (wave % wpt) * 16;
  if (e0 >= E) return;                       // no block-level sync below
  const int t0 = (blockIdx.x * (4 / wpt) + wave / wpt) * 16;
  const int z = blockIdx.z;
  const int kb = z * dchunk, ke = min(d, kb + dchunk);
  const int row = lane & 15, grp = lane >> 4;       // 4 lane groups along K
  const int tok = t0 + row, ex = e0 + row;
  const bool tv = tok < T_, ev = ex < E;
  const T* xa = X + (size_t)(tv ? tok : 0) * d;
  const T* wb = Wg + (size_t)(ev ? ex : 0) * d;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int EPL = 16 / sizeof(T);              // elements per 16-B lane load
  constexpr int KSTEP = EPL * 4;                   // K covered by one wave step
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int k = kb; k < ke; k += KSTEP) {
    const int kk = k + grp * EPL;
    u32x4 a = tv ? *(const u32x4*)(xa + kk) : zero;
    u32x4 b = ev ? *(const u32x4*)(wb + kk) : zero;
    if constexpr (sizeof(T) == 2) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, b),
                                                     acc, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]),
                                                   acc, 0, 0, 0);
    }
  }
  // C layout (16x16): lane holds column (lane & 15), rows 4*(lane>>4) + r.
  const int col = e0 + (lane & 15);
  if (col < E) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + grp * 4 + r;
      if (t < T_) part[((size_t)z * T_ + t) * E + col] = acc[r];
    }
  }
}

// --------------------------------------------------------------------------
// Select: one wave per token.  Lane L holds experts L, L+64, L+128, L+192.
// Key descending, lower id on ties; a NaN key ranks below every number,
// -inf included (the order of a stable ascending sort of -key).  kNoKey, a
// NaN, with id kNoId starts every arg-max: any candidate beats it, so a
// round always ends on a real expert while one is left.
__device__ __forceinline__ bool better(double ka, int ia, double kb, int ib) {
  const bool na = ka != ka, nb = kb != kb;
  if (na || nb) return na == nb ? ia < ib : nb;
  return ka > kb || (ka == kb && ia < ib);
}
#define kNoKey __builtin_nan("")
constexpr int kNoId = 0x7fffffff;

// Wave arg-max of (key, id) over this lane's candidates (already reduced to
// one per lane): the best key, lower id on ties.
__device__ __forceinline__ void wave_best(double& bk, int& bi) {
  for (int o = 32; o > 0; o >>= 1) {
    const double ok_ = __shfl_xor(bk, o);
    const int oi = __shfl_xor(bi, o);
    if (better(ok_, oi, bk, bi)) { bk = ok_; bi = oi; }
  }
}

// Group-limited routing (LLM Internals 14.2.3, node-limited routing: groups
// of E / n_group consecutive experts stand in for nodes).  A group's score is
// the sum of its gk = k / topk_group (>= 1) highest affinities, largest
// first; the topk_group best groups (lower id on ties) stay eligible, every
// other expert's key becomes -inf.  aff: the softmax numerator exp(l - max)
// (same order as the probability) or the sigmoid s, in fp64.
template <int NE>
__device__ __forceinline__ void limit_groups(double (&key)[NE], const double (&aff)[NE], int E,
                                             int k, int n_group, int topk_group, int lane) {
  const int gs = E / n_group;
  int gk = k / topk_group;
  gk = gk < 1 ? 1 : (gk > gs ? gs : gk);
  double gscore = -INFINITY;                 // lane g holds group g's score
  for (int g = 0; g < n_group; ++g) {
    uint32_t taken = 0;
    double acc = 0.0;
    for (int r = 0; r < gk; ++r) {
      double bk = kNoKey;
      int bi = kNoId;
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int e = lane + 64 * i;
        if (e < E && e / gs == g && !((taken >> i) & 1u) && better(aff[i], e, bk, bi)) {
          bk = aff[i];
          bi = e;
        }
      }
      wave_best(bk, bi);
      if (lane == (bi & 63)) taken |= 1u << (bi >> 6);
      acc += bk;
    }
    if (lane == g) gscore = acc;
  }
  uint64_t chosen = 0;
  for (int r = 0; r < topk_group; ++r) {
    const bool cand = lane < n_group && !((chosen >> lane) & 1ull);
    double bk = cand ? gscore : kNoKey;
    int bi = cand ? lane : kNoId;
    wave_best(bk, bi);
    chosen |= 1ull << bi;
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    if (e < E && !((chosen >> (e / gs)) & 1ull)) key[i] = -INFINITY;
  }
}

// Logits of token t for experts lane + 64 i: the split-K partials summed
// in split order z = 0, 1, ... (then the offset), -inf for experts past E or
// a token past T.  Up to 32 partial logits per lane are loaded at once.
template <int NE>
__device__ __forceinline__ void gather_logits(float (&l)[NE], const float* __restrict__ part,
                                              int nsplit, int T_, int E, int t, bool tok_ok,
                                              int lane, const float* __restrict__ offset,
                                              float* __restrict__ logits) {
  bool ok[NE];
  float v[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    ok[i] = tok_ok && lane + 64 * i < E;
    v[i] = 0.f;
  }
  const size_t zs = (size_t)T_ * E;
  const float* base = part + (size_t)t * E + lane;
  // U splits' loads in flight at once (U * NE <= 32 registers), summed in
  // split order; the last batch is predicated, so a split count that is
  // not a multiple of U costs no extra round trips
  constexpr int U = NE >= 4 ? 8 : 16;
  for (int z = 0; z < nsplit; z += U) {
    float q[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NE; ++i)
        q[u][i] = (ok[i] && z + u < nsplit) ? base[(size_t)(z + u) * zs + 64 * i] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (z + u < nsplit)
#pragma unroll
        for (int i = 0; i < NE; ++i) v[i] += q[u][i];
  }
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const int e = lane + 64 * i;
    if (ok[i]) {
      if (offset) v[i] += offset[e];
      if (logits) logits[(size_t)t * E + e] = v[i];
    }
    l[i] = ok[i] ? v[i] : -INFINITY;
  }
}

// One token's scores, top-k and gates, by one wave (lane L holds experts
// L, L + 64, ...): l are the logits (-inf past E or past T), p receives the
// full-row probability (softmax p, or the sigmoid s) for the balance and
// entropy statistics; ids, gates and backups are written for a real token.
template <int NE>
__device__ __forceinline__ void route_token(const float (&l)[NE], float (&p)[NE], int t,
                                            bool tok_ok, int lane, int E,
                                            const float* __restrict__ bias, int score, int k,
                                            int renorm, int n_group, int topk_group,
                                            int32_t* __restrict__ ids, float* __restrict__ wts,
                                            int nb, int32_t* __restrict__ backup) {
  double key[NE], s64[NE];
  double aff[NE];                        // group scores' affinities (fp64)
  if (score == MOE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NE; ++i) m = fmaxf(m, l[i]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
#pragma unroll
    for (int i = 0; i < NE; ++i)
      aff[i] = (n_group > 1 && tok_ok && lane + 64 * i < E) ? exp((double)l[i] - (double)m) : 0.0;
    float zs = 0.f;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      p[i] = (e < E && tok_ok) ? expf(l[i] - m) : 0.f;
      zs += p[i];
    }
    for (int o = 32; o > 0; o >>= 1) zs += __shfl_xor(zs, o);
    const float inv = 1.f / zs;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      p[i] *= inv;                       // full-row softmax probability
      key[i] = (double)l[i];             // selection on the logit
      s64[i] = (double)p[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      const bool ok = (e < E && tok_ok);
      const double s = ok ? 1.0 / (1.0 + exp(-(double)l[i])) : 0.0;
      s64[i] = s;
      aff[i] = s;
      p[i] = (float)s;
      key[i] = ok ? s + (bias ? (double)bias[e] : 0.0) : -INFINITY;
    }
  }
  if (n_group > 1) limit_groups<NE>(key, aff, E, k, n_group, topk_group, lane);
  // Iterative wave arg-max, k rounds (plus nb backup rounds: the next
  // choices in the same key order, -1 for an ineligible expert); lane j
  // keeps the j-th winner.
  uint32_t taken = 0;
  int my_id = 0;
  double my_val = 0.0, tot = 0.0;
  for (int j = 0; j < k + nb; ++j) {
    double bk = kNoKey;
    int bi = kNoId;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && better(key[i], e, bk, bi)) { bk = key[i]; bi = e; }
    }
    wave_best(bk, bi);
    // owner lane marks the winner; every lane fetches its score
    const int oi = bi >> 6, ol = bi & 63;
    double mine = 0.0;
#pragma unroll
    for (int i = 0; i < NE; ++i) if (i == oi) mine = s64[i];
    const double val = __shfl(mine, ol);
    if (lane == ol) taken |= 1u << oi;
    // a top-k pick is always the expert found (k <= E untaken experts
    // exist), even when its key is -inf or NaN; a backup is -1 unless its
    // key is above -inf (an expert outside the chosen groups is not one)
    if (lane == j) { my_id = (j < k || bk > -INFINITY) ? bi : -1; my_val = val; }
    if (j < k) tot += val;                       // fixed order j = 0..k-1
  }
  if (tok_ok && lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = (float)(renorm ? my_val / tot : my_val);
  }
  if (tok_ok && lane >= k && lane < k + nb) backup[(size_t)t * nb + lane - k] = my_id;
}

// Routing entropy of one token, -sum q ln q in fp32 with q = p (softmax) or
// s / sum(s) (sigmoid); wave-reduced, every lane holds it.
template <int NE>
__device__ __forceinline__ float token_entropy(const float (&p)[NE], int score) {
  float zs = 0.f;
  if (score != MOE_SOFTMAX) {
#pragma unroll
    for (int i = 0; i < NE; ++i) zs += p[i];
    for (int o = 32; o > 0; o >>= 1) zs += __shfl_xor(zs, o);
  }
  float h = 0.f;
#pragma unroll
  for (int i = 0; i < NE; ++i) {
    const float q = score == MOE_SOFTMAX ? p[i] : (zs > 0.f ? p[i] / zs : 0.f);
    if (q > 0.f) h -= q * logf(q);
  }
  for (int o = 32; o > 0; o >>= 1) h += __shfl_xor(h, o);
  return h;
}

// Select from split-K logit partials: one wave per token, four tokens per
// block; per-block partials of the entropy and of sum_t p[t][e] in a fixed
// order (token 0 + 1, + 2, + 3).
template <int NE>
__global__ __launch_bounds__(256) void k_router_select(
    const float* __restrict__ part, int nsplit, int T_, int E,
    const float* __restrict__ offset, const float* __restrict__ bias, int score,
    int k, int renorm, int n_group, int topk_group, float* __restrict__ logits,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ ps_part,
    float* __restrict__ ent_part, int nb, int32_t* __restrict__ backup) {
  __shared__ float sp[4][NE * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool tok_ok = t < T_;
  float l[NE], p[NE];
  gather_logits<NE>(l, part, nsplit, T_, E, t, tok_ok, lane, offset, logits);
  route_token<NE>(l, p, t, tok_ok, lane, E, bias, score, k, renorm, n_group, topk_group, ids,
                  wts, nb, backup);
  if (ent_part) {  // per-block partial of the tokens' routing entropies
    const float h = token_entropy<NE>(p, score);
    __shared__ float eh[4];
    if (lane == 0) eh[wave] = tok_ok ? h : 0.f;
    __syncthreads();
    if (threadIdx.x == 0) ent_part[blockIdx.x] = ((eh[0] + eh[1]) + eh[2]) + eh[3];
  }
  if (ps_part) {   // per-block partial of sum_t p[t][e], fixed summation order
#pragma unroll
    for (int i = 0; i < NE; ++i) sp[wave][lane + 64 * i] = tok_ok ? p[i] : 0.f;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
      ps_part[(size_t)blockIdx.x * E + e] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
  }
}

// Fused router for up to 32 experts and many tokens: a block of 16 waves
// computes the logits of 16 tokens over the whole of d into LDS (16x16
// MFMA blocks; the waves split over the 16-expert blocks, then over K, and
// the K parts are added in K order), then every wave routes one token
// exactly as k_router_select does.  The per-four-token partials (entropy,
// sum of p) have k_router_select's layout and summation order, so the
// statistics kernels read them unchanged.  No split-K partials go through
// global memory and one launch is saved.
template <typename T>
__global__ __launch_bounds__(1024) void k_router_fused(
    const T* __restrict__ X, const T* __restrict__ Wg, int T_, int d, int E,
    const float* __restrict__ offset, const float* __restrict__ bias, int score, int k,
    int renorm, int n_group, int topk_group, float* __restrict__ logits,
    int32_t* __restrict__ ids, float* __restrict__ wts, float* __restrict__ ps_part,
    float* __restrict__ ent_part, int nb, int32_t* __restrict__ backup) {
  __shared__ float part[16][16][65];        // [K part][token][expert]
  __shared__ float sp[16][64];              // p of each wave's token
  __shared__ float eh[16];                  // entropy of each wave's token
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16;
  const int nexb = (E + 15) / 16;           // 16-expert blocks (1..4)
  const int wpb = 16 / nexb;                // waves per expert block: K parts
  const int eb = wave % nexb, kq = wave / nexb;
  constexpr int EPL = 16 / sizeof(T);
  constexpr int KSTEP = EPL * 4;
  if (kq < wpb) {
    const int dq = MOE_CEIL_DIV(MOE_CEIL_DIV(d, wpb), KSTEP) * KSTEP;
    const int kb = min(kq * dq, d), ke = min(kb + dq, d);
    const int row = lane & 15, grp = lane >> 4;
    const int tok = t0 + row, ex = eb * 16 + row;
    const bool tv = tok < T_, ev = ex < E;
    const T* xa = X + (size_t)(tv ? tok : 0) * d;
    const T* wb = Wg + (size_t)(ev ? ex : 0) * d;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll 4
    for (int kk0 = kb; kk0 < ke; kk0 += KSTEP) {
      const int kk = kk0 + grp * EPL;
      u32x4 a = tv ? *(const u32x4*)(xa + kk) : zero;
      u32x4 b = ev ? *(const u32x4*)(wb + kk) : zero;
      if constexpr (sizeof(T) == 2) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0,
                                                       0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]),
                                                     acc, 0, 0, 0);
      }
    }
    // C layout: lane holds expert column lane & 15, tokens 4 (lane >> 4) + r
#pragma unroll
    for (int r = 0; r < 4; ++r) part[kq][grp * 4 + r][eb * 16 + (lane & 15)] = acc[r];
  }
  __syncthreads();
  const int t = t0 + wave;                  // this wave's token
  const bool tok_ok = t < T_;
  const bool ok = tok_ok && lane < E;
  float v = 0.f;
  if (ok) {
    for (int q = 0; q < wpb; ++q) v += part[q][wave][lane];   // K order
    if (offset) v += offset[lane];
    if (logits) logits[(size_t)t * E + lane] = v;
  }
  float l[1] = {ok ? v : -INFINITY}, p[1];
  route_token<1>(l, p, t, tok_ok, lane, E, bias, score, k, renorm, n_group, topk_group, ids, wts,
                 nb, backup);
  float h = 0.f;
  if (ent_part) h = token_entropy<1>(p, score);
  if (lane == 0) eh[wave] = tok_ok ? h : 0.f;
  sp[wave][lane] = tok_ok ? p[0] : 0.f;
  __syncthreads();
  // wave g < 4 writes the partials of tokens 4 g .. 4 g + 3 of the block
  if (wave < 4) {
    const int blk4 = blockIdx.x * 4 + wave;
    if ((int64_t)blk4 * 4 < T_) {
      const int w4 = wave * 4;
      if (ent_part && lane == 0)
        ent_part[blk4] = ((eh[w4] + eh[w4 + 1]) + eh[w4 + 2]) + eh[w4 + 3];
      if (ps_part && lane < E)
        ps_part[(size_t)blk4 * E + lane] =
            ((sp[w4][lane] + sp[w4 + 1][lane]) + sp[w4 + 2][lane]) + sp[w4 + 3][lane];
    }
  }
}

// Up to 32 experts: each block then re-reads at most 32 rows of W_g (from
// L2).  With 64 experts the per-block W_g traffic was the larger cost
// (Switch-shaped router 22 -> 39 us), and the tiled router GEMM, which
// shares W_g across 128-token tiles, stays faster.
bool router_fused_ok(int64_t T, int d, int E) {
  return E <= 32 && T >= 2048 && d % 128 == 0 && T <= INT32_MAX;
}

// Final prob_sum: one block per expert, fixed-order tree over block partials.
__global__ __launch_bounds__(256) void k_prob_sum(const float* __restrict__ ps_part,
                                                  int nblk, int E,
                                                  float* __restrict__ prob_sum) {
  __shared__ float red[256];
  const int e = blockIdx.x;
  float acc = 0.f;
  for (int b = threadIdx.x; b < nblk; b += 256) acc += ps_part[(size_t)b * E + e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) prob_sum[e] = red[0];
}

// Balance statistic E * sum_e (counts_e / (T k)) (prob_sum_e / T), in fp64.
__global__ __launch_bounds__(256) void k_balance(const int32_t* __restrict__ counts,
                                                 const float* __restrict__ prob_sum,
                                                 int64_t T_, int k, int E,
                                                 double* __restrict__ out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int e = threadIdx.x; e < E; e += 256)
    acc += (double)counts[e] * (double)prob_sum[e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tk = (double)T_ * (double)k;
    out[0] = (T_ > 0) ? (double)E * red[0] / (tk * (double)T_) : 0.0;
  }
}

// Router health: out = {mean token entropy, load entropy, load CV, drop rate}
// (LLM Internals 14.2.3's routing entropy / per-expert distribution / drop
// rate, AI Knowledge Map's expert-load CV).  One block, fixed-order sums.
__global__ __launch_bounds__(256) void k_router_health(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ n_kept,
                                                       const float* __restrict__ ent_part,
                                                       int nblk, int64_t T_, int k, int E,
                                                       double* __restrict__ out) {
  __shared__ double r0[256], r1[256], r2[256];
  const double tk = (double)T_ * (double)k;
  const double mean = tk / (double)E;
  double a = 0.0, b = 0.0, c = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) a += (double)ent_part[i];
  for (int e = threadIdx.x; e < E; e += 256) {
    const double n = (double)counts[e];
    const double f = tk > 0.0 ? n / tk : 0.0;
    if (f > 0.0) b -= f * log(f);
    c += (n - mean) * (n - mean);
  }
  r0[threadIdx.x] = a;
  r1[threadIdx.x] = b;
  r2[threadIdx.x] = c;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) {
      r0[threadIdx.x] += r0[threadIdx.x + st];
      r1[threadIdx.x] += r1[threadIdx.x + st];
      r2[threadIdx.x] += r2[threadIdx.x + st];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = T_ > 0 ? r0[0] / (double)T_ : 0.0;
    out[1] = r1[0];
    out[2] = mean > 0.0 ? sqrt(r2[0] / (double)E) / mean : 0.0;
    out[3] = tk > 0.0 ? 1.0 - (double)n_kept[0] / tk : 0.0;
  }
}

// --------------------------------------------------------------------------
// Expert-choice routing (LLM Internals 14.2.3, the expert-choice paradigm;
// oscine.io "MoE 03", expert-choice routing): expert e takes the C tokens
// with the highest score in its column, ties to the lower token index.
//
// Scores: keysT[e][t] in fp64, the log of the full-row softmax probability
// l - logsumexp(l) (same order as p), or the logit itself for a sigmoid
// router (same order as s).  One wave per token; 16 tokens per block go
// through LDS so that each expert's row of keys is written in 128-B runs.
constexpr int kEcTok = 16;

template <int NE>
__global__ __launch_bounds__(256) void k_ec_scores(const float* __restrict__ part, int nsplit,
                                                   int T_, int E,
                                                   const float* __restrict__ offset, int score,
                                                   float* __restrict__ logits,
                                                   double* __restrict__ keysT) {
  __shared__ double tile[kEcTok][NE * 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kEcTok;
  for (int r = 0; r < kEcTok / 4; ++r) {
    const int tl = wave * (kEcTok / 4) + r;
    const int t = t0 + tl;
    const bool tok_ok = t < T_;
    float l[NE];
    gather_logits<NE>(l, part, nsplit, T_, E, t, tok_ok, lane, offset, logits);
    double lse = 0.0;
    if (score == MOE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < NE; ++i) m = fmaxf(m, l[i]);
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      double z = 0.0;
#pragma unroll
      for (int i = 0; i < NE; ++i)
        if (tok_ok && lane + 64 * i < E) z += exp((double)l[i] - (double)m);
      for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
      lse = tok_ok ? (double)m + log(z) : 0.0;
    }
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int e = lane + 64 * i;
      // + 0.0 turns a -0.0 key into +0.0, so equal keys have equal bits
      if (e < E) tile[tl][e] = tok_ok ? ((double)l[i] - lse) + 0.0 : 0.0;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < E * kEcTok; idx += 256) {
    const int e = idx / kEcTok, tl = idx % kEcTok;
    if (t0 + tl < T_) keysT[(size_t)e * T_ + t0 + tl] = tile[tl][e];
  }
}

// Order-preserving map of a finite double onto uint64.
__device__ __forceinline__ uint64_t ord_key(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Selection: one 1024-thread block per expert.  An 8-pass MSB-first radix
// select over the 64-bit keys finds the C-th largest key K and how many keys
// equal to K to take (`need`); one ordered pass then takes every key > K and
// the first `need` keys == K in token order, and compacts the taken tokens in
// token order with block-wide ballot scans.  Integer-only decisions on the
// fp64 keys: run-to-run identical.
__global__ __launch_bounds__(1024) void k_ec_select(
    const double* __restrict__ keysT, int T_, int E, int C, int score,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row,
    float* __restrict__ gates, int32_t* __restrict__ row_token,
    int32_t* __restrict__ offsets, int32_t* __restrict__ counts,
    int32_t* __restrict__ n_kept, int tail_rows) {
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* kk = keysT + (size_t)e * T_;
  __shared__ int hist[256];
  __shared__ int s_digit, s_above;
  __shared__ int wsum[2][16];
  if (tid == 0) {
    offsets[e] = e * C;
    if (counts) counts[e] = C;
    if (e == 0) {
      offsets[E] = E * C;
      if (tail_rows > 0) offsets[E + 1] = E * C + tail_rows;
      if (n_kept) n_kept[0] = E * C;
    }
  }
  if (row_token)   // the shared expert's rows follow the E * C routed rows
    for (int t = e * 1024 + tid; t < tail_rows; t += E * 1024) row_token[E * C + t] = t;

  uint64_t prefix = 0, mask = 0;
  int need = C;                       // 1 <= need <= #keys matching prefix
  if (C > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int t = tid; t < T_; t += 1024) {
        const uint64_t u = ord_key(kk[t]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane L owns bins 255-4L .. 252-4L; counts run from the top bin down
        int c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; tot += c[j]; }
        int incl = tot;
        for (int o = 1; o < 64; o <<= 1) {
          const int n = __shfl_up(incl, o);
          if (lane >= o) incl += n;
        }
        int run = incl - tot;
        if (run < need && need <= incl) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (run + c[j] >= need) { s_digit = 255 - 4 * lane - j; s_above = run; break; }
            run += c[j];
          }
        }
      }
      __syncthreads();
      need -= s_above;
      prefix |= (uint64_t)s_digit << shift;
      mask |= 0xFFull << shift;
    }
  }

  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int base_eq = 0, base_pos = 0;
  for (int c0 = 0; c0 < T_; c0 += 1024) {
    const int t = c0 + tid;
    const bool v = t < T_;
    const double key = v ? kk[t] : 0.0;
    const uint64_t u = ord_key(key);
    const bool gt = v && C > 0 && u > prefix;
    const bool eq = v && C > 0 && u == prefix;
    const uint64_t be = __ballot(eq);
    if (lane == 0) wsum[0][wave] = __popcll(be);
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[0][w];
      pre += w < wave ? x : 0;
      tot += x;
    }
    const bool take = gt || (eq && base_eq + pre + __popcll(be & lt) < need);
    const uint64_t bt = __ballot(take);
    if (lane == 0) wsum[1][wave] = __popcll(bt);
    __syncthreads();
    int pre2 = 0, tot2 = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[1][w];
      pre2 += w < wave ? x : 0;
      tot2 += x;
    }
    if (v) {
      const size_t slot = (size_t)t * E + e;
      if (take) {
        const int row = e * C + base_pos + pre2 + __popcll(bt & lt);
        const double g = score == MOE_SOFTMAX ? exp(key) : 1.0 / (1.0 + exp(-key));
        if (sorted_slot) sorted_slot[row] = (int32_t)slot;
        if (row_token) row_token[row] = t;
        slot_row[slot] = row;
        gates[slot] = (float)g;
      } else {
        slot_row[slot] = -1;
        gates[slot] = 0.f;
      }
    }
    base_eq += tot;
    base_pos += tot2;
    __syncthreads();                  // wsum is rewritten by the next chunk
  }
}

// --------------------------------------------------------------- launchers
// K-split of the logits: about one slice per 1024 of d.  On the tiled-GEMM
// path it is doubled while that leaves fewer tiles than CUs, slices stay
// multiples of 128 elements and the partial logits the select pass reads
// stay small (<= 16 MB).
// Waves per 16-token group of the skinny logits kernel (divides 4).
static int router_wpt(int E) { return E > 48 ? 4 : E > 16 ? 2 : 1; }

int router_split(int64_t T, int d, int E, int dtype) {
  int s = d / 1024;
  s = s < 1 ? 1 : (s > 8 ? 8 : s);
  if (router_gemm_ok(dtype, T, d, E, s)) {
    while ((int64_t)router_gemm_tiles(T, E) * s < 256 && s * 2 <= 16 && d % (2 * s) == 0 &&
           (d / (2 * s)) % 128 == 0 && 2 * s * T * (int64_t)E * 4 <= ((int64_t)16 << 20))
      s *= 2;
  } else {
    // skinny kernel: with few tokens, split K further until the grid has
    // about two blocks per CU (each split keeps >= 256 elements of K)
    const int wpt = router_wpt(E);
    const int64_t blocks = MOE_CEIL_DIV(T, 16 * (4 / wpt)) * MOE_CEIL_DIV(E, 16 * wpt);
    while (blocks * s < 512 && d / (2 * s) >= 256 && 2 * s <= 32) s *= 2;
  }
  return s;
}

// Sized for the larger split of the two dtypes, so one size serves both.
size_t route_ws_bytes(int64_t T, int d, int E) {
  const int s0 = router_split(T, d, E, MOE_BF16), s1 = router_split(T, d, E, MOE_F32);
  const size_t split = (size_t)(s0 > s1 ? s0 : s1);
  size_t b = align256(split * (size_t)T * E * sizeof(float));      // partial logits
  b += align256((size_t)MOE_CEIL_DIV(T, 4) * E * sizeof(float));   // prob_sum partials
  b += router_gemm_ws_bytes(T, d, E, (int)split);                    // tiled-GEMM work list
  return b;
}

// Logit partials part[split][T][E] (the first region of ws); returns the
// split through *split_out and the rest of ws through *rest.
static hipError_t launch_logit_partials(const void* X, int dtype, int64_t T, int d,
                                        const void* Wg, int E, void* ws, hipStream_t s,
                                        float** part_out, int* split_out, char** rest) {
  const int split = router_split(T, d, E, dtype);
  const int kstep = 128;   // keep slices a multiple of both lane steps
  const int dchunk = MOE_CEIL_DIV(MOE_CEIL_DIV(d, split), kstep) * kstep;
  char* p = (char*)ws;
  float* part = (float*)p;  p += align256((size_t)split * T * E * sizeof(float));
  char* ps_region = p;      p += align256((size_t)MOE_CEIL_DIV(T, 4) * E * sizeof(float));
  *part_out = part;
  *split_out = split;
  *rest = ps_region;
  if (router_gemm_ok(dtype, T, d, E, split)) {
    // many experts: the LDS-tiled GEMM reads X once and W_g once per M-tile
    return launch_router_gemm(X, Wg, T, d, E, split, part, p, s);
  }
  const int wpt = router_wpt(E);
  dim3 g1((unsigned)MOE_CEIL_DIV(T, 16 * (4 / wpt)), (unsigned)MOE_CEIL_DIV(E, 16 * wpt),
          (unsigned)split);
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(k_router_logits<uint16_t>, g1, dim3(256), 0, s,
                       (const uint16_t*)X, (const uint16_t*)Wg, part, (int)T, d, E, dchunk, wpt);
  else
    hipLaunchKernelGGL(k_router_logits<float>, g1, dim3(256), 0, s,
                       (const float*)X, (const float*)Wg, part, (int)T, d, E, dchunk, wpt);
  return hipGetLastError();
}

hipError_t launch_route(const void* X, int dtype, int64_t T, int d, const void* Wg,
                        int E, const float* bias, const float* offset, int score,
                        int k, int renorm, int n_group, int topk_group, float* logits,
                        int32_t* ids, float* w, float* prob_sum, void* ws, hipStream_t s,
                        float* ent_part, int n_backup, int32_t* backup) {
  if (T == 0) {
    if (prob_sum) return launch_zero_f32(prob_sum, E, s);
    return hipSuccess;
  }
  const int nblk = (int)MOE_CEIL_DIV(T, 4);
  if (router_fused_ok(T, d, E)) {
    // logits and selection in one launch; the per-four-token partials go to
    // the same workspace region as on the split-K path
    const int split = router_split(T, d, E, dtype);
    float* ps_part = (float*)((char*)ws + align256((size_t)split * T * E * sizeof(float)));
    float* psp = prob_sum ? ps_part : nullptr;
    const dim3 grid((unsigned)MOE_CEIL_DIV(T, 16));
    if (dtype == MOE_BF16)
      hipLaunchKernelGGL(k_router_fused<uint16_t>, grid, dim3(1024), 0, s, (const uint16_t*)X,
                         (const uint16_t*)Wg, (int)T, d, E, offset, bias, score, k, renorm,
                         n_group, topk_group, logits, ids, w, psp, ent_part, n_backup, backup);
    else
      hipLaunchKernelGGL(k_router_fused<float>, grid, dim3(1024), 0, s, (const float*)X,
                         (const float*)Wg, (int)T, d, E, offset, bias, score, k, renorm,
                         n_group, topk_group, logits, ids, w, psp, ent_part, n_backup, backup);
    if (prob_sum)
      hipLaunchKernelGGL(k_prob_sum, dim3(E), dim3(256), 0, s, ps_part, nblk, E, prob_sum);
    return hipGetLastError();
  }
  float* part;
  int split;
  char* rest;
  hipError_t err = launch_logit_partials(X, dtype, T, d, Wg, E, ws, s, &part, &split, &rest);
  if (err != hipSuccess) return err;
  float* ps_part = (float*)rest;
  float* psp = prob_sum ? ps_part : nullptr;
  const int ne = MOE_CEIL_DIV(E, 64);
#define MOE_SEL(NE_)                                                                 \
  hipLaunchKernelGGL(k_router_select<NE_>, dim3(nblk), dim3(256), 0, s, part, split, \
                     (int)T, E, offset, bias, score, k, renorm, n_group, topk_group, logits, \
                     ids, w, psp, ent_part, n_backup, backup)
  switch (ne) {
    case 1: MOE_SEL(1); break;
    case 2: MOE_SEL(2); break;
    case 3: MOE_SEL(3); break;
    default: MOE_SEL(4); break;
  }
#undef MOE_SEL
  if (prob_sum)
    hipLaunchKernelGGL(k_prob_sum, dim3(E), dim3(256), 0, s, ps_part, nblk, E, prob_sum);
  return hipGetLastError();
}

hipError_t launch_router_health(const int32_t* counts, const int32_t* n_kept,
                                const float* ent_part, int64_t T, int k, int E, double* out,
                                hipStream_t s) {
  hipLaunchKernelGGL(k_router_health, dim3(1), dim3(256), 0, s, counts, n_kept, ent_part,
                     (int)MOE_CEIL_DIV(T, 4), T, k, E, out);
  return hipGetLastError();
}

// Selection-bias update (LLM Internals 14.2.3, DeepSeek-V3's load rule):
// bias[e] -= gamma if counts[e] > T*k/E, += gamma if below, unchanged if
// equal; the comparison counts[e]*E vs T*k is exact in integers.
__global__ __launch_bounds__(256) void k_bias_update(const int32_t* __restrict__ counts,
                                                     int64_t tk, int E, float gamma,
                                                     float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t load = (int64_t)counts[e] * E;
  if (load > tk) bias[e] -= gamma;
  else if (load < tk) bias[e] += gamma;
}

hipError_t launch_bias_update(const int32_t* counts, int64_t T, int k, int E, float gamma,
                              float* bias, hipStream_t s) {
  hipLaunchKernelGGL(k_bias_update, dim3((unsigned)MOE_CEIL_DIV(E, 256)), dim3(256), 0, s,
                     counts, T * (int64_t)k, E, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_balance(const int32_t* counts, const float* prob_sum, int64_t T, int k,
                          int E, double* out, hipStream_t s) {
  hipLaunchKernelGGL(k_balance, dim3(1), dim3(256), 0, s, counts, prob_sum, T, k, E, out);
  return hipGetLastError();
}

size_t route_ec_ws_bytes(int64_t T, int d, int E) {
  return route_ws_bytes(T, d, E) + align256((size_t)T * E * sizeof(double));
}

hipError_t launch_route_ec(const void* X, int dtype, int64_t T, int d, const void* Wg, int E,
                           const float* offset, int score, int C, float* logits,
                           int32_t* offsets, int32_t* counts, int32_t* n_kept,
                           int32_t* sorted_slot, int32_t* slot_row, float* gates,
                           int32_t* row_token, int tail_rows, void* ws, hipStream_t s) {
  double* keysT = (double*)((char*)ws + route_ws_bytes(T, d, E));
  if (T > 0) {
    float* part;
    int split;
    char* rest;
    hipError_t err = launch_logit_partials(X, dtype, T, d, Wg, E, ws, s, &part, &split, &rest);
    if (err != hipSuccess) return err;
    const unsigned nb = (unsigned)MOE_CEIL_DIV(T, kEcTok);
    const int ne = MOE_CEIL_DIV(E, 64);
#define MOE_ECS(NE_)                                                                      \
  hipLaunchKernelGGL(k_ec_scores<NE_>, dim3(nb), dim3(256), 0, s, part, split, (int)T, E, \
                     offset, score, logits, keysT)
    switch (ne) {
      case 1: MOE_ECS(1); break;
      case 2: MOE_ECS(2); break;
      case 3: MOE_ECS(3); break;
      default: MOE_ECS(4); break;
    }
#undef MOE_ECS
  }
  hipLaunchKernelGGL(k_ec_select, dim3(E), dim3(1024), 0, s, keysT, (int)T, E, C, score,
                     sorted_slot, slot_row, gates, row_token, offsets, counts, n_kept,
                     tail_rows);
  return hipGetLastError();
}

}  // namespace moe
