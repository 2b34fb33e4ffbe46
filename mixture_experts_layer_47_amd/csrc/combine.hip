// Combine: LLM Internals 14.2.1 step 6 and the AI Knowledge Map "MoE" output
// y = sum_{e in S} g_e E_e(x): gate-weighted sum of each token's expert rows,
// read back through the inverse permutation (slot_row), plus the shared
// expert's row.  Dropped slots (row -1) add nothing.  fp32 accumulation in a
// fixed order (j = 0..k-1, then the shared row), one rounding to the output
// type, no atomics.  k may reach 256 (expert-choice routing passes k = E
// with one slot per expert); the kept slots are first compacted in LDS in
// slot order, so the sum only visits them.
#include "common.h"
#include "kernels.h"

namespace moe {

// A block of 512 threads serves 512 / TPT tokens, TPT threads each (TPT a
// multiple of 64 and at least k): narrow rows pack several tokens into a
// block, so blocks stay large enough that their launch cost does not
// dominate (8192 tokens of 2048 columns: 2048 blocks instead of 8192).
template <typename OutT, int TPT>
__global__ __launch_bounds__(512) void k_combine(const float* __restrict__ Yrows,
                                                 const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ w, int64_t T_, int k,
                                                 int d, const float* __restrict__ shared,
                                                 const int32_t* __restrict__ shared_row0,
                                                 OutT* __restrict__ Y) {
  static_assert(TPT % 64 == 0 && TPT <= 512, "whole waves per token");
  constexpr int NTB = 512 / TPT;              // tokens per block
  constexpr int WPT = TPT / 64;               // waves per token
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = threadIdx.x / TPT, lt = threadIdx.x % TPT;
  const int64_t t = (int64_t)blockIdx.x * NTB + grp;
  const bool tok = t < T_;
  __shared__ int32_t rows_[NTB][TPT];
  __shared__ float gw_[NTB][TPT];
  __shared__ int nw[8];
  int32_t* rows = rows_[grp];
  float* gw = gw_[grp];
  // compact this token's kept slots in slot order (k <= TPT: one slot per thread)
  int32_t r = -1;
  float g = 0.f;
  if (tok && lt < k) {
    r = slot_row[t * k + lt];
    g = w[t * k + lt];
  }
  const uint64_t kept = __ballot(r >= 0);
  if (lane == 0) nw[wave] = __popcll(kept);
  __syncthreads();
  const int w0 = grp * WPT;
  int at = 0, n = 0;
  for (int i = 0; i < WPT; ++i) {
    if (w0 + i < wave) at += nw[w0 + i];
    n += nw[w0 + i];
  }
  if (r >= 0) {
    const uint64_t below = lane ? (kept & (~0ull >> (64 - lane))) : 0ull;
    at += __popcll(below);
    rows[at] = r;
    gw[at] = g;
  }
  __syncthreads();
  if (!tok) return;                           // no block barrier below
  const float* sh = nullptr;
  if (shared)
    sh = shared + (size_t)t * d;
  else if (shared_row0)
    sh = Yrows + ((size_t)shared_row0[0] + t) * d;
  // expert row j of this column chunk
  auto row_val = [&](int j, int c) { return *(const float4*)(Yrows + (size_t)rows[j] * d + c); };
  for (int c = lt * 4; c < d; c += TPT * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    // four rows' loads in flight at once; the sum still runs j = 0, 1, ...
    for (; j + 4 <= n; j += 4) {
      float4 y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = row_val(j + u, c);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float gj = gw[j + u];
        acc.x += gj * y[u].x; acc.y += gj * y[u].y; acc.z += gj * y[u].z; acc.w += gj * y[u].w;
      }
    }
    if (j + 2 <= n) {
      const float4 y0 = row_val(j, c), y1 = row_val(j + 1, c);
      const float g0 = gw[j], g1 = gw[j + 1];
      acc.x += g0 * y0.x; acc.y += g0 * y0.y; acc.z += g0 * y0.z; acc.w += g0 * y0.w;
      acc.x += g1 * y1.x; acc.y += g1 * y1.y; acc.z += g1 * y1.z; acc.w += g1 * y1.w;
      j += 2;
    }
    for (; j < n; ++j) {
      const float4 y = row_val(j, c);
      const float gj = gw[j];
      acc.x += gj * y.x; acc.y += gj * y.y; acc.z += gj * y.z; acc.w += gj * y.w;
    }
    if (sh) {
      const float4 y = *(const float4*)(sh + c);
      acc.x += y.x; acc.y += y.y; acc.z += y.z; acc.w += y.w;
    }
    if constexpr (sizeof(OutT) == 2) {
      *(uint2*)(Y + (size_t)t * d + c) =
          make_uint2(bf16x2_bits(acc.x, acc.y), bf16x2_bits(acc.z, acc.w));
    } else {
      *(float4*)(Y + (size_t)t * d + c) = acc;
    }
  }
}

// Threads per token: about 16 columns per thread (four 16-B row loads in
// flight per pass), rounded up to a power of two in [64, 512], and at
// least k rounded up to whole waves.
static int combine_tpt(int64_t k, int d) {
  int tpt = 64;
  while (tpt < 512 && tpt * 16 < d) tpt *= 2;
  while (tpt < 512 && tpt < k) tpt *= 2;
  return tpt;
}

template <typename OutT>
static void run_combine(int tpt, const float* Yrows, const int32_t* slot_row, const float* w,
                        int64_t T, int k, int d, const float* shared, const int32_t* shared_row0,
                        OutT* Y, hipStream_t s) {
  const unsigned nb = (unsigned)MOE_CEIL_DIV(T, 512 / tpt);
#define MOE_COMBINE(TPT_)                                                                      \
  hipLaunchKernelGGL((k_combine<OutT, TPT_>), dim3(nb), dim3(512), 0, s, Yrows, slot_row, w, T, \
                     k, d, shared, shared_row0, Y)
  switch (tpt) {
    case 64: MOE_COMBINE(64); break;
    case 128: MOE_COMBINE(128); break;
    case 256: MOE_COMBINE(256); break;
    default: MOE_COMBINE(512); break;
  }
#undef MOE_COMBINE
}

hipError_t launch_combine(const float* Yrows, const int32_t* slot_row, const float* w, int64_t T,
                          int k, int d, const float* shared, const int32_t* shared_row0, void* Y,
                          int dtype, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int tpt = combine_tpt(k, d);
  if (dtype == MOE_BF16)
    run_combine<uint16_t>(tpt, Yrows, slot_row, w, T, k, d, shared, shared_row0, (uint16_t*)Y, s);
  else
    run_combine<float>(tpt, Yrows, slot_row, w, T, k, d, shared, shared_row0, (float*)Y, s);
  return hipGetLastError();
}

}  // namespace moe
