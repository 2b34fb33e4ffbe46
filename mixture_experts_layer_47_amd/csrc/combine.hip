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

// KS: a second fp32 slab (the down projection's second K-split) is present.
template <typename OutT, bool KS>
__global__ __launch_bounds__(512) void k_combine(const float* __restrict__ Yrows,
                                                 const float* __restrict__ Yrows2,
                                                 const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ w, int k, int d,
                                                 const float* __restrict__ shared,
                                                 const int32_t* __restrict__ shared_row0,
                                                 OutT* __restrict__ Y) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ int32_t rows[256];
  __shared__ float gw[256];
  __shared__ int nw[8];
  int32_t r = -1;
  float g = 0.f;
  if (threadIdx.x < (unsigned)k) {
    r = slot_row[(size_t)t * k + threadIdx.x];
    g = w[(size_t)t * k + threadIdx.x];
  }
  const uint64_t kept = __ballot(r >= 0);
  if (lane == 0) nw[wave] = __popcll(kept);
  __syncthreads();
  int at = 0;
  for (int i = 0; i < wave; ++i) at += nw[i];
  const int n = ((nw[0] + nw[1]) + (nw[2] + nw[3])) + ((nw[4] + nw[5]) + (nw[6] + nw[7]));
  if (r >= 0) {
    const uint64_t below = lane ? (kept & (~0ull >> (64 - lane))) : 0ull;
    at += __popcll(below);
    rows[at] = r;
    gw[at] = g;
  }
  __syncthreads();
  const float* sh = nullptr;
  const float* sh2 = nullptr;
  if (shared) {
    sh = shared + (size_t)t * d;
  } else if (shared_row0) {
    sh = Yrows + ((size_t)shared_row0[0] + t) * d;
    if constexpr (KS) sh2 = Yrows2 + ((size_t)shared_row0[0] + t) * d;
  }
  // Expert row j of this column chunk (K-split partials summed first, in
  // split order).
  auto row_val = [&](int j, int c) {
    const int r = rows[j];
    float4 y = *(const float4*)(Yrows + (size_t)r * d + c);
    if constexpr (KS) {
      const float4 y2 = *(const float4*)(Yrows2 + (size_t)r * d + c);
      y.x += y2.x; y.y += y2.y; y.z += y2.z; y.w += y2.w;
    }
    return y;
  };
  for (int c = threadIdx.x * 4; c < d; c += 512 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int j = 0;
    // four rows' loads in flight at once; the sum still runs j = 0, 1, ...
    for (; j + 4 <= n; j += 4) {
      float4 y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = *(const float4*)(Yrows + (size_t)rows[j + u] * d + c);
      if constexpr (KS) {
        float4 y2[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) y2[u] = *(const float4*)(Yrows2 + (size_t)rows[j + u] * d + c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          y[u].x += y2[u].x; y[u].y += y2[u].y; y[u].z += y2[u].z; y[u].w += y2[u].w;
        }
      }
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
      float4 y = *(const float4*)(sh + c);
      if (sh2) {
        const float4 y2 = *(const float4*)(sh2 + c);
        y.x += y2.x; y.y += y2.y; y.z += y2.z; y.w += y2.w;
      }
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

hipError_t launch_combine(const float* Yrows, const float* Yrows2, const int32_t* slot_row,
                          const float* w, int64_t T, int k, int d, const float* shared,
                          const int32_t* shared_row0, void* Y, int dtype, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)T), block(512);
  if (dtype == MOE_BF16) {
    if (Yrows2)
      hipLaunchKernelGGL((k_combine<uint16_t, true>), grid, block, 0, s, Yrows, Yrows2, slot_row, w,
                         k, d, shared, shared_row0, (uint16_t*)Y);
    else
      hipLaunchKernelGGL((k_combine<uint16_t, false>), grid, block, 0, s, Yrows, Yrows2, slot_row,
                         w, k, d, shared, shared_row0, (uint16_t*)Y);
  } else {
    if (Yrows2)
      hipLaunchKernelGGL((k_combine<float, true>), grid, block, 0, s, Yrows, Yrows2, slot_row, w, k,
                         d, shared, shared_row0, (float*)Y);
    else
      hipLaunchKernelGGL((k_combine<float, false>), grid, block, 0, s, Yrows, Yrows2, slot_row, w,
                         k, d, shared, shared_row0, (float*)Y);
  }
  return hipGetLastError();
}

}  // namespace moe
