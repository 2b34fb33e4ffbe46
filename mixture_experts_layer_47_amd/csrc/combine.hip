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

template <typename OutT>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ Yrows,
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
  __shared__ int nw[4];
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
  const int n = (nw[0] + nw[1]) + (nw[2] + nw[3]);
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
    if (Yrows2) sh2 = Yrows2 + ((size_t)shared_row0[0] + t) * d;
  }
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n; ++j) {
      const int r = rows[j];
      float4 y = *(const float4*)(Yrows + (size_t)r * d + c);
      if (Yrows2) {   // K-split partials are summed first, in split order
        const float4 y2 = *(const float4*)(Yrows2 + (size_t)r * d + c);
        y.x += y2.x; y.y += y2.y; y.z += y2.z; y.w += y2.w;
      }
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
      uint2 o;
      o.x = (uint32_t)f32_to_bf16_bits(acc.x) | ((uint32_t)f32_to_bf16_bits(acc.y) << 16);
      o.y = (uint32_t)f32_to_bf16_bits(acc.z) | ((uint32_t)f32_to_bf16_bits(acc.w) << 16);
      *(uint2*)(Y + (size_t)t * d + c) = o;
    } else {
      *(float4*)(Y + (size_t)t * d + c) = acc;
    }
  }
}

hipError_t launch_combine(const float* Yrows, const float* Yrows2, const int32_t* slot_row,
                          const float* w, int64_t T, int k, int d, const float* shared,
                          const int32_t* shared_row0, void* Y, int dtype, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(k_combine<uint16_t>, dim3((unsigned)T), dim3(256), 0, s, Yrows, Yrows2,
                       slot_row, w, k, d, shared, shared_row0, (uint16_t*)Y);
  else
    hipLaunchKernelGGL(k_combine<float>, dim3((unsigned)T), dim3(256), 0, s, Yrows, Yrows2,
                       slot_row, w, k, d, shared, shared_row0, (float*)Y);
  return hipGetLastError();
}

}  // namespace moe
