// Shared device helpers for the gfx950 MoE kernels (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 is a struct with a union, which keeps
// arrays of it out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

// bf16 <-> fp32 by bit manipulation (bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> two bf16 (lo in bits 15:0) with the gfx950 conversion
// instruction: round to nearest even, the same bits as f32_to_bf16_bits for
// finite inputs.
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(moe_f32x2{lo, hi}, moe_bf16x2));
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
  static constexpr int kBytes = 4;
  __device__ static float to_f32(float v) { return v; }
};
template <> struct ElemTraits<uint16_t> {   // bf16 storage
  static constexpr int kBytes = 2;
  __device__ static float to_f32(uint16_t v) { return bf16_bits_to_f32(v); }
};

// Launch-side helpers (host).
#define MOE_CEIL_DIV(a, b) (((a) + (b) - 1) / (b))

// Map a linear block id onto a logical tile id so that consecutive logical
// tiles run on the same XCD (gfx950 dispatches blocks round-robin over its
// 8 XCDs, each with a private L2).  Bijective on [0, nb).
__device__ __forceinline__ int xcd_swizzle(int bid, int nb) {
  const int q = nb >> 3, r = nb & 7;
  const int x = bid & 7, i = bid >> 3;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}
