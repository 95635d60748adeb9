// Internal helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> packed bfloat16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16_bits(a)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(b)) << 16);
}

__device__ __forceinline__ float silu_f32(float z) {
  // z * sigmoid(z); for very negative z, exp(-z) overflows to inf and the
  // quotient is the correct limit -0.
  return z / (1.0f + __expf(-z));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
