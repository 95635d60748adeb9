// Internal helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // 8 raw bytes

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

// Two floats -> packed bfloat16 pair (low half = a), round to nearest even
// (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// z * sigmoid(z) = z * rcp(1 + exp(-z)), with the hardware reciprocal (about
// one ulp); for very negative z, exp(-z) overflows to inf and the result is
// the correct limit -0.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// 32 bits from the lane that DPP control kCtrl selects within this lane's row.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}

// Butterfly over each group of eight consecutive lanes: swap neighbours, swap
// pairs (quad permutations), then mirror each half-row, which pairs every
// lane of one quad with a lane of the other; after the three steps all eight
// lanes hold the same result (the two operands of every step are swapped
// between the partner lanes, and max and + commute).
constexpr int kDppSwap1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror

__device__ __forceinline__ float max8_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppSwap1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<kDppSwap2>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
}

__device__ __forceinline__ float sum8_f32(float v) {
  v += __uint_as_float(dpp_u32<kDppSwap1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<kDppSwap2>(__float_as_uint(v)));
  return v + __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
}

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<kCtrl>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<kCtrl>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t max8_u64(uint64_t v) {
  uint64_t o = dpp_u64<kDppSwap1>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppSwap2>(v);
  v = o > v ? o : v;
  o = dpp_u64<kDppHalfMirror>(v);
  return o > v ? o : v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = __lane_id();
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
