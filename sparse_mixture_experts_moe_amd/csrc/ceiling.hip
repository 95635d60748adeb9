// Measured ceilings of the device, for the roofline fractions reported beside
// the datasheet ones: a loop of bf16 MFMAs on register-resident operands (no
// memory traffic at all) and a streaming read of a device buffer.  Neither is
// part of the layer.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kProbeThreads = 256;
// dynamic LDS reserved at launch (and never touched): more than half of a
// CU's LDS, so no two workgroups share a CU
constexpr int kProbeLds = 96 * 1024;

// Each wave holds four A and four B fragments taken from `src` (a distinct
// 128-byte slice per lane, so the operands carry the caller's data, e.g.
// random normals) and runs `iters` rounds of the sixteen independent
// v_mfma_f32_32x32x16_bf16 that a 128 x 128 wave tile issues per k step, in
// the same operand order as the grouped GEMM.  The accumulators are summed and
// stored so that none of the work is dead.
__global__ __launch_bounds__(kProbeThreads) void mfma_ceiling_kernel(const bf16x8* __restrict__ src,
                                                                     int iters,
                                                                     float* __restrict__ out) {
  const size_t lane_id = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[lane_id * 8 + i];
    b[i] = src[lane_id * 8 + 4 + i];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc[t / 4][t % 4] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[t % 4], a[t / 4], acc[t / 4][t % 4], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[lane_id] = s;
}

// Grid-stride read of n 16-byte words, sixteen non-temporal loads in flight
// per lane (each word is read once; measured: 6.4-6.5 TB/s with 8192
// workgroups, against 5.9 with eight ordinary loads in flight); every lane
// folds what it read with XOR and stores one word.
__global__ __launch_bounds__(kProbeThreads) void read_ceiling_kernel(const u32x4* __restrict__ p,
                                                                     size_t n,
                                                                     uint32_t* __restrict__ out) {
  constexpr int kUnroll = 16;
  const size_t tid = static_cast<size_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * kProbeThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_mfma_ceiling(const void* src, int blocks, int iters, float* out,
                               hipStream_t stream) {
  ensure_dynamic_lds(reinterpret_cast<const void*>(&mfma_ceiling_kernel), kProbeLds);
  mfma_ceiling_kernel<<<blocks, kProbeThreads, kProbeLds, stream>>>(
      static_cast<const bf16x8*>(src), iters, out);
  return hipGetLastError();
}

hipError_t launch_read_ceiling(const void* buf, size_t bytes, int blocks, uint32_t* out,
                               hipStream_t stream) {
  read_ceiling_kernel<<<blocks, kProbeThreads, 0, stream>>>(static_cast<const u32x4*>(buf),
                                                            bytes / 16, out);
  return hipGetLastError();
}

}  // namespace moe
