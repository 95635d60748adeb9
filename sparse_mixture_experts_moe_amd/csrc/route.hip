// Router: logits = x . w_router^T (+ logit_bias), top-k selection on
// key = logit + select_bias (ties to the lower expert index), and gates that
// renormalise the softmax over the selected logits.
//
// Sources: "Every parameter, every token", section "The gating network";
// "Zen MoDE: Mixture of Distilled Experts Architecture", section "Router
// Architecture" (standard router equation); "Zen-Max: Maximum Capability via
// Mixture-of-Experts Architecture", section "Auxiliary-Loss-Free Load
// Balancing" (selection-only bias).
//
// One workgroup (4 waves) owns 32 tokens.  The router GEMM is HBM-bound
// (x is read once), so the workgroup splits the reduction over d between its
// waves: wave w takes the 32-wide d chunks w, w+4, w+8, ... for all tokens and
// all experts, with bf16 operand fragments loaded straight from global memory
// into v_mfma_f32_16x16x32_bf16 (both operands are contiguous along d, so one
// 16-byte load is one lane's 8-element fragment).  The four partial logit
// tiles are added in LDS in wave order, which fixes the summation order.
// fp32 inputs use FMA.  Top-k then gives each token eight lanes: each lane
// scans an eighth of the experts and the eight combine with three lane
// shuffles, k times.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTokPerBlock = 32;
constexpr int kThreads = 256;
constexpr int kLanesPerTok = kThreads / kTokPerBlock;  // 8

// (v, i) ranks before (bv, bi): larger key first, lower index on equal keys.
__device__ __forceinline__ bool key_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Partial logits of this wave: tokens [t0, t0+32) x experts [0, E) over the d
// chunks wave, wave+4, ...; acc[eb][tb] is the 16x16 block (token block tb,
// expert block eb).  EB = number of 16-wide expert blocks this instance covers.
template <int EB>
__device__ __forceinline__ void router_partial(const uint16_t* __restrict__ x,
                                               const uint16_t* __restrict__ w, int64_t t0,
                                               int ntok, int d, int E, int eb0, int wave,
                                               int lane, f32x4 (&acc)[EB][2]) {
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const bf16x8* xrow[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    int t = tb * 16 + r16;
    t = t < ntok ? t : ntok - 1;  // rows past T read a valid row; results discarded
    xrow[tb] = reinterpret_cast<const bf16x8*>(x + (t0 + t) * d + kq);
  }
  const bf16x8* wrow[EB];
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) {
    int e = (eb0 + eb) * 16 + r16;
    e = e < E ? e : E - 1;
    wrow[eb] = reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(e) * d + kq);
  }
#pragma unroll
  for (int eb = 0; eb < EB; ++eb) acc[eb][0] = acc[eb][1] = f32x4{};
  const int nchunk = d / 32;
#pragma unroll 2
  for (int c = wave; c < nchunk; c += 4) {
    const int o = c * 4;  // 32 elements = 4 fragments of 8
    const bf16x8 a0 = xrow[0][o], a1 = xrow[1][o];
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const bf16x8 b = wrow[eb][o];
      acc[eb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[eb][0], 0, 0, 0);
      acc[eb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[eb][1], 0, 0, 0);
    }
  }
}

// Adds this wave's partial tile into lg[32][ldl] in wave order 0..3.
template <int EB>
__device__ __forceinline__ void router_reduce(float* lg, int ldl, int E, int eb0, int wave,
                                              int lane, const f32x4 (&acc)[EB][2]) {
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        const int e = (eb0 + eb) * 16 + lane % 16;
        if (e >= E) continue;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // D[token][expert]: lane holds expert column lane%16, token rows 4*(lane/16)+j
            float* p = lg + (tb * 16 + (lane / 16) * 4 + j) * ldl + e;
            *p = (w == 0 ? 0.0f : *p) + acc[eb][tb][j];
          }
      }
    }
    __syncthreads();
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv, int64_t T, int d, int E, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias, int logits_in,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  extern __shared__ float lds[];
  const int ldl = E + 1;                        // padded row of the logits tile
  float* lg = lds;                              // [32][E+1]
  float* sb = lds + kTokPerBlock * ldl;         // [E] selection bias
  int* sel = reinterpret_cast<int*>(sb + E);    // [32][k] chosen experts

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock;
  const int ntok = static_cast<int>(T - t0 < kTokPerBlock ? T - t0 : kTokPerBlock);

  for (int e = tid; e < E; e += kThreads) sb[e] = select_bias ? select_bias[e] : 0.0f;

  if (logits_in) {
    for (int i = tid; i < ntok * E; i += kThreads) {
      const int t = i / E, e = i % E;
      lg[t * ldl + e] = logits[(t0 + t) * E + e];
    }
    __syncthreads();
  } else if constexpr (kBf16) {
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    const uint16_t* w = static_cast<const uint16_t*>(wv);
    // expert blocks in groups of 4 (64 experts) to bound the accumulators
    const int eblocks = (E + 15) / 16;
    for (int eb0 = 0; eb0 < eblocks; eb0 += 4) {
      const int n = eblocks - eb0;
      if (n >= 4) {
        f32x4 acc[4][2];
        router_partial<4>(x, w, t0, ntok, d, E, eb0, wave, lane, acc);
        router_reduce<4>(lg, ldl, E, eb0, wave, lane, acc);
      } else if (n == 3) {
        f32x4 acc[3][2];
        router_partial<3>(x, w, t0, ntok, d, E, eb0, wave, lane, acc);
        router_reduce<3>(lg, ldl, E, eb0, wave, lane, acc);
      } else if (n == 2) {
        f32x4 acc[2][2];
        router_partial<2>(x, w, t0, ntok, d, E, eb0, wave, lane, acc);
        router_reduce<2>(lg, ldl, E, eb0, wave, lane, acc);
      } else {
        f32x4 acc[1][2];
        router_partial<1>(x, w, t0, ntok, d, E, eb0, wave, lane, acc);
        router_reduce<1>(lg, ldl, E, eb0, wave, lane, acc);
      }
    }
    if (logit_bias) {
      for (int i = tid; i < ntok * E; i += kThreads) {
        const int t = i / E, e = i % E;
        lg[t * ldl + e] += logit_bias[e];
      }
    }
    __syncthreads();
  } else {
    const float* x = static_cast<const float*>(xv);
    const float* w = static_cast<const float*>(wv);
    for (int i = tid; i < ntok * E; i += kThreads) {
      const int t = i / E, e = i % E;
      const float* xr = x + (t0 + t) * d;
      const float* wr = w + static_cast<int64_t>(e) * d;
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wr[c], acc);
      lg[t * ldl + e] = acc + (logit_bias ? logit_bias[e] : 0.0f);
    }
    __syncthreads();
  }

  if (!logits_in) {
    for (int i = tid; i < ntok * E; i += kThreads) {
      const int t = i / E, e = i % E;
      logits[(t0 + t) * E + e] = lg[t * ldl + e];
    }
  }

  // ---- top-k: eight lanes per token, lane q scans experts q, q+8, ... ----
  const int tt = tid / kLanesPerTok, q = tid % kLanesPerTok;
  const bool active = tt < ntok;
  const float* row = lg + tt * ldl;
  float pv = __builtin_inff();
  int pi = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    if (active) {
      for (int e = q; e < E; e += kLanesPerTok) {
        const float v = select_bias ? __fadd_rn(row[e], sb[e]) : row[e];
        // candidates rank strictly after the previous winner
        const bool after_prev = v < pv || (v == pv && e > pi);
        if (after_prev && key_before(v, e, bv, bi)) {
          bv = v;
          bi = e;
        }
      }
    }
#pragma unroll
    for (int m = 1; m < kLanesPerTok; m <<= 1) {
      const float ov = __shfl_xor(bv, m, kLanesPerTok);
      const int oi = __shfl_xor(bi, m, kLanesPerTok);
      if (key_before(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    pv = bv;
    pi = bi;
    if (active && q == 0) sel[tt * k + j] = bi;
  }
  __syncthreads();

  // ---- gates: softmax over the selected (unbiased) logits ----
  if (active) {
    float m = -__builtin_inff();
    for (int j = 0; j < k; ++j) m = fmaxf(m, row[sel[tt * k + j]]);
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s += expf(row[sel[tt * k + j]] - m);
    const float inv = 1.0f / s;
    for (int j = q; j < k; j += kLanesPerTok) {
      const int e = sel[tt * k + j];
      topk_idx[(t0 + tt) * k + j] = e;
      topk_gate[(t0 + tt) * k + j] = expf(row[e] - m) * inv;
    }
  }
}

}  // namespace

size_t route_lds_bytes(int E, int k) {
  return sizeof(float) * (static_cast<size_t>(kTokPerBlock) * (E + 1) + E) +
         sizeof(int) * static_cast<size_t>(kTokPerBlock) * k;
}

hipError_t launch_route(const void* x, const void* w, bool bf16, int64_t T, int d, int E, int k,
                        const float* logit_bias, const float* select_bias, bool logits_in,
                        float* logits, int32_t* topk_idx, float* topk_gate, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock);
  const size_t lds = route_lds_bytes(E, k);
  // the logits tile can exceed the default 64 KB dynamic LDS limit
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(bf16 ? route_kernel<true>
                                                               : route_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (bf16) {
    route_kernel<true><<<blocks, kThreads, lds, stream>>>(x, w, T, d, E, k, logit_bias, select_bias,
                                                          logits_in ? 1 : 0, logits, topk_idx,
                                                          topk_gate);
  } else {
    route_kernel<false><<<blocks, kThreads, lds, stream>>>(x, w, T, d, E, k, logit_bias,
                                                           select_bias, logits_in ? 1 : 0, logits,
                                                           topk_idx, topk_gate);
  }
  return hipGetLastError();
}

}  // namespace moe
