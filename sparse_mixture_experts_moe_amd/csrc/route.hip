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
// One workgroup (4 waves) owns 64 tokens.  The logits tile [64][E] is formed
// in LDS: bf16 inputs go through v_mfma_f32_16x16x32_bf16 with operand
// fragments loaded straight from global memory (both operands are contiguous
// along d, so one 16-byte load is one lane's 8-element fragment); fp32 inputs
// use FMA.  The epilogue gives each token four lanes: each lane scans a
// quarter of the experts and the four combine with two lane shuffles, k times.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTokPerBlock = 64;
constexpr int kThreads = 256;

// (v, i) ranks before (bv, bi): larger key first, lower index on equal keys.
__device__ __forceinline__ bool key_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void* __restrict__ xv, const void* __restrict__ wv, int64_t T, int d, int E, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias, int logits_in,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  extern __shared__ float lds[];
  const int ldl = E + 1;                        // padded row of the logits tile
  float* lg = lds;                              // [64][E+1]
  float* sb = lds + kTokPerBlock * ldl;         // [E] selection bias
  int* sel = reinterpret_cast<int*>(sb + E);    // [64][k] chosen experts

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock;
  const int ntok = static_cast<int>(T - t0 < kTokPerBlock ? T - t0 : kTokPerBlock);

  for (int e = tid; e < E; e += kThreads) sb[e] = select_bias ? select_bias[e] : 0.0f;

  if (logits_in) {
    for (int i = tid; i < ntok * E; i += kThreads) {
      const int t = i / E, e = i % E;
      lg[t * ldl + e] = logits[(t0 + t) * E + e];
    }
  } else if constexpr (kBf16) {
    // 16x16 output blocks: 4 token blocks x ceil(E/16) expert blocks; wave w
    // takes expert blocks w, w+4, ... for all four token blocks.
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    const uint16_t* w = static_cast<const uint16_t*>(wv);
    const int wave = tid / kWave, lane = tid % kWave;
    const int r16 = lane % 16, kq = (lane / 16) * 8;
    const int eblocks = (E + 15) / 16;
    const bf16x8* xrow[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      int t = tb * 16 + r16;
      t = t < ntok ? t : ntok - 1;  // rows past T read a valid row; results discarded
      xrow[tb] = reinterpret_cast<const bf16x8*>(x + (t0 + t) * d + kq);
    }
    for (int eb = wave; eb < eblocks; eb += 4) {
      int e = eb * 16 + r16;
      e = e < E ? e : E - 1;
      const bf16x8* wrow = reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(e) * d + kq);
      f32x4 acc[4] = {};
      for (int k0 = 0; k0 < d; k0 += 32) {
        const bf16x8 b = wrow[k0 / 8];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 a = xrow[tb][k0 / 8];
          acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[tb], 0, 0, 0);
        }
      }
      // D[token][expert]: lane holds expert column r16, token rows 4*(lane/16)+j.
      const int ecol = eb * 16 + r16;
      if (ecol < E) {
        const float lb = logit_bias ? logit_bias[ecol] : 0.0f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tb * 16 + (lane / 16) * 4 + j;
            lg[t * ldl + ecol] = acc[tb][j] + lb;
          }
      }
    }
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
  }
  __syncthreads();

  if (!logits_in) {
    for (int i = tid; i < ntok * E; i += kThreads) {
      const int t = i / E, e = i % E;
      logits[(t0 + t) * E + e] = lg[t * ldl + e];
    }
  }

  // ---- top-k: four lanes per token, lane q scans experts q, q+4, ... ----
  const int tt = tid / 4, q = tid % 4;
  const bool active = tt < ntok;
  const float* row = lg + tt * ldl;
  float pv = __builtin_inff();
  int pi = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    if (active) {
      for (int e = q; e < E; e += 4) {
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
    for (int m = 1; m <= 2; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 4);
      const int oi = __shfl_xor(bi, m, 4);
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
    for (int j = q; j < k; j += 4) {
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
