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
// Two kernels:
//   router_logits_kernel (bf16): one wave computes a 32-token x 64-expert tile
//     of partial logits over a contiguous range of 32-wide d chunks with
//     v_mfma_f32_16x16x32_bf16; operand fragments come straight from global
//     memory (both operands are contiguous along d, so one 16-byte load is one
//     lane's 8-element fragment).  The d range is split over KS waves so that
//     small batches still occupy the chip; the KS partial tiles go to a
//     workspace and are added in split order by the select kernel, which fixes
//     the summation order (KS = 1 writes the logits directly).
//   route_select_kernel: 32 tokens per workgroup; forms the logits tile in LDS
//     (sum of partials + logit_bias, or fp32 FMA for fp32 inputs, or the
//     caller's logits), writes it out, then gives each token eight lanes for
//     the top-k: each lane scans an eighth of the experts and the eight combine
//     with three lane shuffles, k times; the gates are a softmax over the
//     selected unbiased logits.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTokPerBlock = 32;
constexpr int kThreads = 256;
constexpr int kLanesPerTok = kThreads / kTokPerBlock;  // 8
constexpr int kExpPerTile = 64;                        // experts per logits tile

// (v, i) ranks before (bv, bi): larger key first, lower index on equal keys.
__device__ __forceinline__ bool key_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// grid: (token tiles) x (expert tiles) x KS, one wave each.  NEB expert
// blocks of 16 per tile (NEB = min(4, ceil(E/16)); blocks past E read a valid
// row and are not stored).  The d chunks are consumed in batches of kBatch:
// all fragments of a batch are loaded before its MFMAs, so a wave waits for
// memory once per batch rather than once per chunk.
constexpr int kBatch = 8;

template <int NEB>
__global__ __launch_bounds__(64) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int d, int E,
    int KS, const float* __restrict__ logit_bias, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock;
  const int e0 = blockIdx.y * kExpPerTile;
  const int ks = blockIdx.z;
  const int nchunk = d / 32;
  const int c0 = static_cast<int>(static_cast<int64_t>(nchunk) * ks / KS);
  const int c1 = static_cast<int>(static_cast<int64_t>(nchunk) * (ks + 1) / KS);
  const int r16 = lane % 16, kq = (lane / 16) * 8;
  const bf16x8* xrow[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    int64_t t = t0 + tb * 16 + r16;
    t = t < T ? t : T - 1;  // rows past T read a valid row; results discarded
    xrow[tb] = reinterpret_cast<const bf16x8*>(x + t * d + kq);
  }
  const bf16x8* wrow[NEB];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    int e = e0 + eb * 16 + r16;
    e = e < E ? e : E - 1;
    wrow[eb] = reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(e) * d + kq);
  }
  f32x4 acc[NEB][2];
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) acc[eb][0] = acc[eb][1] = f32x4{};
  int c = c0;
  for (; c + kBatch <= c1; c += kBatch) {
    bf16x8 a[kBatch][2], b[kBatch][NEB];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int o = (c + u) * 4;  // 32 elements = 4 fragments of 8
      a[u][0] = xrow[0][o];
      a[u][1] = xrow[1][o];
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) b[u][eb] = wrow[eb][o];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads in flight
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int eb = 0; eb < NEB; ++eb) {
        acc[eb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][0], b[u][eb], acc[eb][0], 0, 0, 0);
        acc[eb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][1], b[u][eb], acc[eb][1], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  for (; c < c1; ++c) {
    const int o = c * 4;
    const bf16x8 a0 = xrow[0][o], a1 = xrow[1][o];
    bf16x8 b[NEB];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) b[eb] = wrow[eb][o];
#pragma unroll
    for (int eb = 0; eb < NEB; ++eb) {
      acc[eb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b[eb], acc[eb][0], 0, 0, 0);
      acc[eb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b[eb], acc[eb][1], 0, 0, 0);
    }
  }
  // D[token][expert]: lane holds expert column lane%16, token rows 4*(lane/16)+j
  float* o = out + static_cast<int64_t>(ks) * T * E;
#pragma unroll
  for (int eb = 0; eb < NEB; ++eb) {
    const int e = e0 + eb * 16 + r16;
    if (e >= E) continue;
    const float lb = (KS == 1 && logit_bias) ? logit_bias[e] : 0.0f;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + tb * 16 + (lane / 16) * 4 + j;
        if (t < T) o[t * E + e] = acc[eb][tb][j] + lb;
      }
  }
}

// mode: 0 = logits are in `logits` (caller's or written by the logits kernel
// with KS = 1); 1 = sum KS partial tiles from `part` and add logit_bias;
// 2 = fp32 inputs, compute with FMA.
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    int mode, const float* __restrict__ xf, const float* __restrict__ wf,
    const float* __restrict__ part, int KS, int64_t T, int d, int E, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  extern __shared__ float lds[];
  const int ldl = E + 1;                        // padded row of the logits tile
  float* lg = lds;                              // [32][E+1]
  float* sb = lds + kTokPerBlock * ldl;         // [E] selection bias
  int* sel = reinterpret_cast<int*>(sb + E);    // [32][k] chosen experts

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock;
  const int ntok = static_cast<int>(T - t0 < kTokPerBlock ? T - t0 : kTokPerBlock);

  for (int e = tid; e < E; e += kThreads) sb[e] = select_bias ? select_bias[e] : 0.0f;
  if (mode == 1) {
    // the tile's logits are contiguous in every partial: add the KS partials in
    // split order, all loads of one split issued together
    const int n = ntok * E;
    const int64_t base = t0 * E;
    constexpr int kPer = 8;  // logits per thread per pass (32 * 256 / 256 = 32 at most)
    for (int i0 = tid; i0 < n; i0 += kThreads * kPer) {
      float v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + u * kThreads;
        v[u] = i < n ? part[base + i] : 0.0f;
      }
      for (int s = 1; s < KS; ++s) {
        const float* ps = part + static_cast<int64_t>(s) * T * E + base;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int i = i0 + u * kThreads;
          if (i < n) v[u] += ps[i];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + u * kThreads;
        if (i < n) {
          const int t = i / E, e = i % E;
          const float l = v[u] + (logit_bias ? logit_bias[e] : 0.0f);
          logits[base + i] = l;
          lg[t * ldl + e] = l;
        }
      }
    }
  }
  for (int i = tid; mode != 1 && i < ntok * E; i += kThreads) {
    const int t = i / E, e = i % E;
    const int64_t g = (t0 + t) * E + e;
    float v;
    if (mode == 0) {
      v = logits[g];
    } else {
      const float* xr = xf + (t0 + t) * d;
      const float* wr = wf + static_cast<int64_t>(e) * d;
      float acc = 0.0f;
      for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wr[c], acc);
      v = acc + (logit_bias ? logit_bias[e] : 0.0f);
      logits[g] = v;
    }
    lg[t * ldl + e] = v;
  }
  __syncthreads();

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

// d-splits for the logits kernel: enough waves to cover the chip (~1024),
// at most kMaxSplits (the select kernel adds that many partials per logit)
// and at most one split per 32-wide chunk.
constexpr int kMaxSplits = 8;
int route_splits(int64_t T, int d, int E) {
  const int64_t tiles = ((T + kTokPerBlock - 1) / kTokPerBlock) * ((E + kExpPerTile - 1) / kExpPerTile);
  int64_t ks = (1024 + tiles - 1) / tiles;
  const int64_t nchunk = d / 32;
  if (ks > kMaxSplits) ks = kMaxSplits;
  if (ks > nchunk) ks = nchunk;
  return static_cast<int>(ks < 1 ? 1 : ks);
}

}  // namespace

size_t route_lds_bytes(int E, int k) {
  return sizeof(float) * (static_cast<size_t>(kTokPerBlock) * (E + 1) + E) +
         sizeof(int) * static_cast<size_t>(kTokPerBlock) * k;
}

size_t route_workspace_bytes(int64_t T, int d, int E, bool bf16) {
  if (!bf16 || T == 0) return 0;
  const int ks = route_splits(T, d, E);
  return ks > 1 ? sizeof(float) * static_cast<size_t>(ks) * T * E : 0;
}

hipError_t launch_route(const void* x, const void* w, bool bf16, int64_t T, int d, int E, int k,
                        const float* logit_bias, const float* select_bias, bool logits_in,
                        float* logits, int32_t* topk_idx, float* topk_gate, void* ws,
                        hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock);
  const size_t lds = route_lds_bytes(E, k);
  // the logits tile can exceed the default 64 KB dynamic LDS limit
  ensure_dynamic_lds(reinterpret_cast<const void*>(route_select_kernel), static_cast<int>(lds));
  int mode = 0, ks = 1;
  if (!logits_in && bf16) {
    ks = route_splits(T, d, E);
    dim3 grid(blocks, static_cast<unsigned>((E + kExpPerTile - 1) / kExpPerTile),
              static_cast<unsigned>(ks));
    const int neb = (E + 15) / 16 < 4 ? (E + 15) / 16 : 4;
    float* dst = ks > 1 ? static_cast<float*>(ws) : logits;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(w);
    switch (neb) {
      case 1: router_logits_kernel<1><<<grid, 64, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst); break;
      case 2: router_logits_kernel<2><<<grid, 64, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst); break;
      case 3: router_logits_kernel<3><<<grid, 64, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst); break;
      default: router_logits_kernel<4><<<grid, 64, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst); break;
    }
    mode = ks > 1 ? 1 : 0;
  } else if (!logits_in) {
    mode = 2;
  }
  route_select_kernel<<<blocks, kThreads, lds, stream>>>(
      mode, static_cast<const float*>(x), static_cast<const float*>(w),
      static_cast<const float*>(ws), ks, T, d, E, k, logit_bias, select_bias, logits, topk_idx,
      topk_gate);
  return hipGetLastError();
}

}  // namespace moe
