// Router: logits = x . w_router^T (+ logit_bias), top-k selection on
// key = logit + select_bias (ties to the lower expert index; or, on request,
// key = softmax probability + select_bias), and gates that
// renormalise the softmax over the selected logits.  ReLU routing instead
// keeps, of the k largest logits, those above zero, with gate = logit, and
// leaves the remaining slots empty (expert -1, gate 0).
//
// Sources: "Every parameter, every token", section "The gating network";
// "Zen MoDE: Mixture of Distilled Experts Architecture", section "Router
// Architecture" (standard router equation); "Zen MoDE: Mixture of Diverse
// Experts", section "Router" (ReLU gating, an adaptive expert count per
// token); "Zen-Max: Maximum Capability via
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
constexpr int kMaxSplits = 8;  // d-splits of the router GEMM, at most

// The selection order of (key v, expert i) as one unsigned 64-bit number:
// larger keys first, equal keys (-0 and +0 included) to the lower index.  The
// high word maps the float's bits to an order-preserving unsigned integer
// (after -0 -> +0), the low word is ~i, so the larger number ranks first.
// Every finite or infinite key gives a number above 0, which stands for "no
// candidate".
__device__ __forceinline__ uint64_t rank_code(float v, int i) {
  const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~i);
}

// Router GEMM, bf16: a workgroup of four waves takes 128 tokens (32 per wave)
// and every expert, padded to NB blocks of 32 rows (rows past E repeat row
// E-1; their results are not stored).  K (= d) goes in chunks of 64, S =
// 8 / NB chunks per stage: the stage of w (32 KB) is loaded once into LDS, in
// full 128-byte lines, and read by all four waves; each wave loads its
// tokens' fragments of x for the whole stage straight from global memory
// (every x element is used once), issued together with the w loads.
// v_mfma_f32_32x32x16_bf16 takes the w fragment as first operand, so lane l
// accumulates token l & 31 of its wave against experts 8 (r / 4) +
// 4 (l >> 5) + r % 4 of each block.  A 32-wide last chunk (d % 64 == 32)
// runs its first two k steps only.  grid: (ceil(T / 128), KS); split s
// covers chunks [nch s / KS, nch (s + 1) / KS) and writes partial sums to
// out + s T E (the logits themselves, bias added, when KS = 1).
constexpr int kRouterTok = 128;

// Element offset of 16-byte chunk `chunk` (0..7) of row `row` in 64-element
// rows; the XOR spreads the 16 rows read together over distinct bank groups.
__device__ __forceinline__ int rswz(int row, int chunk) {
  return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
}

template <int NB>
__global__ __launch_bounds__(256) void router_logits_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t T, int d, int E,
    int KS, const float* __restrict__ logit_bias, float* __restrict__ out) {
  constexpr int S = 8 / NB;             // chunks per stage
  constexpr int ROWS = NB * 32;
  constexpr int CH = ROWS * 64;         // elements of one chunk of w in LDS
  constexpr int WP = S * CH / (256 * 8);  // 16-byte pieces per thread per stage (8)
  static_assert(WP == 8, "stage of 32 KB");
  __shared__ __align__(16) uint16_t wl[S * CH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouterTok;
  const int ks = blockIdx.y;
  const int nch = (d + 63) / 64;
  const int c0 = static_cast<int>(static_cast<int64_t>(nch) * ks / KS);
  const int c1 = static_cast<int>(static_cast<int64_t>(nch) * (ks + 1) / KS);
  int64_t t = t0 + wave * 32 + (lane & 31);
  const bool tok_ok = t < T;
  t = tok_ok ? t : T - 1;  // rows past T read a valid row; results not stored
  const uint16_t* xr = x + t * d + 8 * (lane >> 5);
  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};

  for (int cs0 = c0; cs0 < c1; cs0 += S) {
    // w pieces of this stage: piece q = tid + 256 p is row (q / 8) % ROWS,
    // slot q % 8 of chunk q / (8 ROWS); the slot holds the swizzled chunk
    bf16x8 wv[WP];
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const int q = tid + 256 * p;
      const int cs = q / (8 * ROWS), row = (q / 8) % ROWS, slot = q % 8;
      int c = cs0 + cs;
      c = c < c1 ? c : c1 - 1;
      int g = slot ^ ((row >> 1) & 7);
      if (64 * c + 64 > d) g &= 3;  // 32-wide last chunk: stay inside the row
      const int e = row < E ? row : E - 1;
      wv[p] = *reinterpret_cast<const bf16x8*>(w + static_cast<int64_t>(e) * d + 64 * c + 8 * g);
    }
    bf16x8 xv[S][4];
#pragma unroll
    for (int cs = 0; cs < S; ++cs) {
      int c = cs0 + cs;
      c = c < c1 ? c : c1 - 1;
      const bool half = 64 * c + 64 > d;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        xv[cs][st] = *reinterpret_cast<const bf16x8*>(xr + 64 * c + 16 * (half ? (st & 1) : st));
    }
    __syncthreads();  // the previous stage's LDS reads are done
#pragma unroll
    for (int p = 0; p < WP; ++p) {
      const int q = tid + 256 * p;
      *reinterpret_cast<bf16x8*>(wl + (q / (8 * ROWS)) * CH + ((q / 8) % ROWS) * 64 + (q % 8) * 8) =
          wv[p];
    }
    __syncthreads();
#pragma unroll
    for (int cs = 0; cs < S; ++cs) {
      const int c = cs0 + cs;
      if (c >= c1) break;
      const int nst = 64 * c + 64 > d ? 2 : 4;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st >= nst) break;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              wl + cs * CH + rswz(32 * b + (lane & 31), 2 * st + (lane >> 5)));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xv[cs][st], acc[b], 0, 0, 0);
        }
      }
    }
  }
  if (!tok_ok) return;
  // runs of four consecutive experts: one 16-byte store each where the run is
  // whole and aligned (E % 4 == 0), else element by element
  float* o = out + static_cast<int64_t>(ks) * T * E + t * E;
  const bool add_bias = KS == 1 && logit_bias;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 32 * b + 8 * q + 4 * (lane >> 5);
      f32x4 v = {acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]};
      if (add_bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += e + j < E ? logit_bias[e + j] : 0.0f;
      }
      if ((E & 3) == 0 && e + 3 < E) {
        *reinterpret_cast<f32x4*>(o + e) = v;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e + j < E) o[e + j] = v[j];
      }
    }
}

// mode: 0 = logits are in `logits` (caller's or written by the logits kernel
// with KS = 1); 1 = sum KS partial tiles from `part` and add logit_bias;
// 2 = fp32 inputs, compute with FMA.
// kProb: the selection key is the softmax probability plus the selection
// bias (instead of the logit plus the bias).
template <int KK, bool kProb>  // keys per lane: experts q, q+8, ... below 8 KK >= E
__global__ __launch_bounds__(kThreads) void route_select_kernel(
    int mode, int relu, const float* __restrict__ xf, const float* __restrict__ wf,
    const float* __restrict__ part, int KS, int64_t T, int d, int E, int k,
    const float* __restrict__ logit_bias, const float* __restrict__ select_bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  extern __shared__ float lds[];
  const int ldl = E + 1;                        // padded row of the logits tile
  float* lg = lds;                              // [32][E+1]
  float* sb = lds + kTokPerBlock * ldl;         // [E] selection bias
  float* lb = sb + E;                           // [E] logit bias
  int* sel = reinterpret_cast<int*>(lb + E);    // [32][k] chosen experts

  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokPerBlock;
  const int ntok = static_cast<int>(T - t0 < kTokPerBlock ? T - t0 : kTokPerBlock);

  for (int e = tid; e < E; e += kThreads) {
    sb[e] = select_bias ? select_bias[e] : 0.0f;
    lb[e] = logit_bias ? logit_bias[e] : 0.0f;
  }
  __syncthreads();
  if (mode == 1) {
    // the tile's logits are contiguous in every partial: all KS partials of a
    // pass are loaded together, then added in split order
    const int n = ntok * E;
    const int64_t base = t0 * E;
    constexpr int kPer = 16;  // logits per thread per pass (one pass for E <= 128)
    // 16-byte accesses need E % 4 == 0 (four logits then share a row and
    // every partial stays 16-byte aligned) and 16-byte aligned buffers
    const bool vec = (E & 3) == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
    if (vec) {
      // thread j of a pass takes logits 4j .. 4j+3
      constexpr int kPer4 = kPer / 4;
      const int n4 = n / 4;
      for (int j0 = tid; j0 < n4; j0 += kThreads * kPer4) {
        f32x4 v[kMaxSplits][kPer4];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
#pragma unroll
          for (int u = 0; u < kPer4; ++u) {
            const int j = j0 + u * kThreads;
            v[sp][u] = (sp < KS && j < n4)
                           ? *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(sp) * T * E +
                                                             base + 4 * j)
                           : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
#pragma unroll
        for (int u = 0; u < kPer4; ++u) {
          const int j = j0 + u * kThreads;
          if (j >= n4) continue;
          f32x4 acc = v[0][u];
#pragma unroll
          for (int sp = 1; sp < kMaxSplits; ++sp)
            if (sp < KS) acc += v[sp][u];
          const int t = (4 * j) / E, e = (4 * j) % E;
          const f32x4 l = acc + f32x4{lb[e], lb[e + 1], lb[e + 2], lb[e + 3]};
          *reinterpret_cast<f32x4*>(logits + base + 4 * j) = l;
#pragma unroll
          for (int c = 0; c < 4; ++c) lg[t * ldl + e + c] = l[c];
        }
      }
    }
    for (int i0 = tid; !vec && i0 < n; i0 += kThreads * kPer) {
      float v[kMaxSplits][kPer];
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const int i = i0 + u * kThreads;
          v[sp][u] = (sp < KS && i < n) ? part[static_cast<int64_t>(sp) * T * E + base + i] : 0.0f;
        }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + u * kThreads;
        if (i >= n) continue;
        float acc = v[0][u];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp)
          if (sp < KS) acc += v[sp][u];
        const int t = i / E, e = i % E;
        const float l = acc + lb[e];
        logits[base + i] = l;
        lg[t * ldl + e] = l;
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
      v = acc + lb[e];
      logits[g] = v;
    }
    lg[t * ldl + e] = v;
  }
  __syncthreads();

  // ---- top-k: eight lanes per token, lane q holds the keys of experts q,
  // q+8, ... in registers (E <= 256: at most 32) ----
  const int tt = tid / kLanesPerTok, q = tid % kLanesPerTok;
  const bool active = tt < ntok;
  const float* row = lg + tt * ldl;
  constexpr int kKeys = KK;
  uint64_t code[kKeys];  // 0: no candidate
  if constexpr (kProb) {
    // p_e = exp(l_e - m) / sum_e' exp(l_e' - m) over all experts (the eight
    // lanes' partial sums added by a fixed butterfly), key = p_e + b_e
    float ex[kKeys];
    float m = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const int e = q + u * kLanesPerTok;
      ex[u] = (active && e < E) ? row[e] : -__builtin_inff();
      m = fmaxf(m, ex[u]);
    }
    m = max8_f32(m);
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const int e = q + u * kLanesPerTok;
      ex[u] = (active && e < E) ? expf(ex[u] - m) : 0.0f;
      s += ex[u];
    }
    s = sum8_f32(s);
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const int e = q + u * kLanesPerTok;
      const float pe = ex[u] / s;
      code[u] = (active && e < E) ? rank_code(select_bias ? __fadd_rn(pe, sb[e]) : pe, e)
                                  : uint64_t{0};
    }
  } else {
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const int e = q + u * kLanesPerTok;
      code[u] = (active && e < E)
                    ? rank_code(select_bias ? __fadd_rn(row[e], sb[e]) : row[e], e)
                    : uint64_t{0};
    }
  }
  // pass j: the first candidate ranking after pass j-1's winner (branch-free)
  uint64_t prev = ~uint64_t{0};
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int u = 0; u < kKeys; ++u) {
      const uint64_t c = code[u] < prev ? code[u] : uint64_t{0};
      best = c > best ? c : best;
    }
    best = max8_u64(best);
    prev = best;
    if (active && q == 0) sel[tt * k + j] = static_cast<int>(~static_cast<uint32_t>(best));
  }
  __syncthreads();

  // ---- ReLU gates: the selected experts with a positive logit, gate = the
  // logit; the slots after them (the order is by descending logit) are empty
  if (active && relu) {
    for (int j = q; j < k; j += kLanesPerTok) {
      const int e = sel[tt * k + j];
      const float l = row[e];
      const bool use = l > 0.0f;
      topk_idx[(t0 + tt) * k + j] = use ? e : -1;
      topk_gate[(t0 + tt) * k + j] = use ? l : 0.0f;
    }
  }
  // ---- gates: softmax over the selected (unbiased) logits ----
  if (active && !relu) {
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

// d-splits for the logits kernel: enough workgroups for two per compute unit
// (~512), at most kMaxSplits (the select kernel adds that many partials per
// logit) and at most one split per 64-wide chunk.
int route_splits(int64_t T, int d, int E) {
  (void)E;
  const int64_t tiles = (T + kRouterTok - 1) / kRouterTok;
  int64_t ks = (512 + tiles - 1) / tiles;
  const int64_t nchunk = (d + 63) / 64;
  if (ks > kMaxSplits) ks = kMaxSplits;
  if (ks > nchunk) ks = nchunk;
  return static_cast<int>(ks < 1 ? 1 : ks);
}

}  // namespace

size_t route_lds_bytes(int E, int k) {
  return sizeof(float) * (static_cast<size_t>(kTokPerBlock) * (E + 1) + 2 * E) +
         sizeof(int) * static_cast<size_t>(kTokPerBlock) * k;
}

size_t route_workspace_bytes(int64_t T, int d, int E, bool bf16) {
  if (!bf16 || T == 0) return 0;
  const int ks = route_splits(T, d, E);
  return ks > 1 ? sizeof(float) * static_cast<size_t>(ks) * T * E : 0;
}

hipError_t launch_route(const void* x, const void* w, bool bf16, int64_t T, int d, int E, int k,
                        const float* logit_bias, const float* select_bias, bool logits_in,
                        bool prob_keys, bool relu, float* logits, int32_t* topk_idx,
                        float* topk_gate, void* ws, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((T + kTokPerBlock - 1) / kTokPerBlock);
  const size_t lds = route_lds_bytes(E, k);
  // the logits tile can exceed the default 64 KB dynamic LDS limit
  const void* sel_fn =
      prob_keys ? (E <= 32   ? reinterpret_cast<const void*>(route_select_kernel<4, true>)
                   : E <= 64  ? reinterpret_cast<const void*>(route_select_kernel<8, true>)
                   : E <= 128 ? reinterpret_cast<const void*>(route_select_kernel<16, true>)
                              : reinterpret_cast<const void*>(route_select_kernel<32, true>))
                : (E <= 32   ? reinterpret_cast<const void*>(route_select_kernel<4, false>)
                   : E <= 64  ? reinterpret_cast<const void*>(route_select_kernel<8, false>)
                   : E <= 128 ? reinterpret_cast<const void*>(route_select_kernel<16, false>)
                              : reinterpret_cast<const void*>(route_select_kernel<32, false>));
  ensure_dynamic_lds(sel_fn, static_cast<int>(lds));
  int mode = 0, ks = 1;
  if (!logits_in && bf16) {
    ks = route_splits(T, d, E);
    dim3 grid(static_cast<unsigned>((T + kRouterTok - 1) / kRouterTok), static_cast<unsigned>(ks));
    float* dst = ks > 1 ? static_cast<float*>(ws) : logits;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(w);
    if (E <= 32) router_logits_kernel<1><<<grid, 256, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst);
    else if (E <= 64) router_logits_kernel<2><<<grid, 256, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst);
    else if (E <= 128) router_logits_kernel<4><<<grid, 256, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst);
    else router_logits_kernel<8><<<grid, 256, 0, stream>>>(xb, wb, T, d, E, ks, logit_bias, dst);
    mode = ks > 1 ? 1 : 0;
  } else if (!logits_in) {
    mode = 2;
  }
#define MOE_SELECT(KK, P)                                                                 \
  route_select_kernel<KK, P><<<blocks, kThreads, lds, stream>>>(                           \
      mode, relu ? 1 : 0, static_cast<const float*>(x), static_cast<const float*>(w),       \
      static_cast<const float*>(ws), ks, T, d, E, k, logit_bias, select_bias, logits,       \
      topk_idx, topk_gate)
#define MOE_SELECT_E(P)                 \
  if (E <= 32) MOE_SELECT(4, P);        \
  else if (E <= 64) MOE_SELECT(8, P);   \
  else if (E <= 128) MOE_SELECT(16, P); \
  else MOE_SELECT(32, P)
  if (prob_keys) {
    MOE_SELECT_E(true);
  } else {
    MOE_SELECT_E(false);
  }
#undef MOE_SELECT_E
#undef MOE_SELECT
  return hipGetLastError();
}

}  // namespace moe
