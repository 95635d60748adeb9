// Combine: out[t] = shared_y[t] + sum over kept slots j of g[t,j] * y_perm[pair_row[t*k+j]],
// accumulated in fp32 in slot order and rounded once.  Without gates (g = 1)
// the same kernel adds the input gradients of a token's kept pairs in the
// backward pass.  With zero-computation experts (router experts past the
// E_ffn FFN experts: zero, then copy, then constant) a slot on such an expert
// contributes g times nothing, the token's own input row, or the expert's
// constant row.
//
// Sources: "Every parameter, every token", sections "The gating network"
// (the output is the gate-weighted sum of the selected experts), "A budget"
// (a dropped pair contributes nothing) and "A shared expert"; "Zen-Max:
// Maximum Capability via Mixture-of-Experts Architecture", section
// "Fine-Grained Expert Architecture" (shared experts are added); "Zen MoDE:
// Mixture of Diverse Experts", section "Router" (zero, copy and constant
// experts that skip the FFN).
//
// HBM-bound: one workgroup per token, each lane handles 8 consecutive
// columns per step (16-byte bf16 loads and stores); the rows of a batch of
// slots (k rounded up to 1, 2, 4 or kSlotBatch; and the shared row) are
// loaded together, unconditionally, before they are added in slot order, so
// a lane waits for memory once per batch.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kSlotBatch = 8;

template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw load_raw(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ void unpack(const Raw& q, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(q[i] << 16);
      v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[8]) {
    unpack(load_raw(p), v);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[8]) {
    const u32x4 q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    *reinterpret_cast<u32x4*>(p) = q;
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

template <>
struct Vec8<float> {
  struct Raw {
    f32x4 a, b;
  };
  static __device__ __forceinline__ Raw load_raw(const float* p) {
    return Raw{reinterpret_cast<const f32x4*>(p)[0], reinterpret_cast<const f32x4*>(p)[1]};
  }
  static __device__ __forceinline__ void unpack(const Raw& q, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = q.a[i];
      v[4 + i] = q.b[i];
    }
  }
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
  static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};

// Workgroup (t, y) covers the whole row of token t (gridDim.y = 1) or its
// columns [8 BLOCK y, 8 BLOCK (y + 1)) (gridDim.y column chunks, so that a few
// tokens still fill the device).
// Zero-computation experts: router ids e_ffn .. e_ffn + n_zero - 1 are zero
// experts, the next n_copy copy experts, the next n_const constant experts
// (rows of cvec).
template <typename YT>
struct Bypass {
  const int32_t* idx;
  int e_ffn, n_zero, n_copy, n_const;
  const YT* x;
  const YT* cvec;
};

// The source row of slot j of token t (NULL: contributes nothing).
template <typename YT, bool kBypass>
__device__ __forceinline__ const YT* slot_row(const YT* y, const int32_t* pr, int j, int64_t t,
                                              int k, int d, const Bypass<YT>& bp) {
  if constexpr (kBypass) {
    const int e = bp.idx[t * k + j] - bp.e_ffn;
    if (e >= 0) {
      if (e < bp.n_zero) return nullptr;
      if (e < bp.n_zero + bp.n_copy) return bp.x + t * d;
      const int c = e - bp.n_zero - bp.n_copy;
      return c < bp.n_const ? bp.cvec + static_cast<int64_t>(c) * d : nullptr;
    }
  }
  const int row = pr[j];
  return row >= 0 ? y + static_cast<int64_t>(row) * d : nullptr;
}

template <typename YT, typename OT, int BLOCK, int KB, bool kBypass = false>
__global__ __launch_bounds__(BLOCK) void combine_kernel(const YT* __restrict__ y,
                                                        const int32_t* __restrict__ pair_row,
                                                        const float* __restrict__ gate, int k,
                                                        int d, const YT* __restrict__ shared,
                                                        OT* __restrict__ out,
                                                        Bypass<YT> bp = Bypass<YT>{}) {
  const int64_t t = blockIdx.x;
  const int32_t* pr = pair_row + t * k;
  const float* g = gate ? gate + t * k : nullptr;  // NULL: every gate is 1
  if ((d & 7) == 0) {
    const int cw = gridDim.y == 1 ? d : BLOCK * 8;  // columns of this workgroup
    const int c0 = static_cast<int>(blockIdx.y) * cw;
    const int cend = min(d, c0 + cw);
    // the first batch's source rows (the same for every lane and column); a
    // slot without one (dropped, a zero expert, or past k) reads the batch's
    // first row instead and contributes nothing, so that the batch's loads
    // and the shared row's go out together before the first is used
    const YT* src0[KB];
    const YT* first0 = nullptr;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      src0[u] = u < k ? slot_row<YT, kBypass>(y, pr, u, t, k, d, bp) : nullptr;
      if (!first0) first0 = src0[u];
    }
    for (int c = c0 + threadIdx.x * 8; c < cend; c += BLOCK * 8) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      typename Vec8<YT>::Raw raw[KB];
      typename Vec8<YT>::Raw sh{};
      if (first0) {
#pragma unroll
        for (int u = 0; u < KB; ++u) raw[u] = Vec8<YT>::load_raw((src0[u] ? src0[u] : first0) + c);
      }
      if (shared) sh = Vec8<YT>::load_raw(shared + t * d + c);
      if (first0) {
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          if (!src0[u]) continue;
          const float gj = g ? g[u] : 1.0f;
          float v[8];
          Vec8<YT>::unpack(raw[u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(gj, v[i], acc[i]);
        }
      }
      for (int j0 = KB; j0 < k; j0 += KB) {  // more than KB slots (k > kSlotBatch)
        const YT* src[KB];
        const YT* first = nullptr;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          src[u] = j0 + u < k ? slot_row<YT, kBypass>(y, pr, j0 + u, t, k, d, bp) : nullptr;
          if (!first) first = src[u];
        }
        if (!first) continue;
#pragma unroll
        for (int u = 0; u < KB; ++u) raw[u] = Vec8<YT>::load_raw((src[u] ? src[u] : first) + c);
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          if (!src[u]) continue;
          const float gj = g ? g[j0 + u] : 1.0f;
          float v[8];
          Vec8<YT>::unpack(raw[u], v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(gj, v[i], acc[i]);
        }
      }
      if (shared) {
        float v[8];
        Vec8<YT>::unpack(sh, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
      }
      Vec8<OT>::store(out + t * d + c, acc);
    }
  } else {
    if (blockIdx.y != 0) return;
    for (int c = threadIdx.x; c < d; c += BLOCK) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        const YT* src = slot_row<YT, kBypass>(y, pr, j, t, k, d, bp);
        if (!src) continue;
        acc = fmaf(g ? g[j] : 1.0f, Vec8<YT>::load1(src + c), acc);
      }
      if (shared) acc += Vec8<YT>::load1(shared + t * d + c);
      Vec8<OT>::store1(out + t * d + c, acc);
    }
  }
}

// Enough workgroups for the device: whole rows per 256-thread workgroup when
// there are many tokens; for a few tokens (decode), 64-thread workgroups on
// 512-column chunks of a row.
// Slots are batched by KB (k rounded up to 1, 2, 4 or kSlotBatch).
template <typename YT, typename OT, int KB, bool kBypass>
void launch_kb(const void* y, const int32_t* pr, const float* g, int64_t T, int k, int d,
               const void* shared, void* out, const Bypass<YT>& bp, hipStream_t stream) {
  if (T >= 1024 || (d & 7) != 0) {
    combine_kernel<YT, OT, 256, KB, kBypass><<<dim3(static_cast<unsigned>(T), 1), 256, 0, stream>>>(
        static_cast<const YT*>(y), pr, g, k, d, static_cast<const YT*>(shared),
        static_cast<OT*>(out), bp);
  } else {
    const unsigned chunks = static_cast<unsigned>((d + 511) / 512);
    combine_kernel<YT, OT, 64, KB, kBypass><<<dim3(static_cast<unsigned>(T), chunks), 64, 0, stream>>>(
        static_cast<const YT*>(y), pr, g, k, d, static_cast<const YT*>(shared),
        static_cast<OT*>(out), bp);
  }
}

template <typename YT, typename OT, bool kBypass>
hipError_t launch_typed(const void* y, const int32_t* pr, const float* g, int64_t T, int k, int d,
                        const void* shared, void* out, const BypassArgs* bpa, hipStream_t stream) {
  Bypass<YT> bp{};
  if (bpa)
    bp = Bypass<YT>{bpa->topk_idx, bpa->e_ffn, bpa->n_zero, bpa->n_copy, bpa->n_const,
                    static_cast<const YT*>(bpa->x), static_cast<const YT*>(bpa->const_rows)};
  const int kb = k <= 1 ? 1 : (k <= 2 ? 2 : (k <= 4 ? 4 : kSlotBatch));
  if (kb == 1) launch_kb<YT, OT, 1, kBypass>(y, pr, g, T, k, d, shared, out, bp, stream);
  else if (kb == 2) launch_kb<YT, OT, 2, kBypass>(y, pr, g, T, k, d, shared, out, bp, stream);
  else if (kb == 4) launch_kb<YT, OT, 4, kBypass>(y, pr, g, T, k, d, shared, out, bp, stream);
  else launch_kb<YT, OT, kSlotBatch, kBypass>(y, pr, g, T, k, d, shared, out, bp, stream);
  return hipGetLastError();
}

template <bool kBypass>
hipError_t launch_any(const void* y, bool y_bf16, const int32_t* pair_row, const float* gate,
                      int64_t T, int k, int d, const void* shared, void* out, bool out_bf16,
                      const BypassArgs* bp, hipStream_t stream) {
  if (y_bf16) {
    return out_bf16
               ? launch_typed<uint16_t, uint16_t, kBypass>(y, pair_row, gate, T, k, d, shared, out, bp, stream)
               : launch_typed<uint16_t, float, kBypass>(y, pair_row, gate, T, k, d, shared, out, bp, stream);
  }
  return out_bf16
             ? launch_typed<float, uint16_t, kBypass>(y, pair_row, gate, T, k, d, shared, out, bp, stream)
             : launch_typed<float, float, kBypass>(y, pair_row, gate, T, k, d, shared, out, bp, stream);
}

}  // namespace

hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* pair_row, const float* gate,
                          int64_t T, int k, int d, const void* shared, void* out, bool out_bf16,
                          hipStream_t stream) {
  return launch_any<false>(y, y_bf16, pair_row, gate, T, k, d, shared, out, out_bf16, nullptr,
                           stream);
}

hipError_t launch_combine_bypass(const void* y, bool y_bf16, const int32_t* pair_row,
                                 const float* gate, int64_t T, int k, int d, const void* shared,
                                 void* out, bool out_bf16, const BypassArgs& bp,
                                 hipStream_t stream) {
  return launch_any<true>(y, y_bf16, pair_row, gate, T, k, d, shared, out, out_bf16, &bp, stream);
}

}  // namespace moe
