// Backward pass of the routing side of the layer: the gate gradients from the
// combine, the logit gradients (renormalised gates, balance loss, z-loss) and
// the gradients of the linear router.
//
// Sources: "Every parameter, every token", sections "The gating network"
// (the selected set is held fixed; gradient reaches the router only through
// the gates of the experts that ran, and experts that were off get none),
// "A balance penalty" (the router is trained on the task and the penalty
// together) and "A budget" (a dropped pair has no expert output); "Zen MoDE: Mixture of
// Distilled Experts Architecture",
// section "Auxiliary Load Balancing Loss"; Zen-Max, section "MoE-Specific
// Training Stability" (z-loss).
//
// All sums run in a fixed order (lane butterflies, per-chunk partials added
// in chunk order): results are deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(q[i] << 16);
    v[2 * i + 1] = __uint_as_float(q[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }

// ---------------------------------------------------------------------------
// dgate[t, j] = sum_i dy[t, i] * y[pair_row[t k + j], i], 0 for a dropped pair,
// and (with dout) the upstream gradient of the kept pair's expert row,
// dout[pair_row[t k + j]] = gate[t, j] * dy[t] (in dy's dtype).
// One wave per token (four per workgroup); each lane takes 8 consecutive
// columns per step; slots go in batches of 8 and the lane partials of each
// slot are added by a butterfly.
// ---------------------------------------------------------------------------
constexpr int kGradSlots = 8;

__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
  *reinterpret_cast<u32x4*>(p) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
__device__ __forceinline__ void store1(float* p, float v) { *p = v; }

// Zero-computation experts (router ids from e_ffn on: n_zero zero, n_copy
// copy, n_const constant experts): a copy slot's output is the token's x row,
// a constant slot's the constant row, a zero slot's nothing.
template <typename YT>
struct BypassBwd {
  const int32_t* idx;
  int e_ffn, n_zero, n_copy, n_const;
  const YT* x;
  const YT* cvec;
};

template <typename DT, typename YT, bool kBypass>
__global__ __launch_bounds__(256) void combine_backward_kernel(const DT* __restrict__ dy,
                                                               const YT* __restrict__ y,
                                                               const int32_t* __restrict__ pair_row,
                                                               const float* __restrict__ gate,
                                                               int64_t T, int k, int d,
                                                               float* __restrict__ dgate,
                                                               DT* __restrict__ dout,
                                                               BypassBwd<YT> bp) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const int32_t* pr = pair_row + t * k;
  const DT* dyr = dy + t * d;
  for (int j0 = 0; j0 < k; j0 += kGradSlots) {
    int rows[kGradSlots];         // expert row of an FFN slot that ran, else -1
    const YT* src[kGradSlots];    // the slot's output row (NULL: none)
    float acc[kGradSlots], gs[kGradSlots];
#pragma unroll
    for (int u = 0; u < kGradSlots; ++u) {
      const int j = j0 + u;
      rows[u] = -1;
      src[u] = nullptr;
      bool ffn = true;
      if constexpr (kBypass) {
        const int e = j < k ? bp.idx[t * k + j] - bp.e_ffn : -1;
        if (e >= 0) {
          ffn = false;
          if (e >= bp.n_zero && e < bp.n_zero + bp.n_copy) {
            src[u] = bp.x + t * d;
          } else if (e >= bp.n_zero + bp.n_copy) {
            const int c = e - bp.n_zero - bp.n_copy;
            if (c < bp.n_const) src[u] = bp.cvec + static_cast<int64_t>(c) * d;
          }
        }
      }
      if (ffn && j < k && pr[j] >= 0) {
        rows[u] = pr[j];
        src[u] = y + static_cast<int64_t>(rows[u]) * d;
      }
      gs[u] = (dout && rows[u] >= 0) ? gate[t * k + j] : 0.0f;
      acc[u] = 0.0f;
    }
    if ((d & 7) == 0) {
      for (int c = lane * 8; c < d; c += kWave * 8) {
        float g[8];
        load8(dyr + c, g);
#pragma unroll
        for (int u = 0; u < kGradSlots; ++u) {
          if (!src[u]) continue;
          float v[8];
          load8(src[u] + c, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[u] = fmaf(g[i], v[i], acc[u]);
          if (dout && rows[u] >= 0) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = gs[u] * g[i];
            store8(dout + static_cast<int64_t>(rows[u]) * d + c, o);
          }
        }
      }
    } else {
      for (int c = lane; c < d; c += kWave) {
        const float g = load1(dyr + c);
#pragma unroll
        for (int u = 0; u < kGradSlots; ++u) {
          if (!src[u]) continue;
          acc[u] = fmaf(g, load1(src[u] + c), acc[u]);
          if (dout && rows[u] >= 0) store1(dout + static_cast<int64_t>(rows[u]) * d + c, gs[u] * g);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGradSlots; ++u) {
      const float s = wave_sum(acc[u]);
      if (lane == 0 && j0 + u < k) dgate[t * k + j0 + u] = src[u] ? s : 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------
// Zero-computation experts, the rest of their backward:
//   dx_acc[t, :] += (sum of g[t, j] over the token's copy slots) dy[t, :]
//   dconst[c, :]  = sum over the slots on constant expert c of g[t, j] dy[t, :]
// The first is one wave per token; the second sums fixed token ranges into
// partials (one workgroup per range, constant expert and 256 columns) that a
// second kernel adds in range order.
// ---------------------------------------------------------------------------
template <typename DT>
__global__ __launch_bounds__(256) void bypass_copy_dx_kernel(
    const DT* __restrict__ dy, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    int64_t T, int k, int d, int copy0, int copy1, float* __restrict__ dx) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  float gsum = 0.0f;
  bool any = false;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e >= copy0 && e < copy1) {
      gsum += gate[t * k + j];
      any = true;
    }
  }
  if (!any) return;
  if ((d & 7) == 0) {
    for (int c = lane * 8; c < d; c += kWave * 8) {
      float g[8], o[8];
      load8(dy + t * d + c, g);
      load8(dx + t * d + c, o);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(gsum, g[i], o[i]);
      store8(dx + t * d + c, o);
    }
  } else {
    for (int c = lane; c < d; c += kWave) dx[t * d + c] += gsum * load1(dy + t * d + c);
  }
}

constexpr int kConstCols = 256;

template <typename DT>
__global__ __launch_bounds__(kConstCols) void bypass_const_partial_kernel(
    const DT* __restrict__ dy, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    int64_t T, int k, int d, int const0, int n_const, int64_t tok_per, float* __restrict__ part) {
  // the gates of this expert's slots, 64 tokens at a time, staged in LDS (0
  // where the slot is on another expert), so the column loop waits on dy only
  __shared__ float g_tok[64];
  const int c = static_cast<int>(blockIdx.x) * kConstCols + threadIdx.x;
  const int s = blockIdx.y, ce = blockIdx.z;
  const int64_t t0 = s * tok_per;
  const int64_t t1 = t0 + tok_per < T ? t0 + tok_per : T;
  float acc = 0.0f;
  for (int64_t tb = t0; tb < t1; tb += 64) {
    const int n = static_cast<int>(t1 - tb < 64 ? t1 - tb : 64);
    if (threadIdx.x < 64) {
      float gs = 0.0f;
      if (static_cast<int>(threadIdx.x) < n) {
        const int64_t t = tb + threadIdx.x;
        for (int j = 0; j < k; ++j)
          if (idx[t * k + j] == const0 + ce) gs += gate[t * k + j];
      }
      g_tok[threadIdx.x] = gs;
    }
    __syncthreads();
    if (c < d)
      for (int i = 0; i < n; ++i)
        if (g_tok[i] != 0.0f) acc = fmaf(g_tok[i], load1(dy + (tb + i) * d + c), acc);
    __syncthreads();
  }
  if (c < d) part[(static_cast<int64_t>(s) * n_const + ce) * d + c] = acc;
}

__global__ __launch_bounds__(256) void bypass_const_reduce_kernel(const float* __restrict__ part,
                                                                  int splits, int n_const, int d,
                                                                  float* __restrict__ dconst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(n_const) * d;
  if (i >= n) return;
  float acc = 0.0f;
  for (int s = 0; s < splits; ++s) acc += part[s * n + i];
  dconst[i] = acc;
}

int bypass_const_splits(int64_t T) {
  const int64_t s = (T + 63) / 64;  // about 64 tokens per range, at most 64 ranges
  return static_cast<int>(s < 1 ? 1 : (s > 64 ? 64 : s));
}

// ---------------------------------------------------------------------------
// dlogits[t, e] = g_j (dg_j - sum_i g_i dg_i)               if e = idx[t, j]
//              + c_bal alpha E / T  p_te (f_e - sum_e' f_e' p_te')
//              + c_z (2 / T) lse_t p_te
// with p_t = softmax(logits[t]), f_e = count[e] / (T k), g the forward's
// gates.  One wave per token; lane l holds experts l, l + 64, ...
// ---------------------------------------------------------------------------
template <int KK>  // experts per lane: 64 KK >= E
__global__ __launch_bounds__(256) void route_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dgate,
    const int32_t* __restrict__ count, int64_t T, int E, int k, int relu, float alpha,
    float c_bal, float c_z, float* __restrict__ dl) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[KK], f[KK];
  float m = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < KK; ++u) {
    const int e = lane + u * kWave;
    v[u] = e < E ? row[e] : -__builtin_inff();
    f[u] = (count && e < E)
               ? static_cast<float>(count[e]) / (static_cast<float>(T) * static_cast<float>(k))
               : 0.0f;
    m = fmaxf(m, v[u]);
  }
  m = wave_max(m);
  float s = 0.0f;
#pragma unroll
  for (int u = 0; u < KK; ++u) {
    v[u] = lane + u * kWave < E ? __expf(v[u] - m) : 0.0f;
    s += v[u];
  }
  s = wave_sum(s);
  const float inv = 1.0f / s;
  float fp = 0.0f;
#pragma unroll
  for (int u = 0; u < KK; ++u) {
    v[u] *= inv;  // p
    fp = fmaf(f[u], v[u], fp);
  }
  fp = wave_sum(fp);
  const float lse = m + __logf(s);
  const float cb = c_bal * alpha * static_cast<float>(E) / static_cast<float>(T);
  const float cz = c_z * 2.0f * lse / static_cast<float>(T);
  // gate term: every lane forms the same inner product in slot order
  const int32_t* ir = idx + t * k;
  const float* gr = gate + t * k;
  const float* dgr = dgate + t * k;
  float inner = 0.0f;
  for (int j = 0; !relu && j < k; ++j) inner = fmaf(gr[j], dgr[j], inner);
  float out[KK];
#pragma unroll
  for (int u = 0; u < KK; ++u) out[u] = cb * v[u] * (f[u] - fp) + cz * v[u];
  for (int j = 0; j < k; ++j) {
    const int e = ir[j];
    // ReLU gate = logit on a used slot (an empty slot holds -1 and matches
    // no expert); softmax gate: g_j (dg_j - sum_i g_i dg_i)
    const float gt = relu ? dgr[j] : gr[j] * (dgr[j] - inner);
#pragma unroll
    for (int u = 0; u < KK; ++u)
      if (e == lane + u * kWave) out[u] += gt;
  }
  float* o = dl + t * E;
#pragma unroll
  for (int u = 0; u < KK; ++u)
    if (lane + u * kWave < E) o[lane + u * kWave] = out[u];
}

// ---------------------------------------------------------------------------
// Linear router.  dx[t, i] (+)= sum_e dl[t, e] W[e, i]: a workgroup takes 32
// tokens and 256 columns, one column per thread; the tokens' dl rows sit in
// LDS expert-major so that each expert's 32 values are read as 8 broadcast
// 16-byte words.
// ---------------------------------------------------------------------------
constexpr int kDxTok = 32;

template <typename WT>
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dl,
                                                        const WT* __restrict__ w, int64_t T, int d,
                                                        int E, float* __restrict__ dx,
                                                        bool accumulate) {
  extern __shared__ __align__(16) float sdl[];  // [E][kDxTok]
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kDxTok;
  for (int i = threadIdx.x; i < E * kDxTok; i += 256) {
    const int e = i / kDxTok, tt = i % kDxTok;
    sdl[i] = t0 + tt < T ? dl[(t0 + tt) * E + e] : 0.0f;
  }
  __syncthreads();
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= d) return;
  float acc[kDxTok];
#pragma unroll
  for (int tt = 0; tt < kDxTok; ++tt) acc[tt] = 0.0f;
  for (int e = 0; e < E; ++e) {
    const float wv = load1(w + static_cast<int64_t>(e) * d + col);
    const f32x4* p = reinterpret_cast<const f32x4*>(sdl + e * kDxTok);
#pragma unroll
    for (int q = 0; q < kDxTok / 4; ++q) {
      const f32x4 a = p[q];
#pragma unroll
      for (int z = 0; z < 4; ++z) acc[4 * q + z] = fmaf(a[z], wv, acc[4 * q + z]);
    }
  }
#pragma unroll
  for (int tt = 0; tt < kDxTok; ++tt) {
    if (t0 + tt >= T) break;
    float* o = dx + (t0 + tt) * d + col;
    *o = accumulate ? *o + acc[tt] : acc[tt];
  }
}

// dw[e, i] = sum_t dl[t, e] x[t, i]: workgroup (column tile of 256, expert
// tile of kExp, token chunk c) writes the chunk's partial sums to
// part[c][e][i]; router_dw_reduce_kernel adds the chunks in order.  The
// expert tile is the smallest of 8, 16 or 32 that holds E (E > 32 takes
// several tiles); each thread loads the x values of 8 tokens before their
// FMAs, which still run token by token in order.
constexpr int kDwExpMax = 32;
constexpr int kDwSub = 64;  // tokens staged in LDS at a time
constexpr int kDwLd = 8;    // x loads in flight per thread

template <typename XT, int kExp>
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ dl,
                                                        const XT* __restrict__ x, int64_t T, int d,
                                                        int E, int64_t chunk,
                                                        float* __restrict__ part) {
  __shared__ __align__(16) float sdl[kDwSub][kExp];
  const int col = blockIdx.x * 256 + threadIdx.x;
  const int e0 = blockIdx.y * kExp;
  const int64_t c0 = static_cast<int64_t>(blockIdx.z) * chunk;
  const int64_t c1 = c0 + chunk < T ? c0 + chunk : T;
  float acc[kExp];
#pragma unroll
  for (int u = 0; u < kExp; ++u) acc[u] = 0.0f;
  for (int64_t s0 = c0; s0 < c1; s0 += kDwSub) {
    __syncthreads();
    for (int i = threadIdx.x; i < kDwSub * kExp; i += 256) {
      const int tt = i / kExp, u = i % kExp;
      const int64_t t = s0 + tt;
      sdl[tt][u] = (t < c1 && e0 + u < E) ? dl[t * E + e0 + u] : 0.0f;
    }
    __syncthreads();
    if (col < d) {
      const int n = static_cast<int>(c1 - s0 < kDwSub ? c1 - s0 : kDwSub);
      for (int tb = 0; tb < n; tb += kDwLd) {
        float xv[kDwLd];
#pragma unroll
        for (int z = 0; z < kDwLd; ++z)  // tokens past the staged ones load nothing
          xv[z] = tb + z < n ? load1(x + (s0 + tb + z) * d + col) : 0.0f;
#pragma unroll
        for (int z = 0; z < kDwLd; ++z) {
          if (tb + z >= n) break;
          const f32x4* p = reinterpret_cast<const f32x4*>(&sdl[tb + z][0]);
#pragma unroll
          for (int q = 0; q < kExp / 4; ++q) {
            const f32x4 a = p[q];
#pragma unroll
            for (int w = 0; w < 4; ++w) acc[4 * q + w] = fmaf(a[w], xv[z], acc[4 * q + w]);
          }
        }
      }
    }
  }
  if (col >= d) return;
#pragma unroll
  for (int u = 0; u < kExp; ++u)
    if (e0 + u < E) part[(static_cast<int64_t>(blockIdx.z) * E + e0 + u) * d + col] = acc[u];
}

__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float* __restrict__ part,
                                                               int nchunk, int64_t n,
                                                               float* __restrict__ dw) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
#pragma unroll 8
  for (int c = 0; c < nchunk; ++c) s += part[c * n + i];  // in chunk order
  dw[i] = s;
}

// dlogit_bias[e] = sum_t dl[t, e]: one workgroup per expert, thread i sums
// tokens i, i + 256, ... in order, then a fixed tree.
__global__ __launch_bounds__(256) void router_db_kernel(const float* __restrict__ dl, int64_t T,
                                                        int E, float* __restrict__ db) {
  __shared__ float s[256];
  const int e = blockIdx.x;
  float acc = 0.0f;
  for (int64_t t = threadIdx.x; t < T; t += 256) acc += dl[t * E + e];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) s[threadIdx.x] += s[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) db[e] = s[0];
}

// token chunks of the dw partials: enough workgroups to cover the device
int dw_exp_tile(int E) { return E <= 8 ? 8 : (E <= 16 ? 16 : kDwExpMax); }

int dw_chunks(int64_t T, int d, int E) {
  const int et = dw_exp_tile(E);
  const int64_t tiles = static_cast<int64_t>((d + 255) / 256) * ((E + et - 1) / et);
  int64_t c = (1024 + tiles - 1) / tiles;
  const int64_t cmax = (T + kDwSub - 1) / kDwSub;
  if (c > cmax) c = cmax;
  return static_cast<int>(c < 1 ? 1 : c);
}

template <typename T_>
hipError_t router_backward_typed(const void* x, const void* w, const float* dl, int64_t T, int d,
                                 int E, float* dw, float* db, float* dx, bool acc, float* part,
                                 hipStream_t stream) {
  const T_* xp = static_cast<const T_*>(x);
  const T_* wp = static_cast<const T_*>(w);
  if (dx) {
    const dim3 grid((d + 255) / 256, static_cast<unsigned>((T + kDxTok - 1) / kDxTok));
    router_dx_kernel<T_><<<grid, 256, sizeof(float) * E * kDxTok, stream>>>(dl, wp, T, d, E, dx,
                                                                             acc);
  }
  if (dw) {
    const int nchunk = dw_chunks(T, d, E);
    const int64_t chunk = (T + nchunk - 1) / nchunk;
    const int et = dw_exp_tile(E);
    const dim3 grid((d + 255) / 256, (E + et - 1) / et, static_cast<unsigned>(nchunk));
    if (et == 8)
      router_dw_kernel<T_, 8><<<grid, 256, 0, stream>>>(dl, xp, T, d, E, chunk, part);
    else if (et == 16)
      router_dw_kernel<T_, 16><<<grid, 256, 0, stream>>>(dl, xp, T, d, E, chunk, part);
    else
      router_dw_kernel<T_, kDwExpMax><<<grid, 256, 0, stream>>>(dl, xp, T, d, E, chunk, part);
    const int64_t n = static_cast<int64_t>(E) * d;
    router_dw_reduce_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
        part, nchunk, n, dw);
  }
  if (db) router_db_kernel<<<E, 256, 0, stream>>>(dl, T, E, db);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_backward(const void* dy, bool dy_bf16, const void* y, bool y_bf16,
                                   const int32_t* pair_row, const float* gate, int64_t T, int k,
                                   int d, float* dgate, void* dout, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
#define MOE_CB(DT, YT)                                                                         \
  combine_backward_kernel<DT, YT, false><<<grid, 256, 0, stream>>>(                            \
      static_cast<const DT*>(dy), static_cast<const YT*>(y), pair_row, gate, T, k, d, dgate,   \
      static_cast<DT*>(dout), BypassBwd<YT>{})
  if (dy_bf16 && y_bf16) MOE_CB(uint16_t, uint16_t);
  else if (dy_bf16) MOE_CB(uint16_t, float);
  else if (y_bf16) MOE_CB(float, uint16_t);
  else MOE_CB(float, float);
#undef MOE_CB
  return hipGetLastError();
}

hipError_t launch_combine_backward_bypass(const void* dy, bool dy_bf16, const void* y,
                                          bool y_bf16, const int32_t* pair_row, const float* gate,
                                          int64_t T, int k, int d, const BypassArgs& b,
                                          float* dgate, void* dout, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
#define MOE_CB(DT, YT)                                                                         \
  combine_backward_kernel<DT, YT, true><<<grid, 256, 0, stream>>>(                             \
      static_cast<const DT*>(dy), static_cast<const YT*>(y), pair_row, gate, T, k, d, dgate,   \
      static_cast<DT*>(dout),                                                                  \
      BypassBwd<YT>{b.topk_idx, b.e_ffn, b.n_zero, b.n_copy, b.n_const,                        \
                    static_cast<const YT*>(b.x), static_cast<const YT*>(b.const_rows)})
  if (dy_bf16 && y_bf16) MOE_CB(uint16_t, uint16_t);
  else if (dy_bf16) MOE_CB(uint16_t, float);
  else if (y_bf16) MOE_CB(float, uint16_t);
  else MOE_CB(float, float);
#undef MOE_CB
  return hipGetLastError();
}

size_t bypass_backward_workspace_bytes(int64_t T, int d, int n_const) {
  return sizeof(float) * static_cast<size_t>(bypass_const_splits(T)) * n_const * d;
}

hipError_t launch_bypass_backward(const void* dy, bool dy_bf16, const int32_t* idx,
                                  const float* gate, int64_t T, int k, int d, int e_ffn,
                                  int n_zero, int n_copy, int n_const, float* dx_acc,
                                  float* dconst, void* ws, hipStream_t stream) {
  if (n_copy > 0 && dx_acc) {
    const unsigned grid = static_cast<unsigned>((T + 3) / 4);
    const int c0 = e_ffn + n_zero, c1 = c0 + n_copy;
    if (dy_bf16)
      bypass_copy_dx_kernel<uint16_t><<<grid, 256, 0, stream>>>(
          static_cast<const uint16_t*>(dy), idx, gate, T, k, d, c0, c1, dx_acc);
    else
      bypass_copy_dx_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(dy), idx,
                                                             gate, T, k, d, c0, c1, dx_acc);
  }
  if (n_const > 0 && dconst) {
    const int splits = bypass_const_splits(T);
    const int64_t tok_per = (T + splits - 1) / splits;
    const int const0 = e_ffn + n_zero + n_copy;
    float* part = static_cast<float*>(ws);
    dim3 grid(static_cast<unsigned>((d + kConstCols - 1) / kConstCols),
              static_cast<unsigned>(splits), static_cast<unsigned>(n_const));
    if (dy_bf16)
      bypass_const_partial_kernel<uint16_t><<<grid, kConstCols, 0, stream>>>(
          static_cast<const uint16_t*>(dy), idx, gate, T, k, d, const0, n_const, tok_per, part);
    else
      bypass_const_partial_kernel<float><<<grid, kConstCols, 0, stream>>>(
          static_cast<const float*>(dy), idx, gate, T, k, d, const0, n_const, tok_per, part);
    const int64_t n = static_cast<int64_t>(n_const) * d;
    bypass_const_reduce_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
        part, splits, n_const, d, dconst);
  }
  return hipGetLastError();
}

hipError_t launch_route_backward(const float* logits, const int32_t* idx, const float* gate,
                                 const float* dgate, const int32_t* count, int64_t T, int E, int k, bool relu,
                                 float alpha, float c_bal, float c_z, float* dlogits,
                                 hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>((T + 3) / 4);
#define MOE_RB(KK)                                                                          \
  route_backward_kernel<KK><<<grid, 256, 0, stream>>>(logits, idx, gate, dgate, count, T, E, k, \
                                                      relu ? 1 : 0, alpha, c_bal, c_z, dlogits)
  if (E <= 64) MOE_RB(1);
  else if (E <= 128) MOE_RB(2);
  else MOE_RB(4);
#undef MOE_RB
  return hipGetLastError();
}

size_t router_backward_workspace_bytes(int64_t T, int d, int E) {
  return sizeof(float) * static_cast<size_t>(dw_chunks(T, d, E)) * E * d;
}

hipError_t launch_router_backward(const void* x, const void* w_router, bool bf16, const float* dl,
                                  int64_t T, int d, int E, float* dw_router, float* dlogit_bias,
                                  float* dx, bool dx_accumulate, void* ws, hipStream_t stream) {
  float* part = static_cast<float*>(ws);
  return bf16 ? router_backward_typed<uint16_t>(x, w_router, dl, T, d, E, dw_router, dlogit_bias,
                                                dx, dx_accumulate, part, stream)
              : router_backward_typed<float>(x, w_router, dl, T, d, E, dw_router, dlogit_bias, dx,
                                             dx_accumulate, part, stream);
}

}  // namespace moe
