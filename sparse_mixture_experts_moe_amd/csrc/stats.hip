// Switch balance statistics and the router z-loss.
//   f[e] = count[e] / (T k);  P[e] = mean_t softmax(logits[t])[e];
//   loss = alpha E sum_e f[e] P[e];  zloss = mean_t (logsumexp logits[t])^2.
//
// Sources: "Zen MoDE: Mixture of Distilled Experts Architecture", section
// "Auxiliary Load Balancing Loss"; "Every parameter, every token", section
// "A balance penalty"; "Zen-Max: Maximum Capability via Mixture-of-Experts
// Architecture", section "MoE-Specific Training Stability" (z-loss).
//
// Deterministic: workgroup b owns a fixed block of 64 tokens, taken 32 at a
// time with eight lanes per token (each lane holds an eighth of the token's
// logits in registers; max and sum-exp combine with lane shuffles); the
// probabilities of the 32 tokens are summed per expert in token order and
// accumulated over the two rounds, giving partials[b][E].  One workgroup then
// adds the partials: 1024 threads sum fixed segments of blocks per expert in
// fp64, and the segments are added in segment order; the z-loss partials go
// through a fixed fp64 tree.  With a single block (T <= 64) that block
// finishes the statistics itself, with the same operations.  The eight lanes
// of a token combine through DPP moves.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTok = 64;        // tokens per partial block
constexpr int kRound = 32;      // tokens per round
constexpr int kLanes = 8;       // lanes per token

// kFinal (one block of tokens, T <= kTok): the block also finishes the
// statistics, with exactly the operations stats_final_kernel would apply to
// its single partial (the sums over empty segments add only zeros).
template <int KK, bool kFinal>  // logits per lane: experts q, q+8, ... below 8 KK >= E
__global__ __launch_bounds__(256) void stats_partial_kernel(
    const float* __restrict__ logits, int64_t T, int E, float* __restrict__ part,
    float* __restrict__ zpart, const int32_t* __restrict__ count, int k, float alpha,
    float* __restrict__ f, float* __restrict__ P, float* __restrict__ loss,
    float* __restrict__ zloss) {
  extern __shared__ float sp[];  // [kRound][E] probabilities of the current round
  __shared__ float zs[kRound];
  const int tid = threadIdx.x;
  const int tt = tid / kLanes, q = tid % kLanes;
  const int64_t tb0 = static_cast<int64_t>(blockIdx.x) * kTok;
  float acc = 0.0f;    // this thread's expert column sum (thread e < E)
  float zacc = 0.0f;   // thread 0: sum of lse^2
  for (int r = 0; r < kTok / kRound; ++r) {
    const int64_t t = tb0 + r * kRound + tt;
    const bool active = t < T;
    const float* row = logits + (active ? t : 0) * E;
    float v[KK];
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      const int e = q + u * kLanes;
      v[u] = (active && e < E) ? row[e] : -__builtin_inff();
    }
    float m = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < KK; ++u) m = fmaxf(m, v[u]);
    m = max8_f32(m);
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      if (q + u * kLanes < E) {
        v[u] = active ? expf(v[u] - m) : 0.0f;
        s += v[u];
      }
    }
    s = sum8_f32(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      const int e = q + u * kLanes;
      if (e < E) sp[tt * E + e] = active ? v[u] * inv : 0.0f;  // (inactive: s = 0)
    }
    if (q == 0) {
      const float lse = m + logf(s);
      zs[tt] = active ? lse * lse : 0.0f;
    }
    __syncthreads();
    if (tid < E)
      for (int u = 0; u < kRound; ++u) acc += sp[u * E + tid];
    if (tid == 0)
      for (int u = 0; u < kRound; ++u) zacc += zs[u];
    __syncthreads();
  }
  if constexpr (!kFinal) {
    if (tid < E) part[static_cast<int64_t>(blockIdx.x) * E + tid] = acc;
    if (tid == 0) zpart[blockIdx.x] = zacc;
  } else {
    __shared__ double fp[256];
    double term = 0.0;
    if (tid < E) {
      const double pe = static_cast<double>(acc) / static_cast<double>(T);
      const double fe = static_cast<double>(count[tid]) / (static_cast<double>(T) * k);
      P[tid] = static_cast<float>(pe);
      f[tid] = static_cast<float>(fe);
      term = fe * pe;
    }
    fp[tid] = term;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
      if (tid < st) fp[tid] += fp[tid + st];
      __syncthreads();
    }
    if (tid == 0) {
      loss[0] = static_cast<float>(static_cast<double>(alpha) * E * fp[0]);
      if (zloss) zloss[0] = static_cast<float>(static_cast<double>(zacc) / static_cast<double>(T));
    }
  }
}

__global__ __launch_bounds__(1024) void stats_final_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ zpart,
                                                           int nblk, const int32_t* __restrict__ count,
                                                           int64_t T, int E, int k, float alpha,
                                                           float* __restrict__ f,
                                                           float* __restrict__ P,
                                                           float* __restrict__ loss,
                                                           float* __restrict__ zloss) {
  __shared__ double seg[1024];
  __shared__ double fp[256];
  __shared__ double zt[1024];
  const int tid = threadIdx.x;
  const int nseg = 1024 / E;  // segments per expert (E <= 256 -> >= 4)
  const int e = tid % E, sgi = tid / E;
  double acc = 0.0;
  if (sgi < nseg) {
    const int b0 = static_cast<int>(static_cast<int64_t>(nblk) * sgi / nseg);
    const int b1 = static_cast<int>(static_cast<int64_t>(nblk) * (sgi + 1) / nseg);
    for (int b = b0; b < b1; ++b) acc += part[static_cast<int64_t>(b) * E + e];
  }
  seg[tid] = acc;
  __syncthreads();
  double term = 0.0;
  if (tid < E) {
    double tot = 0.0;
    for (int u = 0; u < nseg; ++u) tot += seg[u * E + tid];
    const double pe = tot / static_cast<double>(T);
    const double fe = static_cast<double>(count[tid]) / (static_cast<double>(T) * k);
    P[tid] = static_cast<float>(pe);
    f[tid] = static_cast<float>(fe);
    term = fe * pe;
  }
  if (tid < 256) fp[tid] = term;
  // z-loss partials: thread i sums blocks i, i + 1024, ... in order, then a
  // fixed tree adds the 1024 sums
  double z = 0.0;
  if (zloss)
    for (int b = tid; b < nblk; b += 1024) z += zpart[b];
  zt[tid] = z;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) {
      zt[tid] += zt[tid + s];
      if (tid < 128 && s <= 128) fp[tid] += fp[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    loss[0] = static_cast<float>(static_cast<double>(alpha) * E * fp[0]);
    if (zloss) zloss[0] = static_cast<float>(zt[0] / static_cast<double>(T));
  }
}

}  // namespace

int64_t stats_blocks(int64_t T) { return (T + kTok - 1) / kTok; }

hipError_t launch_balance_stats(const float* logits, const int32_t* count, int64_t T, int E, int k,
                                float alpha, float* f, float* P, float* loss, float* zloss,
                                float* part, float* zpart, hipStream_t stream) {
  const int64_t nblk = stats_blocks(T);
  const size_t lds = sizeof(float) * kRound * E;
  const unsigned g = static_cast<unsigned>(nblk);
#define MOE_STATS(KK, FIN)                                                                 \
  stats_partial_kernel<KK, FIN><<<g, 256, lds, stream>>>(logits, T, E, part, zpart, count, k, \
                                                         alpha, f, P, loss, zloss)
#define MOE_STATS_E(FIN)                    \
  if (E <= 32) MOE_STATS(4, FIN);           \
  else if (E <= 64) MOE_STATS(8, FIN);      \
  else if (E <= 128) MOE_STATS(16, FIN);    \
  else MOE_STATS(32, FIN)
  if (nblk == 1) {  // one block: it finishes the statistics itself
    MOE_STATS_E(true);
    return hipGetLastError();
  }
  MOE_STATS_E(false);
#undef MOE_STATS_E
#undef MOE_STATS
  stats_final_kernel<<<1, 1024, 0, stream>>>(part, zpart, static_cast<int>(nblk), count, T, E, k,
                                             alpha, f, P, loss, zloss);
  return hipGetLastError();
}

}  // namespace moe
