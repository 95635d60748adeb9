// Switch balance statistics and the router z-loss.
//   f[e] = count[e] / (T k);  P[e] = mean_t softmax(logits[t])[e];
//   loss = alpha E sum_e f[e] P[e];  zloss = mean_t (logsumexp logits[t])^2.
//
// Sources: "Zen MoDE: Mixture of Distilled Experts Architecture", section
// "Auxiliary Load Balancing Loss"; "Every parameter, every token", section
// "A balance penalty"; "Zen-Max: Maximum Capability via Mixture-of-Experts
// Architecture", section "MoE-Specific Training Stability" (z-loss).
//
// Deterministic: workgroup b sums a fixed 256-token block into partials[b][E]
// (fp32, token order), then one workgroup adds the partials in block order in
// fp64.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTok = 256;

__global__ __launch_bounds__(256) void stats_partial_kernel(const float* __restrict__ logits,
                                                            int64_t T, int E,
                                                            float* __restrict__ part,
                                                            float* __restrict__ zpart) {
  __shared__ float sm[kTok], sinv[kTok], slse2[kTok];
  const int tid = threadIdx.x;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  const int ntok = static_cast<int>(T - t0 < kTok ? T - t0 : kTok);
  if (tid < ntok) {
    const float* row = logits + (t0 + tid) * E;
    float m = -__builtin_inff();
    for (int e = 0; e < E; ++e) m = fmaxf(m, row[e]);
    float s = 0.0f;
    for (int e = 0; e < E; ++e) s += expf(row[e] - m);
    sm[tid] = m;
    sinv[tid] = 1.0f / s;
    const float lse = m + logf(s);
    slse2[tid] = lse * lse;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float acc = 0.0f;
    for (int t = 0; t < ntok; ++t) acc += expf(logits[(t0 + t) * E + e] - sm[t]) * sinv[t];
    part[static_cast<int64_t>(blockIdx.x) * E + e] = acc;
  }
  if (tid == 0) {
    float z = 0.0f;
    for (int t = 0; t < ntok; ++t) z += slse2[t];
    zpart[blockIdx.x] = z;
  }
}

__global__ __launch_bounds__(256) void stats_final_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ zpart,
                                                          int nblk, const int32_t* __restrict__ count,
                                                          int64_t T, int E, int k, float alpha,
                                                          float* __restrict__ f,
                                                          float* __restrict__ P,
                                                          float* __restrict__ loss,
                                                          float* __restrict__ zloss) {
  __shared__ double fp[256];
  const int tid = threadIdx.x;
  double term = 0.0;
  if (tid < E) {
    double acc = 0.0;
    for (int b = 0; b < nblk; ++b) acc += part[static_cast<int64_t>(b) * E + tid];
    const double pe = acc / static_cast<double>(T);
    const double fe = static_cast<double>(count[tid]) / (static_cast<double>(T) * k);
    P[tid] = static_cast<float>(pe);
    f[tid] = static_cast<float>(fe);
    term = fe * pe;
  }
  fp[tid] = term;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) fp[tid] += fp[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    loss[0] = static_cast<float>(static_cast<double>(alpha) * E * fp[0]);
    if (zloss) {
      double z = 0.0;
      for (int b = 0; b < nblk; ++b) z += zpart[b];
      zloss[0] = static_cast<float>(z / static_cast<double>(T));
    }
  }
}

}  // namespace

int64_t stats_blocks(int64_t T) { return (T + kTok - 1) / kTok; }

hipError_t launch_balance_stats(const float* logits, const int32_t* count, int64_t T, int E, int k,
                                float alpha, float* f, float* P, float* loss, float* zloss,
                                float* part, float* zpart, hipStream_t stream) {
  const int64_t nblk = stats_blocks(T);
  stats_partial_kernel<<<static_cast<unsigned>(nblk), 256, 0, stream>>>(logits, T, E, part, zpart);
  stats_final_kernel<<<1, 256, 0, stream>>>(part, zpart, static_cast<int>(nblk), count, T, E, k,
                                            alpha, f, P, loss, zloss);
  return hipGetLastError();
}

}  // namespace moe
