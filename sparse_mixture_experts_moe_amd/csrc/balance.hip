// Per-step load-balancing updates from the routed counts of the last step.
//
//   select_bias[e] += step * sign(T k - E count[e])        (float32 add)
//   fbar[e]  = beta fbar[e] + (1 - beta) f[e],  f[e] = count[e] / (T k)
//   C_e      = cf_base + gamma (fbar[e] - 1 / E)            (float64)
//   capacity[e] = clamp(ceil(C_e T k / E), 0, T)
//
// Sources: "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
// section "Auxiliary-Loss-Free Load Balancing" (a per-expert bias moved after
// each step against the expert's load deviation: overloaded experts down,
// underloaded up); "Zen MoDE: Mixture of Distilled Experts Architecture",
// section "Adaptive Capacity Factors" (C_e(t) = C_base + gamma (fbar_e -
// 1/N_E) from a rolling load statistic).
//
// Every value is an exactly specified sequence of IEEE operations (the
// direction of the bias step in integer arithmetic, the rest one rounded
// operation at a time with contraction into FMAs switched off), so the
// results are reproducible bit for bit on any IEEE implementation.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {


namespace {

__global__ __launch_bounds__(256) void balance_update_kernel(
    const int32_t* __restrict__ count, int64_t T, int k, int E, float* __restrict__ select_bias,
    float bias_step, float* __restrict__ f_bar, float decay, double cf_base, double gamma,
    int32_t* __restrict__ capacity) {
  // one IEEE operation at a time, each rounded to nearest: no contraction
  // into fused multiply-adds (the intrinsics' own definitions would allow it)
#pragma clang fp contract(off)
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const int64_t c = count[e];
  const int64_t pairs = T * k;
  if (select_bias) {
    const int64_t dev = pairs - static_cast<int64_t>(E) * c;  // target - load, times E
    const float sgn = dev > 0 ? 1.0f : (dev < 0 ? -1.0f : 0.0f);
    const float delta = bias_step * sgn;
    select_bias[e] = select_bias[e] + delta;
  }
  const float f = static_cast<float>(static_cast<double>(c) / static_cast<double>(pairs));
  const float keep = decay * f_bar[e];
  const float take = (1.0f - decay) * f;
  const float fb = keep + take;
  f_bar[e] = fb;
  if (capacity) {
    const double inv_e = 1.0 / static_cast<double>(E);
    const double dev_e = static_cast<double>(fb) - inv_e;
    const double scaled = gamma * dev_e;
    const double ce = cf_base + scaled;
    const double num = ce * static_cast<double>(pairs);
    const double q = num / static_cast<double>(E);
    const int64_t cap = q <= 0.0 ? 0 : (q >= static_cast<double>(T) ? T : static_cast<int64_t>(ceil(q)));
    capacity[e] = static_cast<int32_t>(cap);
  }
}

}  // namespace

hipError_t launch_balance_update(const int32_t* count, int64_t T, int k, int E, float* select_bias,
                                 float bias_step, float* f_bar, float decay, double cf_base,
                                 double gamma, int32_t* capacity, hipStream_t stream) {
  balance_update_kernel<<<(E + 255) / 256, 256, 0, stream>>>(count, T, k, E, select_bias,
                                                             bias_step, f_bar, decay, cf_base,
                                                             gamma, capacity);
  return hipGetLastError();
}

}  // namespace moe
