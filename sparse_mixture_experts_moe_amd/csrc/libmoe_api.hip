// C-ABI of libmoe: argument checks, workspace layout and kernel launches.
// The operations and their sources are documented in include/libmoe.h.
#include "../../include/libmoe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <charconv>
#include <mutex>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.hpp"

namespace moe {

int compute_units() {
  static std::atomic<int> cache[64];  // per device, 0 = not yet known
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

void ensure_dynamic_lds(const void* kernel, int bytes) {
  // (kernel, device, bytes) triples already applied; a short fixed table suffices
  // (a handful of kernels times the visible devices)
  struct Entry {
    std::atomic<const void*> fn{nullptr};
    std::atomic<int> dev{-1};
    std::atomic<int> bytes{0};
  };
  static Entry table[256];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  for (auto& e : table) {
    const void* f = e.fn.load(std::memory_order_acquire);
    if (f == nullptr) break;
    if (f == kernel && e.dev.load() == dev && e.bytes.load() >= bytes) return;
  }
  std::lock_guard<std::mutex> lock(mu);
  (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  for (auto& e : table) {
    if (e.fn.load() == nullptr) {
      e.dev.store(dev);
      e.bytes.store(bytes);
      e.fn.store(kernel, std::memory_order_release);
      return;
    }
    if (e.fn.load() == kernel && e.dev.load() == dev) {
      if (e.bytes.load() < bytes) e.bytes.store(bytes);
      return;
    }
  }
}

}  // namespace moe

namespace {

thread_local char g_err[512];

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool valid_dtype(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
int elem_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or type";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_capacity(double cf, int64_t T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return -2;
  if (!std::isfinite(cf) || cf <= 0.0) return -1;
  if (T == 0) return 0;
  // shortest round-trip decimal of cf: digits * 10^exp10
  char buf[64];
  const auto res = std::to_chars(buf, buf + sizeof(buf), cf);
  *res.ptr = '\0';
  unsigned __int128 digits = 0;
  int exp10 = 0;
  bool frac = false;
  const char* p = buf;
  for (; *p && *p != 'e' && *p != 'E'; ++p) {
    if (*p == '.') {
      frac = true;
      continue;
    }
    digits = digits * 10 + static_cast<unsigned>(*p - '0');
    if (frac) --exp10;
  }
  if (*p == 'e' || *p == 'E') exp10 += static_cast<int>(strtol(p + 1, nullptr, 10));
  const unsigned __int128 pairs = static_cast<unsigned __int128>(T) * static_cast<unsigned>(k);
  if (pairs > (static_cast<unsigned __int128>(1) << 64)) return INT64_MAX;
  unsigned __int128 num = digits * pairs;  // < 2^57 * 2^64
  unsigned __int128 den = static_cast<unsigned>(E);
  const unsigned __int128 kCap = static_cast<unsigned __int128>(1) << 125;
  if (exp10 >= 0) {
    for (int i = 0; i < exp10; ++i) {
      if (num > kCap / 10) return INT64_MAX;
      num *= 10;
    }
  } else {
    // the divisor E * 10^-exp10 exceeds num once 10^-exp10 > num: budget 1
    for (int i = 0; i < -exp10; ++i) {
      if (den > num) return 1;
      den *= 10;
    }
  }
  const unsigned __int128 c = (num + den - 1) / den;
  if (c > static_cast<unsigned __int128>(INT64_MAX)) return INT64_MAX;
  return static_cast<int64_t>(c);
}

// ---------------------------------------------------------------------------
size_t moe_route_workspace(int64_t T, int d, int E, int k, moe_dtype_t dt) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || !valid_dtype(dt)) return 0;
  if (E > moe::kMaxExperts || d % 32 != 0) return 0;
  return moe::route_workspace_bytes(T, d, E, dt == MOE_BF16);
}

moe_status_t moe_route(const void* x, const void* w_router, moe_dtype_t dt, int64_t T, int d, int E,
                       int k, const float* logit_bias, const float* select_bias,
                       unsigned flags, float* logits, int32_t* topk_idx, float* topk_gate,
                       void* ws, size_t ws_bytes, void* stream) {
  const bool logits_in = (flags & MOE_ROUTE_LOGITS_IN) != 0;
  const bool prob_keys = (flags & MOE_ROUTE_BIAS_ON_PROBS) != 0;
  const bool relu = (flags & MOE_ROUTE_RELU) != 0;
  if (flags & ~(MOE_ROUTE_LOGITS_IN | MOE_ROUTE_BIAS_ON_PROBS | MOE_ROUTE_RELU))
    return fail(MOE_EINVAL, "moe_route: unknown flags 0x%x", flags);
  if (relu && (prob_keys || select_bias))
    return fail(MOE_EINVAL, "moe_route: ReLU routing takes no selection bias");
  if (T < 0) return fail(MOE_EINVAL, "moe_route: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_route: need 1 <= k <= E");
  if (!valid_dtype(dt)) return fail(MOE_EINVAL, "moe_route: bad dtype %d", dt);
  if (!logits_in && d < 1) return fail(MOE_EINVAL, "moe_route: d < 1");
  if (E > moe::kMaxExperts) return fail(MOE_EUNSUPPORTED, "moe_route: E > %d", moe::kMaxExperts);
  if (k > moe::kMaxTopK) return fail(MOE_EUNSUPPORTED, "moe_route: k > %d", moe::kMaxTopK);
  if (!logits_in && dt == MOE_BF16 && d % 32 != 0)
    return fail(MOE_EUNSUPPORTED, "moe_route: bf16 needs d %% 32 == 0");
  if (T == 0) return ok();  // per-token buffers of zero size may be NULL
  if (!logits || !topk_idx || !topk_gate)
    return fail(MOE_EINVAL, "moe_route: NULL output pointer");
  if (!logits_in && (!x || !w_router)) return fail(MOE_EINVAL, "moe_route: NULL x or w_router");
  const size_t need = logits_in ? 0 : moe::route_workspace_bytes(T, d, E, dt == MOE_BF16);
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_EWORKSPACE, "moe_route: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(moe::launch_route(x, w_router, dt == MOE_BF16, T, d, E, k, logit_bias,
                                      select_bias, logits_in, prob_keys, relu, logits, topk_idx,
                                      topk_gate, ws, as_stream(stream)),
                    "moe_route");
}

// ---------------------------------------------------------------------------
size_t moe_permute_workspace(int64_t T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const int64_t R = T * k;
  return align256(sizeof(int32_t) * static_cast<size_t>(R)) +
         align256(sizeof(int32_t) * static_cast<size_t>(moe::permute_chunks(R)) * E);
}

moe_status_t moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, int64_t capacity,
                         const void* x, moe_dtype_t dt, int d, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* pair_row, int32_t* row_pair,
                         void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_permute: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_permute: need 1 <= k <= E");
  if (!expert_count || !expert_offset) return fail(MOE_EINVAL, "moe_permute: NULL pointer");
  if (T > 0 && (!topk_idx || !pair_row || !row_pair))
    return fail(MOE_EINVAL, "moe_permute: NULL pointer");
  if (x && (!x_perm || d < 1 || !valid_dtype(dt)))
    return fail(MOE_EINVAL, "moe_permute: gather needs x_perm, d >= 1 and a valid dtype");
  if (E > moe::kMaxExperts) return fail(MOE_EUNSUPPORTED, "moe_permute: E > %d", moe::kMaxExperts);
  if (T * k > INT32_MAX) return fail(MOE_EUNSUPPORTED, "moe_permute: T*k exceeds int32");
  const size_t need = moe_permute_workspace(T, k, E);
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_EWORKSPACE, "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
  if (T == 0) {
    // no pairs: counts and offsets are all zero
    hipError_t e = moe::launch_fill_i32(expert_count, E, 0, as_stream(stream));
    if (e == hipSuccess) e = moe::launch_fill_i32(expert_offset, E + 1, 0, as_stream(stream));
    return hip_status(e, "moe_permute");
  }
  int32_t* local_rank = static_cast<int32_t*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             align256(sizeof(int32_t) * static_cast<size_t>(T * k)));
  return hip_status(moe::launch_permute(topk_idx, T, k, E, capacity, nullptr, x, elem_bytes(dt), d,
                                        expert_count, expert_offset, pair_row, row_pair, x_perm,
                                        local_rank, hist, as_stream(stream)),
                    "moe_permute");
}

}  // extern "C"

namespace {

// Scratch of moe_permute_noalloc: moe_permute's workspace (the local ranks,
// int32 [T k], then the per-chunk histograms, int32 [chunks, E]) for at most
// kNoAllocMaxPairs pairs and kMaxExperts experts, 5 MiB.  Each device that
// runs the library holds its own copy until the process ends.  Every word a
// call reads is written earlier in the same call, so nothing needs clearing.
constexpr int64_t kNoAllocMaxPairs = int64_t{1} << 20;
constexpr size_t kNoAllocRankBytes = sizeof(int32_t) * static_cast<size_t>(kNoAllocMaxPairs);
constexpr size_t kNoAllocScratchBytes =
    kNoAllocRankBytes +
    sizeof(int32_t) * static_cast<size_t>((kNoAllocMaxPairs + 1023) / 1024) * moe::kMaxExperts;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of this device's `scratch` (in host code the array's name is
// only a stand-in, not a device address), looked up once per device with that
// device current.  nullptr with `err` set if the lookup fails.
void* scratch_address(hipError_t& err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E,
                                 int64_t capacity, const void* x, moe_dtype_t dt, int d,
                                 int32_t* expert_count, int32_t* expert_offset,
                                 int32_t* pair_row, int32_t* row_pair, void* x_perm,
                                 void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_permute_noalloc: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_permute_noalloc: need 1 <= k <= E");
  if (!expert_count || !expert_offset) return fail(MOE_EINVAL, "moe_permute_noalloc: NULL pointer");
  if (T > 0 && (!topk_idx || !pair_row || !row_pair))
    return fail(MOE_EINVAL, "moe_permute_noalloc: NULL pointer");
  if (x && (!x_perm || d < 1 || !valid_dtype(dt)))
    return fail(MOE_EINVAL, "moe_permute_noalloc: gather needs x_perm, d >= 1 and a valid dtype");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_permute_noalloc: E > %d", moe::kMaxExperts);
  if (T > kNoAllocMaxPairs || T * k > kNoAllocMaxPairs)
    return fail(MOE_EUNSUPPORTED,
                "moe_permute_noalloc: T*k = %lld pairs exceeds the static scratch (%lld pairs)",
                static_cast<long long>(T) * k, static_cast<long long>(kNoAllocMaxPairs));
  hipError_t e = hipSuccess;
  if (T == 0) {
    e = moe::launch_fill_i32(expert_count, E, 0, as_stream(stream));
    if (e == hipSuccess) e = moe::launch_fill_i32(expert_offset, E + 1, 0, as_stream(stream));
    return hip_status(e, "moe_permute_noalloc");
  }
  if (static_cast<size_t>(moe::permute_chunks(T * k)) * E * sizeof(int32_t) >
      kNoAllocScratchBytes - kNoAllocRankBytes)
    return fail(MOE_EUNSUPPORTED, "moe_permute_noalloc: histograms exceed the static scratch");
  void* ws = scratch_address(e);
  if (!ws) return hip_status(e, "moe_permute_noalloc: hipGetSymbolAddress(scratch)");
  int32_t* local_rank = static_cast<int32_t*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + kNoAllocRankBytes);
  return hip_status(moe::launch_permute(topk_idx, T, k, E, capacity, nullptr, x, elem_bytes(dt), d,
                                        expert_count, expert_offset, pair_row, row_pair, x_perm,
                                        local_rank, hist, as_stream(stream)),
                    "moe_permute_noalloc");
}

moe_status_t moe_permute_budgets(const int32_t* topk_idx, int64_t T, int k, int E,
                                 const int32_t* expert_capacity, const void* x, moe_dtype_t dt,
                                 int d, int32_t* expert_count, int32_t* expert_offset,
                                 int32_t* pair_row, int32_t* row_pair, void* x_perm, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!expert_capacity) return fail(MOE_EINVAL, "moe_permute_budgets: NULL expert_capacity");
  if (T < 0) return fail(MOE_EINVAL, "moe_permute_budgets: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_permute_budgets: need 1 <= k <= E");
  if (!expert_count || !expert_offset) return fail(MOE_EINVAL, "moe_permute_budgets: NULL pointer");
  if (T > 0 && (!topk_idx || !pair_row || !row_pair))
    return fail(MOE_EINVAL, "moe_permute_budgets: NULL pointer");
  if (x && (!x_perm || d < 1 || !valid_dtype(dt)))
    return fail(MOE_EINVAL, "moe_permute_budgets: gather needs x_perm, d >= 1 and a valid dtype");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_permute_budgets: E > %d", moe::kMaxExperts);
  if (T * k > INT32_MAX) return fail(MOE_EUNSUPPORTED, "moe_permute_budgets: T*k exceeds int32");
  const size_t need = moe_permute_workspace(T, k, E);
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_EWORKSPACE, "moe_permute_budgets: workspace %zu < %zu bytes", ws_bytes, need);
  if (T == 0) {
    hipError_t e = moe::launch_fill_i32(expert_count, E, 0, as_stream(stream));
    if (e == hipSuccess) e = moe::launch_fill_i32(expert_offset, E + 1, 0, as_stream(stream));
    return hip_status(e, "moe_permute_budgets");
  }
  int32_t* local_rank = static_cast<int32_t*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             align256(sizeof(int32_t) * static_cast<size_t>(T * k)));
  return hip_status(moe::launch_permute(topk_idx, T, k, E, -1, expert_capacity, x,
                                        elem_bytes(dt), d, expert_count, expert_offset, pair_row,
                                        row_pair, x_perm, local_rank, hist, as_stream(stream)),
                    "moe_permute_budgets");
}

moe_status_t moe_balance_update(const int32_t* expert_count, int64_t T, int k, int E,
                                float* select_bias, float bias_step, float* load_ema,
                                float ema_decay, double cf_base, double gamma,
                                int32_t* expert_capacity, void* stream) {
  if (T < 1 || k < 1 || E < 1 || k > E)
    return fail(MOE_EINVAL, "moe_balance_update: need T >= 1 and 1 <= k <= E");
  if (!expert_count || !load_ema) return fail(MOE_EINVAL, "moe_balance_update: NULL pointer");
  if (!std::isfinite(bias_step) || !std::isfinite(ema_decay) || !std::isfinite(cf_base) ||
      !std::isfinite(gamma))
    return fail(MOE_EINVAL, "moe_balance_update: non-finite step, decay, cf_base or gamma");
  if (ema_decay < 0.0f || ema_decay > 1.0f)
    return fail(MOE_EINVAL, "moe_balance_update: ema_decay outside [0, 1]");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_balance_update: E > %d", moe::kMaxExperts);
  if (T > INT32_MAX || T * k > (int64_t{1} << 53))
    return fail(MOE_EUNSUPPORTED, "moe_balance_update: T too large");
  return hip_status(moe::launch_balance_update(expert_count, T, k, E, select_bias, bias_step,
                                               load_ema, ema_decay, cf_base, gamma,
                                               expert_capacity, as_stream(stream)),
                    "moe_balance_update");
}

// ---------------------------------------------------------------------------
namespace {

moe_status_t check_experts(const char* fn, int dt, int d, int h, int G, int64_t max_rows,
                           const int32_t* group_offset) {
  if (d < 1 || h < 1 || G < 1 || max_rows < 0)
    return fail(MOE_EINVAL, "%s: need d, h, G >= 1 and max_rows >= 0", fn);
  if (!valid_dtype(dt)) return fail(MOE_EINVAL, "%s: dtype", fn);
  if (!group_offset) return fail(MOE_EINVAL, "%s: NULL group_offset", fn);
  if (dt == MOE_BF16 && (d % 64 != 0 || h % 64 != 0))
    return fail(MOE_EUNSUPPORTED, "%s: bf16 needs d %% 64 == 0 and h %% 64 == 0", fn);
  if (dt == MOE_BF16 && static_cast<int64_t>(d) * h * 2 > static_cast<int64_t>(UINT32_MAX))
    return fail(MOE_EUNSUPPORTED, "%s: bf16 expert weight matrix over 4 GiB", fn);
  if (max_rows > INT32_MAX || static_cast<int64_t>(G) * (max_rows + 1) > INT32_MAX)
    return fail(MOE_EUNSUPPORTED, "%s: too many rows", fn);
  return MOE_OK;
}

size_t tile_table_bytes(int G) { return align256(moe::tile_table_bytes(G)); }

}  // namespace

size_t moe_expert_group_workspace(int G) {
  return G < 1 ? 0 : tile_table_bytes(G) + moe::split_k_workspace_bytes();
}

size_t moe_expert_down_workspace(int G) {
  return G < 1 ? 0 : tile_table_bytes(G) + moe::split_k_workspace_bytes();
}

size_t moe_expert_swiglu_workspace(int64_t max_rows, int d, int h, int G, moe_dtype_t dt) {
  if (max_rows < 0 || d < 1 || h < 1 || G < 1 || !valid_dtype(dt)) return 0;
  return align256(static_cast<size_t>(max_rows) * h * elem_bytes(dt)) +
         moe_expert_down_workspace(G);
}

namespace {

moe_status_t gate_up_call(const void* a, moe_dtype_t dt, int d, int h, int G,
                          const int32_t* group_offset, int64_t max_rows, const int32_t* a_rows,
                          int a_rows_div, const void* w_gate, const void* w_up, void* hid,
                          void* ws, size_t ws_bytes, int max_cus, void* stream) {
  moe_status_t st = check_experts("moe_expert_gate_up", dt, d, h, G, max_rows, group_offset);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return ok();  // no rows: buffers of zero size may be NULL
  if (!a || !w_gate || !w_up || !hid) return fail(MOE_EINVAL, "moe_expert_gate_up: NULL pointer");
  if (a_rows && a_rows_div < 1) return fail(MOE_EINVAL, "moe_expert_gate_up: a_rows_div < 1");
  if (ws_bytes < moe_expert_group_workspace(G) || !ws)
    return fail(MOE_EWORKSPACE, "moe_expert_gate_up: workspace %zu < %zu bytes", ws_bytes,
                moe_expert_group_workspace(G));
  moe::SwigluArgs s{};
  s.a = a;
  s.bf16 = dt == MOE_BF16;
  s.d = d;
  s.h = h;
  s.G = G;
  s.group_offset = group_offset;
  s.max_rows = max_rows;
  s.a_rows = a_rows;
  s.a_div = a_rows ? a_rows_div : 1;
  s.w_gate = w_gate;
  s.w_up = w_up;
  s.hid = hid;
  s.mstart = static_cast<int32_t*>(ws);
  s.sk_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + tile_table_bytes(G));
  s.max_cus = max_cus;
  return hip_status(moe::launch_gate_up(s, as_stream(stream)), "moe_expert_gate_up");
}

moe_status_t down_call(const void* hid, moe_dtype_t dt, int d, int h, int G,
                       const int32_t* group_offset, int64_t max_rows, const void* w_down, void* y,
                       moe_dtype_t y_dt, void* ws, size_t ws_bytes, int max_cus, void* stream) {
  moe_status_t st = check_experts("moe_expert_down", dt, d, h, G, max_rows, group_offset);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return ok();  // no rows: buffers of zero size may be NULL
  if (!valid_dtype(y_dt)) return fail(MOE_EINVAL, "moe_expert_down: dtype");
  if (!hid || !w_down || !y) return fail(MOE_EINVAL, "moe_expert_down: NULL pointer");
  if (ws_bytes < moe_expert_down_workspace(G) || !ws)
    return fail(MOE_EWORKSPACE, "moe_expert_down: workspace %zu < %zu bytes", ws_bytes,
                moe_expert_down_workspace(G));
  moe::SwigluArgs s{};
  s.bf16 = dt == MOE_BF16;
  s.d = d;
  s.h = h;
  s.G = G;
  s.group_offset = group_offset;
  s.max_rows = max_rows;
  s.w_down = w_down;
  s.y = y;
  s.y_bf16 = y_dt == MOE_BF16;
  s.hid = const_cast<void*>(hid);
  s.mstart = static_cast<int32_t*>(ws);
  s.sk_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + tile_table_bytes(G));
  s.max_cus = max_cus;
  return hip_status(moe::launch_down(s, as_stream(stream)), "moe_expert_down");
}

moe_status_t swiglu_call(const void* a, moe_dtype_t dt, int d, int h, int G,
                         const int32_t* group_offset, int64_t max_rows, const int32_t* a_rows,
                         int a_rows_div, const void* w_gate, const void* w_up,
                         const void* w_down, void* y, moe_dtype_t y_dt, void* ws,
                         size_t ws_bytes, int max_cus, void* stream) {
  moe_status_t st = check_experts("moe_expert_swiglu", dt, d, h, G, max_rows, group_offset);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return ok();  // no rows: buffers of zero size may be NULL
  if (!valid_dtype(y_dt)) return fail(MOE_EINVAL, "moe_expert_swiglu: dtype");
  if (!a || !w_gate || !w_up || !w_down || !y)
    return fail(MOE_EINVAL, "moe_expert_swiglu: NULL pointer");
  if (a_rows && a_rows_div < 1) return fail(MOE_EINVAL, "moe_expert_swiglu: a_rows_div < 1");
  const size_t need = moe_expert_swiglu_workspace(max_rows, d, h, G, dt);
  if (ws_bytes < need || !ws)
    return fail(MOE_EWORKSPACE, "moe_expert_swiglu: workspace %zu < %zu bytes", ws_bytes, need);
  const size_t hid_bytes = align256(static_cast<size_t>(max_rows) * h * elem_bytes(dt));
  void* hid = ws;
  void* table = static_cast<char*>(ws) + hid_bytes;
  st = gate_up_call(a, dt, d, h, G, group_offset, max_rows, a_rows, a_rows_div, w_gate, w_up,
                    hid, table, ws_bytes - hid_bytes, max_cus, stream);
  if (st != MOE_OK) return st;
  return down_call(hid, dt, d, h, G, group_offset, max_rows, w_down, y, y_dt, table,
                   ws_bytes - hid_bytes, max_cus, stream);
}

}  // namespace

moe_status_t moe_expert_gate_up(const void* a, moe_dtype_t dt, int d, int h, int G,
                                const int32_t* group_offset, int64_t max_rows,
                                const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                const void* w_up, void* hid, void* ws, size_t ws_bytes,
                                void* stream) {
  return gate_up_call(a, dt, d, h, G, group_offset, max_rows, a_rows, a_rows_div, w_gate, w_up,
                      hid, ws, ws_bytes, 0, stream);
}

moe_status_t moe_expert_down(const void* hid, moe_dtype_t dt, int d, int h, int G,
                             const int32_t* group_offset, int64_t max_rows, const void* w_down,
                             void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes, void* stream) {
  return down_call(hid, dt, d, h, G, group_offset, max_rows, w_down, y, y_dt, ws, ws_bytes, 0,
                   stream);
}

moe_status_t moe_expert_swiglu_gather(const void* a, moe_dtype_t dt, int d, int h, int G,
                                      const int32_t* group_offset, int64_t max_rows,
                                      const int32_t* a_rows, int a_rows_div,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes,
                                      void* stream) {
  return swiglu_call(a, dt, d, h, G, group_offset, max_rows, a_rows, a_rows_div, w_gate, w_up,
                     w_down, y, y_dt, ws, ws_bytes, 0, stream);
}

moe_status_t moe_expert_swiglu_cus(const void* a, moe_dtype_t dt, int d, int h, int G,
                                   const int32_t* group_offset, int64_t max_rows,
                                   const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                   const void* w_up, const void* w_down, void* y,
                                   moe_dtype_t y_dt, void* ws, size_t ws_bytes, int max_cus,
                                   void* stream) {
  return swiglu_call(a, dt, d, h, G, group_offset, max_rows, a_rows, a_rows_div, w_gate, w_up,
                     w_down, y, y_dt, ws, ws_bytes, max_cus, stream);
}

moe_status_t moe_expert_swiglu(const void* a, moe_dtype_t dt, int d, int h, int G,
                               const int32_t* group_offset, int64_t max_rows, const void* w_gate,
                               const void* w_up, const void* w_down, void* y, moe_dtype_t y_dt,
                               void* ws, size_t ws_bytes, void* stream) {
  return moe_expert_swiglu_gather(a, dt, d, h, G, group_offset, max_rows, nullptr, 1, w_gate,
                                  w_up, w_down, y, y_dt, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
moe_status_t moe_combine(const void* y_perm, moe_dtype_t y_dt, const int32_t* pair_row,
                         const float* topk_gate, int64_t T, int k, int d,
                         const void* shared_y, void* out, moe_dtype_t out_dt, void* stream) {
  if (T < 0 || k < 1 || d < 1) return fail(MOE_EINVAL, "moe_combine: need T >= 0, k >= 1, d >= 1");
  if (!valid_dtype(y_dt) || !valid_dtype(out_dt)) return fail(MOE_EINVAL, "moe_combine: dtype");
  if (T == 0) return ok();
  if (!y_perm || !pair_row || !out) return fail(MOE_EINVAL, "moe_combine: NULL pointer");
  return hip_status(moe::launch_combine(y_perm, y_dt == MOE_BF16, pair_row, topk_gate, T, k, d,
                                        shared_y, out, out_dt == MOE_BF16, as_stream(stream)),
                    "moe_combine");
}

moe_status_t moe_combine_bypass(const void* y_perm, moe_dtype_t y_dt, const int32_t* pair_row,
                                const int32_t* topk_idx, const float* topk_gate, int64_t T,
                                int k, int d, int E_ffn, int n_zero, int n_copy, int n_const,
                                const void* x, const void* const_rows, const void* shared_y,
                                void* out, moe_dtype_t out_dt, void* stream) {
  if (T < 0 || k < 1 || d < 1)
    return fail(MOE_EINVAL, "moe_combine_bypass: need T >= 0, k >= 1, d >= 1");
  if (E_ffn < 0 || n_zero < 0 || n_copy < 0 || n_const < 0)
    return fail(MOE_EINVAL, "moe_combine_bypass: negative expert count");
  if (static_cast<int64_t>(E_ffn) + n_zero + n_copy + n_const > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_combine_bypass: more than %d router experts",
                moe::kMaxExperts);
  if (!valid_dtype(y_dt) || !valid_dtype(out_dt))
    return fail(MOE_EINVAL, "moe_combine_bypass: dtype");
  if (T == 0) return ok();
  if (!pair_row || !topk_idx || !out || (E_ffn > 0 && !y_perm))
    return fail(MOE_EINVAL, "moe_combine_bypass: NULL pointer");
  if ((n_copy > 0 && !x) || (n_const > 0 && !const_rows))
    return fail(MOE_EINVAL, "moe_combine_bypass: NULL x or const_rows");
  const moe::BypassArgs bp{topk_idx, E_ffn, n_zero, n_copy, n_const, x, const_rows};
  return hip_status(moe::launch_combine_bypass(y_perm, y_dt == MOE_BF16, pair_row, topk_gate, T,
                                               k, d, shared_y, out, out_dt == MOE_BF16, bp,
                                               as_stream(stream)),
                    "moe_combine_bypass");
}

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
moe_status_t moe_expert_gate_up_train(const void* a, moe_dtype_t dt, int d, int h, int G,
                                      const int32_t* group_offset, int64_t max_rows,
                                      const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                      const void* w_up, void* hid, void* uv, void* ws,
                                      size_t ws_bytes, void* stream) {
  moe_status_t st = check_experts("moe_expert_gate_up_train", dt, d, h, G, max_rows, group_offset);
  if (st != MOE_OK) return st;
  if (max_rows == 0) return ok();
  if (!a || !w_gate || !w_up || !hid || !uv)
    return fail(MOE_EINVAL, "moe_expert_gate_up_train: NULL pointer");
  if (a_rows && a_rows_div < 1) return fail(MOE_EINVAL, "moe_expert_gate_up_train: a_rows_div < 1");
  if (ws_bytes < moe_expert_group_workspace(G) || !ws)
    return fail(MOE_EWORKSPACE, "moe_expert_gate_up_train: workspace %zu < %zu bytes", ws_bytes,
                moe_expert_group_workspace(G));
  moe::SwigluArgs s{};
  s.a = a;
  s.bf16 = dt == MOE_BF16;
  s.d = d;
  s.h = h;
  s.G = G;
  s.group_offset = group_offset;
  s.max_rows = max_rows;
  s.a_rows = a_rows;
  s.a_div = a_rows ? a_rows_div : 1;
  s.w_gate = w_gate;
  s.w_up = w_up;
  s.hid = hid;
  s.uv = uv;
  s.mstart = static_cast<int32_t*>(ws);
  s.sk_ws = reinterpret_cast<float*>(static_cast<char*>(ws) + tile_table_bytes(G));
  return hip_status(moe::launch_gate_up(s, as_stream(stream)), "moe_expert_gate_up_train");
}

namespace {

struct BwdLayout {
  size_t table, sk, zero, xs, dab, total;
};

BwdLayout bwd_layout(int64_t max_rows, int d, int h, int G, bool gather, bool bf16) {
  BwdLayout L{};
  size_t o = 0;
  L.table = o;
  o += tile_table_bytes(G);
  L.sk = o;
  if (bf16) o += moe::split_k_workspace_bytes();
  L.zero = o;
  if (bf16) o += align256(2 * static_cast<size_t>(d > 2 * h ? d : 2 * h));
  L.xs = o;
  if (bf16 && gather) o += align256(2 * static_cast<size_t>(max_rows) * d);
  L.dab = o;
  o += align256((bf16 ? 2 : 4) * static_cast<size_t>(max_rows) * 2 * h);
  L.total = o;
  return L;
}

}  // namespace

size_t moe_expert_swiglu_backward_workspace(int64_t max_rows, int d, int h, int G, moe_dtype_t dt,
                                            int gather) {
  if (max_rows < 0 || d < 1 || h < 1 || G < 1 || !valid_dtype(dt)) return 0;
  return bwd_layout(max_rows, d, h, G, gather != 0, dt == MOE_BF16).total;
}

moe_status_t moe_expert_swiglu_backward(const void* a, moe_dtype_t dt, int d, int h, int G,
                                        const int32_t* group_offset, int64_t max_rows,
                                        const int32_t* a_rows, int a_rows_div, const void* dout,
                                        const void* uv, const void* hid, const void* w_gate,
                                        const void* w_up, const void* w_down, float* da,
                                        float* dw_gate, float* dw_up, float* dw_down, void* ws,
                                        size_t ws_bytes, void* stream) {
  const char* fn = "moe_expert_swiglu_backward";
  moe_status_t st = check_experts(fn, dt, d, h, G, max_rows, group_offset);
  if (st != MOE_OK) return st;
  if (dt == MOE_BF16 && static_cast<int64_t>(d) * h * 4 > static_cast<int64_t>(UINT32_MAX))
    return fail(MOE_EUNSUPPORTED, "%s: 4 d h over 2^32", fn);
  if (static_cast<int64_t>(G) * ((d + 255) / 256) * ((h + 255) / 256) > INT32_MAX / 2)
    return fail(MOE_EUNSUPPORTED, "%s: too many weight-gradient tiles", fn);
  if (!w_gate || !w_up || !w_down || !dw_gate || !dw_up || !dw_down)
    return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if (max_rows > 0 && (!a || !dout || !uv || !hid || !da))
    return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if (a_rows && a_rows_div < 1) return fail(MOE_EINVAL, "%s: a_rows_div < 1", fn);
  const BwdLayout L = bwd_layout(max_rows, d, h, G, a_rows != nullptr, dt == MOE_BF16);
  if (ws_bytes < L.total || !ws)
    return fail(MOE_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  moe::SwigluBwdArgs b{};
  b.a = a;
  b.bf16 = dt == MOE_BF16;
  b.d = d;
  b.h = h;
  b.G = G;
  b.group_offset = group_offset;
  b.max_rows = max_rows;
  b.a_rows = a_rows;
  b.a_div = a_rows ? a_rows_div : 1;
  b.dout = dout;
  b.uv = uv;
  b.hid = hid;
  b.w_gate = w_gate;
  b.w_up = w_up;
  b.w_down = w_down;
  b.da = da;
  b.dw_gate = dw_gate;
  b.dw_up = dw_up;
  b.dw_down = dw_down;
  b.mstart = reinterpret_cast<int32_t*>(w + L.table);
  b.sk_ws = reinterpret_cast<float*>(w + L.sk);
  b.zero = reinterpret_cast<uint16_t*>(w + L.zero);
  b.xs = (a_rows && dt == MOE_BF16) ? reinterpret_cast<uint16_t*>(w + L.xs) : nullptr;
  b.dab = w + L.dab;
  return hip_status(moe::launch_expert_backward(b, as_stream(stream)), fn);
}

moe_status_t moe_combine_backward(const void* dy, moe_dtype_t dy_dt, const void* y_perm,
                                  moe_dtype_t y_dt, const int32_t* pair_row,
                                  const float* topk_gate, int64_t T, int k, int d, float* dgate,
                                  void* dout, void* stream) {
  if (T < 0 || k < 1 || d < 1)
    return fail(MOE_EINVAL, "moe_combine_backward: need T >= 0, k >= 1, d >= 1");
  if (!valid_dtype(dy_dt) || !valid_dtype(y_dt))
    return fail(MOE_EINVAL, "moe_combine_backward: dtype");
  if (T == 0) return ok();
  if (!dy || !y_perm || !pair_row || !dgate || (dout && !topk_gate))
    return fail(MOE_EINVAL, "moe_combine_backward: NULL pointer");
  return hip_status(moe::launch_combine_backward(dy, dy_dt == MOE_BF16, y_perm, y_dt == MOE_BF16,
                                                 pair_row, topk_gate, T, k, d, dgate, dout,
                                                 as_stream(stream)),
                    "moe_combine_backward");
}

moe_status_t moe_route_backward(const float* logits, const int32_t* topk_idx,
                                const float* topk_gate, const float* dgate,
                                const int32_t* expert_count, int64_t T, int E, int k,
                                unsigned flags, float alpha, float coef_balance, float coef_z,
                                float* dlogits, void* stream) {
  if (flags & ~MOE_ROUTE_RELU) return fail(MOE_EINVAL, "moe_route_backward: unknown flags 0x%x", flags);
  if (T < 0) return fail(MOE_EINVAL, "moe_route_backward: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_route_backward: need 1 <= k <= E");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_route_backward: E > %d", moe::kMaxExperts);
  if (T == 0) return ok();
  if (!logits || !topk_idx || !topk_gate || !dgate || !dlogits ||
      (coef_balance != 0.0f && !expert_count))
    return fail(MOE_EINVAL, "moe_route_backward: NULL pointer");
  return hip_status(moe::launch_route_backward(logits, topk_idx, topk_gate, dgate, expert_count, T,
                                               E, k, (flags & MOE_ROUTE_RELU) != 0, alpha,
                                               coef_balance, coef_z, dlogits, as_stream(stream)),
                    "moe_route_backward");
}

static moe_status_t check_bypass(const char* fn, int64_t T, int k, int d, int E_ffn, int n_zero,
                                 int n_copy, int n_const) {
  if (T < 0 || k < 1 || d < 1) return fail(MOE_EINVAL, "%s: need T >= 0, k >= 1, d >= 1", fn);
  if (E_ffn < 0 || n_zero < 0 || n_copy < 0 || n_const < 0)
    return fail(MOE_EINVAL, "%s: negative expert count", fn);
  if (static_cast<int64_t>(E_ffn) + n_zero + n_copy + n_const > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "%s: more than %d router experts", fn, moe::kMaxExperts);
  return MOE_OK;
}

moe_status_t moe_combine_backward_bypass(const void* dy, moe_dtype_t dy_dt,
                                         const void* y_perm, moe_dtype_t y_dt,
                                         const int32_t* pair_row, const int32_t* topk_idx,
                                         const float* topk_gate, int64_t T, int k, int d,
                                         int E_ffn, int n_zero, int n_copy, int n_const,
                                         const void* x, const void* const_rows, float* dgate,
                                         void* dout, void* stream) {
  const char* fn = "moe_combine_backward_bypass";
  moe_status_t st = check_bypass(fn, T, k, d, E_ffn, n_zero, n_copy, n_const);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dy_dt) || !valid_dtype(y_dt)) return fail(MOE_EINVAL, "%s: dtype", fn);
  if (T == 0) return ok();
  if (!dy || !pair_row || !topk_idx || !dgate || (E_ffn > 0 && !y_perm) || (dout && !topk_gate))
    return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if ((n_copy > 0 && !x) || (n_const > 0 && !const_rows))
    return fail(MOE_EINVAL, "%s: NULL x or const_rows", fn);
  const moe::BypassArgs bp{topk_idx, E_ffn, n_zero, n_copy, n_const, x, const_rows};
  return hip_status(moe::launch_combine_backward_bypass(dy, dy_dt == MOE_BF16, y_perm,
                                                        y_dt == MOE_BF16, pair_row, topk_gate, T, k,
                                                        d, bp, dgate, dout, as_stream(stream)),
                    fn);
}

size_t moe_bypass_backward_workspace(int64_t T, int d, int n_const) {
  if (T < 0 || d < 1 || n_const < 0) return 0;
  return align256(moe::bypass_backward_workspace_bytes(T, d, n_const));
}

moe_status_t moe_bypass_backward(const void* dy, moe_dtype_t dy_dt, const int32_t* topk_idx,
                                 const float* topk_gate, int64_t T, int k, int d, int E_ffn,
                                 int n_zero, int n_copy, int n_const, float* dx_acc, float* dconst,
                                 void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_bypass_backward";
  moe_status_t st = check_bypass(fn, T, k, d, E_ffn, n_zero, n_copy, n_const);
  if (st != MOE_OK) return st;
  if (!valid_dtype(dy_dt)) return fail(MOE_EINVAL, "%s: dtype", fn);
  if (T == 0) return ok();
  if (!dy || !topk_idx || !topk_gate) return fail(MOE_EINVAL, "%s: NULL pointer", fn);
  if ((n_copy > 0 && !dx_acc) || (n_const > 0 && !dconst))
    return fail(MOE_EINVAL, "%s: NULL dx_acc or dconst", fn);
  const size_t need = n_const > 0 ? moe_bypass_backward_workspace(T, d, n_const) : 0;
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return hip_status(moe::launch_bypass_backward(dy, dy_dt == MOE_BF16, topk_idx, topk_gate, T, k, d,
                                                E_ffn, n_zero, n_copy, n_const, dx_acc, dconst, ws,
                                                as_stream(stream)),
                    fn);
}

size_t moe_router_backward_workspace(int64_t T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return 0;
  return align256(moe::router_backward_workspace_bytes(T, d, E));
}

moe_status_t moe_router_backward(const void* x, const void* w_router, moe_dtype_t dt,
                                 const float* dlogits, int64_t T, int d, int E, float* dw_router,
                                 float* dlogit_bias, float* dx, int accumulate_dx, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (T < 0 || d < 1 || E < 1) return fail(MOE_EINVAL, "moe_router_backward: need T >= 0, d, E >= 1");
  if (!valid_dtype(dt)) return fail(MOE_EINVAL, "moe_router_backward: dtype");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_router_backward: E > %d", moe::kMaxExperts);
  if (T == 0) {
    // no tokens: the weight and bias gradients are zero
    hipStream_t s = as_stream(stream);
    hipError_t e = hipSuccess;
    if (dw_router) e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(dw_router), static_cast<int64_t>(E) * d, 0, s);
    if (e == hipSuccess && dlogit_bias) e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(dlogit_bias), E, 0, s);
    return hip_status(e, "moe_router_backward");
  }
  if (!dlogits || (dw_router && !x) || (dx && !w_router))
    return fail(MOE_EINVAL, "moe_router_backward: NULL pointer");
  const size_t need = dw_router ? moe_router_backward_workspace(T, d, E) : 0;
  if (ws_bytes < need || (need && !ws))
    return fail(MOE_EWORKSPACE, "moe_router_backward: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(moe::launch_router_backward(x, w_router, dt == MOE_BF16, dlogits, T, d, E,
                                                dw_router, dlogit_bias, dx, accumulate_dx != 0, ws,
                                                as_stream(stream)),
                    "moe_router_backward");
}

// ---------------------------------------------------------------------------
size_t moe_balance_stats_workspace(int64_t T, int E) {
  if (T < 0 || E < 1) return 0;
  const size_t nb = static_cast<size_t>(moe::stats_blocks(T));
  return align256(sizeof(float) * nb * E) + align256(sizeof(float) * nb);
}

moe_status_t moe_balance_stats_z(const float* logits, const int32_t* expert_count, int64_t T,
                                 int E, int k, float alpha, float* f, float* P, float* loss,
                                 float* zloss, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0) return fail(MOE_EINVAL, "moe_balance_stats: T < 0");
  if (E < 1 || k < 1 || k > E) return fail(MOE_EINVAL, "moe_balance_stats: need 1 <= k <= E");
  if (!expert_count || !f || !P || !loss || (T > 0 && !logits))
    return fail(MOE_EINVAL, "moe_balance_stats: NULL pointer");
  if (E > moe::kMaxExperts)
    return fail(MOE_EUNSUPPORTED, "moe_balance_stats: E > %d", moe::kMaxExperts);
  if (T == 0) {
    // no tokens: every statistic is written as zero
    hipStream_t st = as_stream(stream);
    hipError_t e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(f), E, 0, st);
    if (e == hipSuccess) e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(P), E, 0, st);
    if (e == hipSuccess) e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(loss), 1, 0, st);
    if (e == hipSuccess && zloss) e = moe::launch_fill_i32(reinterpret_cast<int32_t*>(zloss), 1, 0, st);
    return hip_status(e, "moe_balance_stats");
  }
  const size_t need = moe_balance_stats_workspace(T, E);
  if (ws_bytes < need || !ws)
    return fail(MOE_EWORKSPACE, "moe_balance_stats: workspace %zu < %zu bytes", ws_bytes, need);
  const size_t nb = static_cast<size_t>(moe::stats_blocks(T));
  float* part = static_cast<float*>(ws);
  float* zpart = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(sizeof(float) * nb * E));
  return hip_status(moe::launch_balance_stats(logits, expert_count, T, E, k, alpha, f, P, loss,
                                              zloss, part, zpart, as_stream(stream)),
                    "moe_balance_stats");
}

moe_status_t moe_balance_stats(const float* logits, const int32_t* expert_count, int64_t T,
                               int E, int k, float alpha, float* f, float* P, float* loss,
                               void* ws, size_t ws_bytes, void* stream) {
  return moe_balance_stats_z(logits, expert_count, T, E, k, alpha, f, P, loss, nullptr, ws,
                             ws_bytes, stream);
}

// ---------------------------------------------------------------------------
moe_status_t moe_probe_mfma_bf16(const void* src, int blocks, int iters, float* out,
                                 void* stream) {
  if (blocks < 1 || iters < 1) return fail(MOE_EINVAL, "moe_probe_mfma_bf16: blocks, iters >= 1");
  if (!src || !out) return fail(MOE_EINVAL, "moe_probe_mfma_bf16: NULL pointer");
  return hip_status(moe::launch_mfma_ceiling(src, blocks, iters, out, as_stream(stream)),
                    "moe_probe_mfma_bf16");
}

moe_status_t moe_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* out,
                            void* stream) {
  if (blocks < 1 || bytes < 16 || bytes % 16 != 0)
    return fail(MOE_EINVAL, "moe_probe_read: need blocks >= 1 and bytes a positive multiple of 16");
  if (!buf || !out) return fail(MOE_EINVAL, "moe_probe_read: NULL pointer");
  return hip_status(moe::launch_read_ceiling(buf, bytes, blocks, out, as_stream(stream)),
                    "moe_probe_read");
}

}  // extern "C"
