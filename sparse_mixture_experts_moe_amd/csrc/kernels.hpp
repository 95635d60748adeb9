// Internal launch interface between the C-ABI layer (libmoe_api.hip) and the
// kernel translation units.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Raises a kernel's dynamic-LDS limit to `bytes` once per (kernel, device);
// later calls are a lock-free lookup (libmoe_api.hip).
void ensure_dynamic_lds(const void* kernel, int bytes);

constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 32;

// route.hip
size_t route_lds_bytes(int E, int k);
size_t route_workspace_bytes(int64_t T, int d, int E, bool bf16);
hipError_t launch_route(const void* x, const void* w, bool bf16, int64_t T, int d, int E, int k,
                        const float* logit_bias, const float* select_bias, bool logits_in,
                        bool prob_keys, bool relu, float* logits, int32_t* topk_idx,
                        float* topk_gate, void* ws, hipStream_t stream);

// permute.hip
int64_t permute_chunks(int64_t R);
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);
hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int64_t cap,
                          const int32_t* cap_e, const void* x, int elem_bytes, int d,
                          int32_t* count, int32_t* offset,
                          int32_t* pair_row, int32_t* row_pair, void* x_perm,
                          int32_t* local_rank, int32_t* hist, hipStream_t stream);

// grouped_gemm.hip
struct SwigluArgs {
  const void* a;
  bool bf16;
  int d, h, G;
  const int32_t* group_offset;
  int64_t max_rows;
  const int32_t* a_rows;
  int a_div;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* y;
  bool y_bf16;
  void* hid;        // [max_rows, h] in the compute dtype
  void* uv;         // gate/up only: [max_rows, 2h] pre-activations kept (interleaved), or NULL
  int32_t* mstart;  // workspace: tile table (tile_table_bytes(G))
  float* sk_ws;     // workspace: split-K partial tiles (down projection), or NULL
  int max_cus;      // bf16 tiled GEMMs: persistent workgroups at most (<= 0: one per compute unit)
};
// bytes of the split-K partial-tile workspace of the down projection
size_t split_k_workspace_bytes();
size_t tile_table_bytes(int G);  // tile table, XCD runs and work counters of the grouped GEMMs
// compute units of the current device (cached per device), 0 if unknown
int compute_units();
hipError_t launch_gate_up(const SwigluArgs& args, hipStream_t stream);
hipError_t launch_down(const SwigluArgs& args, hipStream_t stream);

// backward pass of the experts (bf16)
struct SwigluBwdArgs {
  const void* a;
  bool bf16;                // else fp32 (every tensor below in the same dtype)
  int d, h, G;
  const int32_t* group_offset;
  int64_t max_rows;
  const int32_t* a_rows;
  int a_div;
  const void* dout;         // [max_rows, d] upstream gradient of each row's expert output
  const void* uv;           // [max_rows, 2h] pre-activations of the forward
  const void* hid;          // [max_rows, h] hidden activation of the forward
  const void* w_gate;       // [G, h, d]
  const void* w_up;         // [G, h, d]
  const void* w_down;       // [G, d, h]
  float* da;                // [max_rows, d]
  float* dw_gate;           // [G, h, d]
  float* dw_up;             // [G, h, d]
  float* dw_down;           // [G, d, h]
  // workspace
  int32_t* mstart;          // tile table
  float* sk_ws;             // split-K partial tiles
  uint16_t* zero;           // [max(d, 2h)] zeros
  uint16_t* xs;             // [max_rows, d] gathered rows (when a_rows is given)
  void* dab;                // [max_rows, 2h] interleaved (du, dv)
};
hipError_t launch_expert_backward(const SwigluBwdArgs& args, hipStream_t stream);

// combine.hip
hipError_t launch_combine(const void* y, bool y_bf16, const int32_t* pair_row, const float* gate,
                          int64_t T, int k, int d, const void* shared, void* out, bool out_bf16,
                          hipStream_t stream);
// Zero-computation experts of moe_combine_bypass (router ids past e_ffn:
// n_zero zero, n_copy copy, n_const constant experts; x and const_rows in the
// dtype of y).
struct BypassArgs {
  const int32_t* topk_idx;
  int e_ffn, n_zero, n_copy, n_const;
  const void* x;
  const void* const_rows;
};
hipError_t launch_combine_bypass(const void* y, bool y_bf16, const int32_t* pair_row,
                                 const float* gate, int64_t T, int k, int d, const void* shared,
                                 void* out, bool out_bf16, const BypassArgs& bp,
                                 hipStream_t stream);

// backward.hip: combine, gate/router and router-linear gradients
hipError_t launch_combine_backward(const void* dy, bool dy_bf16, const void* y, bool y_bf16,
                                   const int32_t* pair_row, const float* gate, int64_t T, int k,
                                   int d, float* dgate, void* dout, hipStream_t stream);
// Zero-computation experts in the backward pass (BypassArgs as in the combine).
hipError_t launch_combine_backward_bypass(const void* dy, bool dy_bf16, const void* y,
                                          bool y_bf16, const int32_t* pair_row, const float* gate,
                                          int64_t T, int k, int d, const BypassArgs& b,
                                          float* dgate, void* dout, hipStream_t stream);
size_t bypass_backward_workspace_bytes(int64_t T, int d, int n_const);
hipError_t launch_bypass_backward(const void* dy, bool dy_bf16, const int32_t* idx,
                                  const float* gate, int64_t T, int k, int d, int e_ffn,
                                  int n_zero, int n_copy, int n_const, float* dx_acc,
                                  float* dconst, void* ws, hipStream_t stream);
hipError_t launch_route_backward(const float* logits, const int32_t* idx, const float* gate,
                                 const float* dgate, const int32_t* count, int64_t T, int E, int k, bool relu,
                                 float alpha, float c_bal, float c_z, float* dlogits,
                                 hipStream_t stream);
size_t router_backward_workspace_bytes(int64_t T, int d, int E);
hipError_t launch_router_backward(const void* x, const void* w_router, bool bf16, const float* dl,
                                  int64_t T, int d, int E, float* dw_router, float* dlogit_bias,
                                  float* dx, bool dx_accumulate, void* ws, hipStream_t stream);

// balance.hip: per-step load-balancing updates
hipError_t launch_balance_update(const int32_t* count, int64_t T, int k, int E, float* select_bias,
                                 float bias_step, float* f_bar, float decay, double cf_base,
                                 double gamma, int32_t* capacity, hipStream_t stream);

// stats.hip
int64_t stats_blocks(int64_t T);
hipError_t launch_balance_stats(const float* logits, const int32_t* count, int64_t T, int E, int k,
                                float alpha, float* f, float* P, float* loss, float* zloss,
                                float* part, float* zpart, hipStream_t stream);

// measured device ceilings (not part of the layer)
hipError_t launch_mfma_ceiling(const void* src, int blocks, int iters, float* out,
                               hipStream_t stream);
hipError_t launch_read_ceiling(const void* buf, size_t bytes, int blocks, uint32_t* out,
                               hipStream_t stream);

}  // namespace moe
