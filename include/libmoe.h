/*
 * libmoe -- a sparse Mixture-of-Experts feed-forward layer on AMD Instinct
 * MI355X (gfx950): its forward pass, its backward pass, the per-step
 * load-balancing updates and two routing variants.
 *
 * The layer, as the pages define it:
 *   - a linear router gives one logit per expert ("Every parameter, every
 *     token", section "The gating network"; "Zen MoDE: Mixture of Distilled
 *     Experts Architecture", section "Router Architecture", standard router
 *     equation);
 *   - the k largest are kept and their softmax renormalised into gates that
 *     sum to one (same sections);
 *   - an optional per-expert bias moves the selection only ("Zen-Max: Maximum
 *     Capability via Mixture-of-Experts Architecture", section
 *     "Auxiliary-Loss-Free Load Balancing");
 *   - an optional per-expert capacity drops pairs over the budget ("Every
 *     parameter, every token", section "A budget"; "Zen MoDE: Mixture of Distilled Experts
 *     Architecture", section
 *     "Adaptive Capacity Factors");
 *   - each token runs its k SwiGLU experts (Zen-Max, section "Fine-Grained
 *     Expert Architecture", expert equation) plus any always-on shared experts
 *     (same section; "Every parameter, every token", section "A shared
 *     expert"), and the output is the gate-weighted sum ("The gating network");
 *   - the Switch balance statistics f, P and alpha*N*sum(f*P) are emitted
 *     alongside ("Zen MoDE: Mixture of Distilled Experts Architecture", section "Auxiliary
 *     Load Balancing Loss";
 *     "Every parameter, every token", section "A balance penalty").
 *
 * One layer call is five library calls:
 *   moe_route -> moe_permute -> moe_expert_swiglu (routed experts; and once
 *   more for the shared experts, which may run on a second stream from the
 *   start of the call, on part of the chip: moe_expert_swiglu_cus) ->
 *   moe_combine, plus moe_balance_stats.
 * The backward pass, the balancing updates (moe_balance_update,
 * moe_permute_budgets) and the routing variants (MOE_ROUTE_RELU: ReLU
 * routing; moe_combine_bypass: zero, copy and constant experts, "Zen MoDE:
 * Mixture of Diverse Experts", section "Router") are described where they are declared below.
 *   - "Outputs are overwritten, never accumulated into" holds for every call
 *     except where a declaration says "accumulated" (moe_router_backward's
 *     dx on request, moe_bypass_backward's dx_acc).
 *
 * General contract
 *   - Every pointer is a DEVICE pointer unless marked (host).  Buffers are
 *     owned by the caller; the library never allocates or frees memory and
 *     keeps no device state besides its code objects and the static scratch
 *     array of moe_permute_noalloc.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     default stream) and never synchronises.  Device-resident sizes (expert
 *     counts and offsets) stay on the device.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is enqueued and moe_last_error() describes it.
 *     MOE_EINVAL: a required pointer is NULL or a size is out of range.
 *     MOE_EUNSUPPORTED: a shape these kernels do not implement.
 *     MOE_EWORKSPACE: ws_bytes is below the size the *_workspace query gave.
 *     MOE_EHIP: a kernel launch failed (hipGetLastError after the launch).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Outputs are overwritten, never accumulated into.  Inputs are read only.
 *     Inputs, outputs and workspace must not overlap.
 *   - Token count T = 0 is a valid no-op (moe_permute then writes zero counts
 *     and offsets, moe_balance_stats zero statistics).
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs (no floating-point atomics, fixed reduction orders).
 *   - Calls on different streams with different buffers may run concurrently.
 *
 * Layouts (row-major, contiguous)
 *   x         [T, d]          activations, dtype dt
 *   w_router  [E, d]          router rows, dtype dt
 *   w_gate    [G, h, d]       per-expert gate projection (the transpose of the
 *   w_up      [G, h, d]       page's right-multiplied x W form, so every GEMM
 *   w_down    [G, d, h]       operand is contiguous along its reduction axis)
 *   pair p = t*k + j is slot j of token t.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* moe_route flag: skip the router GEMM and read the logits the caller put in
 * `logits` (used to test selection on identical logits). */
#define MOE_ROUTE_LOGITS_IN 1u
/* moe_route flag: the selection key is the routing probability plus the
 * selection bias, key = softmax(logits[t,:])[e] + select_bias[e], as Zen-Max
 * writes it (section "Auxiliary-Loss-Free Load Balancing", s_ij =
 * softmax(x_i W_g)_j + b_j), instead of the default logit plus bias. */
#define MOE_ROUTE_BIAS_ON_PROBS 2u
/* moe_route flag: ReLU routing ("Zen MoDE: Mixture of Diverse Experts", section
 * "Router": ReLU gating
 * gives each token an adaptive number of experts instead of a fixed top-k).
 * Reading: the gate of expert e is max(logits[t,e], 0) with no
 * renormalisation; a token's slots hold, of its k largest logits, those above
 * zero, in descending order (ties to the lower index), topk_gate = the logit;
 * the remaining slots are empty: topk_idx = -1, topk_gate = 0.  k is then the
 * most experts a token may use.  Not combinable with select_bias or
 * MOE_ROUTE_BIAS_ON_PROBS. */
#define MOE_ROUTE_RELU 4u

/* Limits of these kernels (MOE_EUNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 32

/* Version of this interface (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static description of a status code (host string, never NULL). */
const char* moe_status_string(moe_status_t status);

/* Detail of the last failed call on this host thread (host string, never
 * NULL; empty after a successful call). */
const char* moe_last_error(void);

/* Per-expert token budget C = ceil(cf * T * k / E).
 * "Zen MoDE: Mixture of Distilled Experts Architecture", section "Adaptive Capacity
 * Factors": capacity = factor * tokens /
 * experts; "Every parameter, every token", section "A budget": a factor above
 * one leaves slack.  Reading: tokens are counted as routed pairs T*k, and the
 * quotient is rounded up.  cf is read as the shortest decimal that
 * round-trips to the double (1.1 means 11/10) and the product is rounded up
 * exactly, in integer arithmetic.  Returns -1 (unlimited) for cf <= 0 or a
 * non-finite cf, -2 for T < 0, k < 1 or E < 1; saturates at INT64_MAX. */
int64_t moe_capacity(double cf, int64_t T, int k, int E);

/* ------------------------------------------------------------------------ */
/* moe_route: router logits, top-k selection and renormalised gates.
 *
 *   logits[t,e] = sum_i x[t,i] * w_router[e,i] + logit_bias[e]      (fp32)
 *   key[t,e]    = logits[t,e] + select_bias[e]   (one fp32 add, RNE)
 *   topk_idx[t] = the k experts with the largest keys, in descending key
 *                 order; equal keys go to the lower expert index (for both
 *                 membership and order)
 *   topk_gate[t,j] = exp(l_j - m) / sum_{i in topk} exp(l_i - m), l the
 *                 logits WITHOUT select_bias, m their maximum over the set.
 * Sources: "Every parameter, every token", section "The gating network";
 * "Zen MoDE: Mixture of Distilled Experts Architecture", section "Router Architecture";
 * Zen-Max, section
 * "Auxiliary-Loss-Free Load Balancing" (bias moves the choice only).
 *
 * x [T,d], w_router [E,d] in dtype dt; products accumulate in fp32.
 * logit_bias [E] fp32 or NULL: part of the logits (the gates and
 *   moe_balance_stats see it).
 * select_bias [E] fp32 or NULL: selection key only.
 * flags: MOE_ROUTE_LOGITS_IN reads `logits` instead of computing them
 *   (x and w_router may then be NULL; logit_bias is ignored);
 *   MOE_ROUTE_BIAS_ON_PROBS selects on key = p[t,e] + select_bias[e] with
 *   p[t,:] = softmax(logits[t,:]) over all E experts (fp32: p_e =
 *   exp(l_e - m) / sum, m the row maximum; then one fp32 add), same ties
 *   and order rule; the gates are unchanged.
 * logits [T,E] fp32 out (in with LOGITS_IN); topk_idx [T,k] int32 out;
 * topk_gate [T,k] fp32 out.
 * Limits: 1 <= k <= E <= MOE_MAX_EXPERTS, k <= MOE_MAX_TOPK; for bf16
 * d % 32 == 0.  Logits must be finite.
 * Workspace: moe_route_workspace(T, d, E, k, dt) bytes (partial sums when the
 * reduction over d is split across waves for small batches; 0 when it is not
 * and with MOE_ROUTE_LOGITS_IN).
 */
size_t moe_route_workspace(int64_t T, int d, int E, int k, moe_dtype_t dt);
moe_status_t moe_route(const void* x, const void* w_router, moe_dtype_t dt, int64_t T, int d, int E,
                       int k, const float* logit_bias, const float* select_bias,
                       unsigned flags, float* logits, int32_t* topk_idx, float* topk_gate,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_permute: group the routed pairs by expert, apply the capacity drop,
 * and (optionally) gather the token rows into expert order.
 *
 *   count[e]    = #{p : topk_idx[p] == e}               (before any drop)
 *   rank(p)     = #{p' < p : topk_idx[p'] == topk_idx[p]}  (token order)
 *   kept(p)     = capacity < 0 || rank(p) < capacity
 *   offset      = exclusive prefix sum of min(count[e], capacity), [E+1]
 *   pair_row[p] = offset[e] + rank(p) if kept(p) else -1
 *   row_pair[r] = the pair at row r for r < offset[E], -1 for r >= offset[E]
 *   x_perm[r,:] = x[row_pair[r] / k, :] for r < offset[E] (rows past offset[E]
 *                 are left untouched)
 * Sources: "Every parameter, every token", sections "A budget" (pairs past
 * the budget are dropped and continue through the residual) and "What you
 * still pay for" (a token travels to its assigned expert).  Reading: an
 * expert keeps its first `capacity` pairs in token order.
 *
 * topk_idx [T,k] int32; a slot whose expert lies outside [0,E) (the empty
 * slots of MOE_ROUTE_RELU hold -1) is not routed: it is not counted, takes
 * no budget and gets pair_row -1.  capacity < 0 means unlimited.
 * x [T,d] in dtype dt, or NULL to skip the gather (x_perm then unused).
 * Outputs (int32): expert_count [E], expert_offset [E+1], pair_row [T*k],
 * row_pair [T*k]; x_perm [T*k, d] dtype dt.
 * Workspace: moe_permute_workspace(T, k, E) bytes.
 */
size_t moe_permute_workspace(int64_t T, int k, int E);
moe_status_t moe_permute(const int32_t* topk_idx, int64_t T, int k, int E, int64_t capacity,
                         const void* x, moe_dtype_t dt, int d, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* pair_row, int32_t* row_pair,
                         void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_permute_noalloc: moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Arguments, results and
 * errors are those of moe_permute; the workspace is instead a static device
 * array of the library (5 MiB per device, held until the process ends), so
 * T*k may be at most 1048576 pairs (MOE_EUNSUPPORTED beyond) and E at most
 * MOE_MAX_EXPERTS.  The call allocates nothing.  Every call on a device
 * shares that device's array: calls that overlap on one device (concurrent
 * streams, several host threads) race and must be serialised by the caller.
 * The first call on a device looks up the array's device address (with that
 * device current); a failure there returns MOE_EHIP. */
moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int k, int E,
                                 int64_t capacity, const void* x, moe_dtype_t dt, int d,
                                 int32_t* expert_count, int32_t* expert_offset,
                                 int32_t* pair_row, int32_t* row_pair, void* x_perm,
                                 void* stream);

/* moe_permute_budgets: moe_permute with one budget per expert,
 *   kept(p) = rank(p) < expert_capacity[topk_idx[p]]
 * (expert_capacity [E] int32 on the device, each >= 0; everything else as
 * moe_permute).  Source: "Zen MoDE: Mixture of Distilled Experts Architecture", section
 * "Adaptive Capacity Factors"
 * (capacity per expert); the budgets typically come from moe_balance_update. */
moe_status_t moe_permute_budgets(const int32_t* topk_idx, int64_t T, int k, int E,
                                 const int32_t* expert_capacity, const void* x, moe_dtype_t dt,
                                 int d, int32_t* expert_count, int32_t* expert_offset,
                                 int32_t* pair_row, int32_t* row_pair, void* x_perm, void* ws,
                                 size_t ws_bytes, void* stream);

/* moe_balance_update: the per-step load-balancing updates, from the pre-drop
 * counts of the last step (expert_count of moe_permute, T tokens, k slots):
 *   select_bias[e] += bias_step * sign(T k - E expert_count[e])   (float32)
 *       (an overloaded expert's selection bias falls, an underloaded one's
 *       rises; unchanged at the mean load), if select_bias is not NULL;
 *   load_ema[e] = ema_decay * load_ema[e] + (1 - ema_decay) * f[e],
 *       f[e] = expert_count[e] / (T k) (each product and the sum rounded to
 *       float32, f rounded once from the exact quotient);
 *   expert_capacity[e] = clamp(ceil(C_e T k / E), 0, T) with
 *       C_e = cf_base + gamma (load_ema[e] - 1/E) on the updated load_ema,
 *       in float64, if expert_capacity is not NULL.
 * Sources: Zen-Max, section "Auxiliary-Loss-Free Load Balancing" (bias moved
 * after each step against the load deviation); "Zen MoDE: Mixture of Distilled Experts
 * Architecture", section "Adaptive
 * Capacity Factors" (C_e(t) = C_base + gamma (fbar_e - 1/N_E) from rolling
 * load statistics).  The pages give neither the step size, the rolling
 * window nor gamma: they are the arguments (ema_decay in [0, 1]; 0 uses this
 * step's load alone).  Every operation is a fixed IEEE sequence: results are
 * bit-reproducible.  select_bias, load_ema [E] fp32 in/out; expert_count [E]
 * int32; expert_capacity [E] int32 out. */
moe_status_t moe_balance_update(const int32_t* expert_count, int64_t T, int k, int E,
                                float* select_bias, float bias_step, float* load_ema,
                                float ema_decay, double cf_base, double gamma,
                                int32_t* expert_capacity, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_expert_swiglu: G SwiGLU experts over contiguous row groups.
 *
 * For each group g and each row r in [group_offset[g], group_offset[g+1]):
 *   u       = a[r] . w_gate[g]^T,  v = a[r] . w_up[g]^T           ([h])
 *   hid     = SiLU(u) * v,  SiLU(z) = z / (1 + exp(-z))
 *   y[r]    = hid . w_down[g]^T                                   ([d])
 * Source: Zen-Max, section "Fine-Grained Expert Architecture", expert
 * equation (SiLU(x W_gate) * x W_up) W_down.  Shared experts are one call
 * with G = 1, group_offset = {0, T}, a = x, and the shared experts' weights
 * concatenated along the hidden axis (sum_s SwiGLU_s = SwiGLU of the
 * concatenation, exactly).
 *
 * a [max_rows, d] in dtype dt; weights in dtype dt; products accumulate in
 * fp32; the hidden activation is stored in dtype dt (bf16: rounded to nearest
 * even).  group_offset [G+1] int32 on the device, non-decreasing, with
 * group_offset[0] == 0 and group_offset[G] <= max_rows (host bound).
 * y [max_rows, d] in dtype y_dt (rows past group_offset[G] untouched).
 * Limits: bf16 needs d % 64 == 0, h % 64 == 0 and 2 d h < 2^32 (one
 * expert's weight matrix addressed with 32-bit offsets), else
 * MOE_EUNSUPPORTED.
 * Workspace: moe_expert_swiglu_workspace(max_rows, d, h, G, dt) bytes.
 *
 * moe_expert_swiglu_gather: the same with the rows read through an index,
 *   a_r = a[r]                       if a_rows == NULL
 *       = a[a_rows[r] / a_rows_div]  otherwise (token rows straight from x
 *         through moe_permute's row_pair, a_rows_div = k),
 * a_rows [max_rows] int32 or NULL, a_rows_div >= 1 (MOE_EINVAL otherwise).
 */
size_t moe_expert_swiglu_workspace(int64_t max_rows, int d, int h, int G, moe_dtype_t dt);
moe_status_t moe_expert_swiglu(const void* a, moe_dtype_t dt, int d, int h, int G,
                               const int32_t* group_offset, int64_t max_rows, const void* w_gate,
                               const void* w_up, const void* w_down, void* y, moe_dtype_t y_dt,
                               void* ws, size_t ws_bytes, void* stream);
moe_status_t moe_expert_swiglu_gather(const void* a, moe_dtype_t dt, int d, int h, int G,
                                      const int32_t* group_offset, int64_t max_rows,
                                      const int32_t* a_rows, int a_rows_div,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes,
                                      void* stream);

/* moe_expert_swiglu_cus: moe_expert_swiglu_gather whose tiled bf16 GEMMs run
 * as persistent launches of at most max_cus workgroups (one per compute unit;
 * rounded down to a multiple of 8, at least 8; max_cus <= 0 or at least the
 * device's compute units: all of them), so that work enqueued on another
 * stream at the same time keeps the other compute units.  A layer starts its
 * shared experts this way on a second stream with the call, beside the
 * routing, which then still finds free compute units.  Only the launch width
 * changes: the tile order, its split among the XCDs and the split along K
 * follow the device's compute-unit count, so y is bit-identical to
 * moe_expert_swiglu_gather's.  The fp32 path and the few-row weight stream
 * (groups averaging at most 64 rows) ignore max_cus.  Same source, arguments,
 * limits and workspace as moe_expert_swiglu_gather. */
moe_status_t moe_expert_swiglu_cus(const void* a, moe_dtype_t dt, int d, int h, int G,
                                   const int32_t* group_offset, int64_t max_rows,
                                   const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                   const void* w_up, const void* w_down, void* y,
                                   moe_dtype_t y_dt, void* ws, size_t ws_bytes, int max_cus,
                                   void* stream);

/* The two halves of moe_expert_swiglu_gather, for callers that keep the
 * hidden activation or time the two expert GEMMs apart (same sources, limits
 * and row-group semantics as moe_expert_swiglu_gather).
 *
 * moe_expert_gate_up: hid[r, :] = SiLU(a_r . w_gate[g]^T) * (a_r . w_up[g]^T)
 *   for r < group_offset[G]; hid [max_rows, h] in dtype dt (rows past
 *   group_offset[G] untouched).
 * moe_expert_down:    y[r, :] = hid[r, :] . w_down[g]^T; y [max_rows, d] in
 *   y_dt.
 * Workspace: moe_expert_group_workspace(G) bytes for moe_expert_gate_up,
 * moe_expert_down_workspace(G) bytes for moe_expert_down (today the same
 * size): a tile table and 64 MiB of fp32 partial sums.  Work that would leave
 * compute units idle is split along K (the last round of output tiles of a
 * long-K GEMM; a few-row group whose weight slabs alone are too few waves,
 * such as a shared expert at decode) and the parts are added in a fixed order
 * afterwards, so results stay deterministic.  The workspace contents need no
 * initialisation and are dead after the call. */
size_t moe_expert_group_workspace(int G);
size_t moe_expert_down_workspace(int G);
moe_status_t moe_expert_gate_up(const void* a, moe_dtype_t dt, int d, int h, int G,
                                const int32_t* group_offset, int64_t max_rows,
                                const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                const void* w_up, void* hid, void* ws, size_t ws_bytes,
                                void* stream);
moe_status_t moe_expert_down(const void* hid, moe_dtype_t dt, int d, int h, int G,
                             const int32_t* group_offset, int64_t max_rows, const void* w_down,
                             void* y, moe_dtype_t y_dt, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_combine: gate-weighted sum of the kept expert rows plus the shared
 * output.
 *
 *   out[t,:] = shared_y[t,:] + sum_{j : pair_row[t*k+j] >= 0}
 *                                topk_gate[t,j] * y_perm[pair_row[t*k+j], :]
 * summed in fp32 in slot order j = 0..k-1, then the shared term, then
 * rounded once to out_dt.  A dropped pair contributes nothing and the other
 * gates are not renormalised.  The residual is NOT added.
 * Sources: "Every parameter, every token", sections "The gating network"
 * (y = g1 Expert1(x) + g2 Expert2(x)), "A budget" and "A shared expert";
 * Zen-Max, section "Fine-Grained Expert Architecture" (shared experts added).
 *
 * y_perm [*, d] in y_dt; pair_row [T*k] int32; topk_gate [T,k] fp32, or
 * NULL for gates of 1 (the backward pass sums a token's input gradients
 * this way); shared_y [T,d] in y_dt or NULL; out [T,d] in out_dt.
 */
moe_status_t moe_combine(const void* y_perm, moe_dtype_t y_dt, const int32_t* pair_row,
                         const float* topk_gate, int64_t T, int k, int d,
                         const void* shared_y, void* out, moe_dtype_t out_dt, void* stream);

/* moe_combine_bypass: moe_combine for a router whose experts past the first
 * E_ffn are zero-computation experts ("Zen MoDE: Mixture of Diverse Experts",
 * section "Router": zero,
 * copy and constant experts let a token skip the FFN compute).  Router ids
 * E_ffn .. E_ffn+n_zero-1 are zero experts, the next n_copy copy experts, the
 * next n_const constant experts.  Slot j of token t adds, in slot order,
 *   topk_gate[t,j] * y_perm[pair_row[t*k+j], :]   if topk_idx[t,j] < E_ffn
 *                                                 and pair_row >= 0,
 *   nothing                                       for a zero expert,
 *   topk_gate[t,j] * x[t, :]                      for a copy expert,
 *   topk_gate[t,j] * const_rows[c, :]             for constant expert c,
 * then the shared term, rounded once (readings: zero outputs 0, copy outputs
 * its input, constant c outputs a fixed row v_c; the gates are the plain
 * top-k softmax over all router experts).  The FFN experts' rows come from
 * moe_permute_budgets with a budget of 0 for the zero-computation experts,
 * so they take no rows; their pair_row is not read.
 * topk_idx [T,k] int32; x [T,d] and const_rows [n_const,d] in y_dt (x may be
 * NULL when n_copy == 0, const_rows when n_const == 0); other arguments as
 * moe_combine.  Ids at or past E_ffn+n_zero+n_copy+n_const contribute
 * nothing. */
moe_status_t moe_combine_bypass(const void* y_perm, moe_dtype_t y_dt, const int32_t* pair_row,
                                const int32_t* topk_idx, const float* topk_gate, int64_t T,
                                int k, int d, int E_ffn, int n_zero, int n_copy, int n_const,
                                const void* x, const void* const_rows, const void* shared_y,
                                void* out, moe_dtype_t out_dt, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_balance_stats(_z): Switch balance statistics and the router z-loss.
 *
 *   f[e]  = expert_count[e] / (T * k)       (pre-drop counts; sum f = 1)
 *   P[e]  = (1/T) sum_t softmax(logits[t,:])[e]
 *   loss  = alpha * E * sum_e f[e] * P[e]
 *   zloss = (1/T) sum_t (log sum_e exp logits[t,e])^2
 * Sources: "Zen MoDE: Mixture of Distilled Experts Architecture", section "Auxiliary Load
 * Balancing Loss" (f counts
 * membership in TopK, P the average routing probability, alpha = 0.01);
 * "Every parameter, every token", section "A balance penalty"; Zen-Max,
 * section "MoE-Specific Training Stability" (router z-loss).  Readings:
 * f is normalised by T*k so that uniform routing gives loss = alpha for any
 * k; P uses the full softmax of the logits (logit_bias included, selection
 * bias excluded); N = E.
 *
 * logits [T,E] fp32; expert_count [E] int32; outputs fp32: f [E], P [E],
 * loss [1]; moe_balance_stats_z also writes zloss [1] (zloss may be NULL
 * there).  Sums are fixed-order.
 * Workspace: moe_balance_stats_workspace(T, E) bytes (both calls).
 */
size_t moe_balance_stats_workspace(int64_t T, int E);
moe_status_t moe_balance_stats(const float* logits, const int32_t* expert_count, int64_t T,
                               int E, int k, float alpha, float* f, float* P, float* loss,
                               void* ws, size_t ws_bytes, void* stream);
moe_status_t moe_balance_stats_z(const float* logits, const int32_t* expert_count, int64_t T,
                                 int E, int k, float alpha, float* f, float* P, float* loss,
                                 float* zloss, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Backward pass.
 *
 * The objective differentiated is J = <dy, y> + coef_balance * loss +
 * coef_z * zloss, with y the layer output, dy its upstream gradient and
 * loss, zloss the outputs of moe_balance_stats_z.  Sources: "Every parameter,
 * every token", section "The gating network" (the selected set is held fixed
 * on the way forward; gradient reaches the router only through the gate
 * weights of the experts that ran; an expert that was off for a token gets no
 * gradient from it), sections "A balance penalty" (router trained on the
 * task and the penalty together) and "A budget" (a dropped pair skips its
 * expert update); "Zen MoDE: Mixture of Distilled Experts Architecture", section
 * "Auxiliary Load Balancing Loss"; Zen-Max,
 * sections "Fine-Grained Expert Architecture" and "MoE-Specific Training
 * Stability".  Readings: no gradient flows through the selection, the
 * capacity drop, the counts f or the selection bias; a dropped pair's gate
 * gets no gradient from the output but stays in the renormalising softmax.
 *
 * A layer step: moe_expert_gate_up_train + moe_expert_down (forward, keeping
 * the pre-activations uv, the hidden activation hid and the expert rows
 * y_perm), then
 *   moe_combine_backward        dgate, and dout = gate * dy per kept row
 *   moe_route_backward          dlogits
 *   moe_expert_swiglu_backward  routed experts (dout rows, a = x gathered
 *                               through row_pair) and shared experts (dout = dy)
 *   moe_router_backward         router weights, logit bias, dx (accumulate)
 *   moe_combine(da_perm, NULL gates, shared_y = the accumulated dx) -> dx
 * Every gradient output is fp32 and written (not accumulated) unless stated.
 * The bf16 expert kernels keep u, v and du, dv in bf16 (rounded to nearest
 * even) between GEMMs.
 */

/* moe_expert_gate_up_train: moe_expert_gate_up that also keeps the
 * pre-activations for the backward pass, interleaved per hidden unit:
 *   uv[r, 2c] = a_r . w_gate[g][c],  uv[r, 2c + 1] = a_r . w_up[g][c]
 * uv [max_rows, 2h] in dtype dt.  The bf16 path runs the tiled kernel at
 * every row count.  Workspace: moe_expert_group_workspace(G). */
moe_status_t moe_expert_gate_up_train(const void* a, moe_dtype_t dt, int d, int h, int G,
                                      const int32_t* group_offset, int64_t max_rows,
                                      const int32_t* a_rows, int a_rows_div, const void* w_gate,
                                      const void* w_up, void* hid, void* uv, void* ws,
                                      size_t ws_bytes, void* stream);

/* moe_expert_swiglu_backward: gradients of G SwiGLU experts over row groups
 * (same group semantics, gather and limits as moe_expert_swiglu_gather).  For row r
 * of group g with a_r = a[a_rows[r] / a_rows_div] (or a[r]) and dout_r the
 * upstream gradient of the row's expert output (gate already applied):
 *   u, v    = uv[r, 0::2], uv[r, 1::2]    (from moe_expert_gate_up_train)
 *   hid_r   = hid[r]                       (SiLU(u) * v, from the same call)
 *   dhid    = dout_r . w_down[g]                                 ([h])
 *   du      = dhid * v * SiLU'(u),  dv = dhid * SiLU(u)
 *   da[r]   = du . w_gate[g] + dv . w_up[g]                      ([d], fp32)
 *   dw_gate[g] = sum_r du_r^T a_r,  dw_up[g] = sum_r dv_r^T a_r  ([h, d], fp32)
 *   dw_down[g] = sum_r dout_r^T hid_r                            ([d, h], fp32)
 * with SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z).  A group without rows
 * gets zero weight gradients.  The weights are the forward's (w_gate, w_up
 * [G, h, d], w_down [G, d, h]); the kernels read them along their leading
 * axis directly (no transposed copies).  Routed experts: a = x, a_rows =
 * row_pair, a_rows_div = k, dout from moe_combine_backward.  Shared experts:
 * a = x, a_rows = NULL, dout = dy, G = 1 (concatenated hidden axis).
 * bf16 additionally needs 4 d h < 2^32 (fp32 runs plain FMA tiles).  dout,
 * uv, hid in dt with rows
 * in group order ([max_rows, *]); da [max_rows, d] fp32 (rows past
 * group_offset[G] untouched).
 * Workspace: moe_expert_swiglu_backward_workspace(max_rows, d, h, G, dt,
 * a_rows != NULL) bytes (tile table, split-K partials, a zero row, the
 * gathered rows of a when a_rows is given, and du, dv interleaved in bf16: about
 * 2 max_rows (2h + d) bytes plus 64 MiB); contents need no initialisation
 * and are dead after the call. */
size_t moe_expert_swiglu_backward_workspace(int64_t max_rows, int d, int h, int G, moe_dtype_t dt,
                                            int gather);
moe_status_t moe_expert_swiglu_backward(const void* a, moe_dtype_t dt, int d, int h, int G,
                                        const int32_t* group_offset, int64_t max_rows,
                                        const int32_t* a_rows, int a_rows_div, const void* dout,
                                        const void* uv, const void* hid, const void* w_gate,
                                        const void* w_up, const void* w_down, float* da,
                                        float* dw_gate, float* dw_up, float* dw_down, void* ws,
                                        size_t ws_bytes, void* stream);

/* moe_combine_backward: the gate gradients of the combine,
 *   dgate[t, j] = sum_i dy[t, i] * y_perm[pair_row[t*k+j], i]   (fp32)
 * and 0 for a dropped pair (pair_row < 0); with dout non-NULL also the
 * upstream gradient of every kept expert row,
 *   dout[pair_row[t*k+j], :] = topk_gate[t, j] * dy[t, :]       (dy_dt)
 * Source: "The gating network" (y = sum_j g_j Expert_j(x)).  dy [T, d] in
 * dy_dt; y_perm [*, d] in y_dt (the expert rows moe_expert_down wrote);
 * topk_gate [T, k] fp32 (needed with dout); dgate [T, k] fp32; dout [*, d]
 * or NULL (rows of dropped pairs do not exist; other rows untouched). */
moe_status_t moe_combine_backward(const void* dy, moe_dtype_t dy_dt, const void* y_perm,
                                  moe_dtype_t y_dt, const int32_t* pair_row,
                                  const float* topk_gate, int64_t T, int k, int d, float* dgate,
                                  void* dout, void* stream);

/* moe_route_backward: dJ/dlogits [T, E] fp32,
 *   dl[t,e] = g_tj (dgate_tj - sum_i g_ti dgate_ti)    for e = topk_idx[t,j]
 *           + coef_balance * alpha * E / T * p_te (f_e - sum_e' f_e' p_te')
 *           + coef_z * (2 / T) * lse_t * p_te
 * with g = topk_gate (the forward's gates), p_t = softmax(logits[t,:]),
 * lse_t = log sum_e exp logits[t,e], f_e = expert_count[e] / (T k) (the
 * pre-drop counts of moe_permute).  Sources: "The gating network" (softmax
 * over the selected set), "Zen MoDE: Mixture of Distilled Experts Architecture" "Auxiliary
 * Load Balancing Loss", Zen-Max
 * "MoE-Specific Training Stability".  expert_count may be NULL when
 * coef_balance == 0.
 * flags: 0, or MOE_ROUTE_RELU for the ReLU-routed forward (its gate is the
 * logit on a used slot, so the gate term becomes dl[t,e] = dgate_tj for
 * e = topk_idx[t,j] >= 0; empty slots (-1) contribute nothing; the balance
 * and z-loss terms are unchanged, k being the most experts per token). */
/* moe_combine_backward_bypass: moe_combine_backward for the layer with
 * zero-computation experts (the forward's moe_combine_bypass; same router
 * numbering).  dgate[t,j] = <dy[t], out_j> with out_j the slot's output row:
 * y_perm[pair_row] for an FFN slot that ran, x[t] for a copy expert, the
 * constant row for a constant expert, nothing (dgate 0) for a zero expert,
 * a dropped pair or an id past the last; dout (optional) as
 * moe_combine_backward, for the FFN slots that ran.  x and const_rows in
 * y_dt.  Source: "Zen MoDE: Mixture of Diverse Experts", section "Router"
 * (zero-computation experts). */
moe_status_t moe_combine_backward_bypass(const void* dy, moe_dtype_t dy_dt,
                                         const void* y_perm, moe_dtype_t y_dt,
                                         const int32_t* pair_row, const int32_t* topk_idx,
                                         const float* topk_gate, int64_t T, int k, int d,
                                         int E_ffn, int n_zero, int n_copy, int n_const,
                                         const void* x, const void* const_rows, float* dgate,
                                         void* dout, void* stream);

/* moe_bypass_backward: the rest of the zero-computation experts' backward,
 *   dx_acc[t,:] += (sum of topk_gate[t,j] over t's copy slots) * dy[t,:]
 *   dconst[c,:]  = sum over the slots on constant expert c of topk_gate * dy
 * dx_acc [T,d] fp32 (accumulated; may be NULL when n_copy == 0), dconst
 * [n_const,d] fp32 (written; may be NULL when n_const == 0), summed over
 * fixed token ranges added in range order (deterministic).  Workspace:
 * moe_bypass_backward_workspace(T, d, n_const) bytes. */
size_t moe_bypass_backward_workspace(int64_t T, int d, int n_const);
moe_status_t moe_bypass_backward(const void* dy, moe_dtype_t dy_dt, const int32_t* topk_idx,
                                 const float* topk_gate, int64_t T, int k, int d, int E_ffn,
                                 int n_zero, int n_copy, int n_const, float* dx_acc, float* dconst,
                                 void* ws, size_t ws_bytes, void* stream);

moe_status_t moe_route_backward(const float* logits, const int32_t* topk_idx,
                                const float* topk_gate, const float* dgate,
                                const int32_t* expert_count, int64_t T, int E, int k,
                                unsigned flags, float alpha, float coef_balance, float coef_z,
                                float* dlogits, void* stream);

/* moe_router_backward: gradients of logits = x w_router^T + logit_bias:
 *   dw_router[e, i] = sum_t dlogits[t, e] x[t, i]       [E, d] fp32
 *   dlogit_bias[e]  = sum_t dlogits[t, e]                [E]    fp32
 *   dx[t, i]        = (accumulate_dx ? dx[t, i] : 0) + sum_e dlogits[t, e] w_router[e, i]
 * x, w_router in dtype dt; dx [T, d] fp32.  Any of dw_router, dlogit_bias,
 * dx may be NULL (not computed).  Sums over tokens go through fixed
 * per-chunk partials (deterministic).  Source: "The gating network" (a
 * linear gate).  Workspace: moe_router_backward_workspace(T, d, E) bytes
 * (only when dw_router is requested). */
size_t moe_router_backward_workspace(int64_t T, int d, int E);
moe_status_t moe_router_backward(const void* x, const void* w_router, moe_dtype_t dt,
                                 const float* dlogits, int64_t T, int d, int E, float* dw_router,
                                 float* dlogit_bias, float* dx, int accumulate_dx, void* ws,
                                 size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement probes: what the device sustains, for roofline fractions
 * against a measured ceiling beside the datasheet peaks.  They compute
 * nothing of the layer.
 *
 * moe_probe_mfma_bf16: `blocks` workgroups of 256 threads (each holds more
 * than half of a CU's LDS, so one runs per CU; pass the CU count to cover
 * the chip).  Every lane loads 8 fragments of 8 bf16 from src[lane * 64 ..]
 * (src holds blocks * 256 * 64 bf16, e.g. random normals: the operands'
 * bit patterns set the power drawn and so the clock), then each wave issues
 * iters * 16 v_mfma_f32_32x32x16_bf16 on them, 32768 FLOP each, with no
 * memory traffic.  out [blocks * 256] fp32 receives each lane's accumulator
 * sum.  FLOP per launch: blocks * 4 * iters * 16 * 32768.
 *
 * moe_probe_read: reads bytes (a positive multiple of 16) of buf once, in
 * 16-byte loads spread over `blocks` workgroups of 256 threads (grid
 * stride); out [blocks * 256] uint32 receives each lane's XOR of what it
 * read.  Bytes per launch: bytes.
 */
moe_status_t moe_probe_mfma_bf16(const void* src, int blocks, int iters, float* out,
                                 void* stream);
moe_status_t moe_probe_read(const void* buf, size_t bytes, int blocks, uint32_t* out,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
