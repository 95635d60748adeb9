"""ctypes binding of libmoe (include/libmoe.h): argument marshalling only.

Each Python function has the name of the C entry point it calls, takes torch
tensors (device tensors for every buffer), allocates the outputs it is not
given, enqueues on the current HIP stream and returns the outputs.  All of the
computation happens in the library's kernels; nothing here falls back to any
other implementation: if the library is missing, importing this module fails.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBMOE_PATH", os.path.join(_HERE, "lib", "libmoe.so"))

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_LOGITS_IN = 1
MOE_ROUTE_BIAS_ON_PROBS = 2
MOE_ROUTE_RELU = 4
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 32


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"libmoe status {status}: {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmoe is not built ({LIB_PATH} missing); run "
            "`python -m sparse_mixture_experts_moe_amd.build`")
    return ctypes.CDLL(LIB_PATH)


_L = _load()

_p, _i, _i64, _sz, _u, _f, _d = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                  ctypes.c_uint, ctypes.c_float, ctypes.c_double)
_SIGS = {
    "moe_abi_version": (_i, []),
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_capacity": (_i64, [_d, _i64, _i, _i]),
    "moe_route_workspace": (_sz, [_i64, _i, _i, _i, _i]),
    "moe_route": (_i, [_p, _p, _i, _i64, _i, _i, _i, _p, _p, _u, _p, _p, _p, _p, _sz, _p]),
    "moe_permute_workspace": (_sz, [_i64, _i, _i]),
    "moe_permute": (_i, [_p, _i64, _i, _i, _i64, _p, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_permute_budgets": (_i, [_p, _i64, _i, _i, _p, _p, _i, _i, _p, _p, _p, _p, _p, _p, _sz,
                                 _p]),
    "moe_permute_noalloc": (_i, [_p, _i64, _i, _i, _i64, _p, _i, _i, _p, _p, _p, _p, _p, _p]),
    "moe_balance_update": (_i, [_p, _i64, _i, _i, _p, _f, _p, _f, _d, _d, _p, _p]),
    "moe_expert_swiglu_workspace": (_sz, [_i64, _i, _i, _i, _i]),
    "moe_expert_swiglu": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _p, _p, _p, _i, _p, _sz, _p]),
    "moe_expert_swiglu_gather": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p, _p, _p, _i,
                                      _p,
                               _sz, _p]),
    "moe_expert_swiglu_cus": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p, _p, _p, _i, _p,
                                   _sz, _i, _p]),
    "moe_expert_group_workspace": (_sz, [_i]),
    "moe_expert_down_workspace": (_sz, [_i]),
    "moe_expert_gate_up": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p, _p, _p, _sz, _p]),
    "moe_expert_down": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _p, _i, _p, _sz, _p]),
    "moe_combine": (_i, [_p, _i, _p, _p, _i64, _i, _i, _p, _p, _i, _p]),
    "moe_combine_bypass": (_i, [_p, _i, _p, _p, _p, _i64, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p,
                                _i, _p]),
    "moe_balance_stats_workspace": (_sz, [_i64, _i]),
    "moe_balance_stats": (_i, [_p, _p, _i64, _i, _i, _f, _p, _p, _p, _p, _sz, _p]),
    "moe_balance_stats_z": (_i, [_p, _p, _i64, _i, _i, _f, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_expert_gate_up_train": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p, _p, _p, _p,
                                      _sz, _p]),
    "moe_expert_swiglu_backward_workspace": (_sz, [_i64, _i, _i, _i, _i, _i]),
    "moe_expert_swiglu_backward": (_i, [_p, _i, _i, _i, _i, _p, _i64, _p, _i, _p, _p, _p, _p, _p,
                                        _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_combine_backward": (_i, [_p, _i, _p, _i, _p, _p, _i64, _i, _i, _p, _p, _p]),
    "moe_combine_backward_bypass": (_i, [_p, _i, _p, _i, _p, _p, _p, _i64, _i, _i, _i, _i, _i, _i,
                                         _p, _p, _p, _p, _p]),
    "moe_bypass_backward_workspace": (_sz, [_i64, _i, _i]),
    "moe_bypass_backward": (_i, [_p, _i, _p, _p, _i64, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz,
                                 _p]),
    "moe_route_backward": (_i, [_p, _p, _p, _p, _p, _i64, _i, _i, _u, _f, _f, _f, _p, _p]),
    "moe_router_backward_workspace": (_sz, [_i64, _i, _i]),
    "moe_router_backward": (_i, [_p, _p, _i, _p, _i64, _i, _i, _p, _p, _p, _i, _p, _sz, _p]),
    "moe_probe_mfma_bf16": (_i, [_p, _i, _i, _p, _p]),
    "moe_probe_read": (_i, [_p, _sz, _i, _p, _p]),
}
EXPORTED = tuple(_SIGS)
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_L, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(status: int):
    if status != MOE_OK:
        raise MoEError(status, _L.moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


_TORCH_DT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libmoe needs contiguous tensors")


# ---------------------------------------------------------------------------
def moe_abi_version() -> int:
    return _L.moe_abi_version()


def moe_status_string(status: int) -> str:
    return _L.moe_status_string(status).decode()


def moe_last_error() -> str:
    return _L.moe_last_error().decode()


def moe_capacity(cf: float, T: int, k: int, E: int) -> int:
    return _L.moe_capacity(float(cf), T, k, E)


def moe_route_workspace(T, d, E, k, dt) -> int:
    return _L.moe_route_workspace(T, d, E, k, dt)


def moe_route(x, w_router, k, logit_bias=None, select_bias=None, *, logits=None, topk_idx=None,
              topk_gate=None, logits_in=False, bias_on_probs=False, relu=False, ws=None,
              stream=None):
    """Router logits, top-k experts and renormalised gates.  With
    ``logits_in`` the given ``logits`` [T, E] are used instead of x W_r^T;
    ``bias_on_probs`` selects on softmax probability + selection bias;
    ``relu`` is ReLU routing (at most k experts with a positive logit, gate =
    logit, empty slots -1 / 0)."""
    if logits_in:
        T, E = logits.shape
        dt, d = MOE_F32, 0
        dev = logits.device
    else:
        T, d = x.shape
        E = w_router.shape[0]
        dt = _dt(x)
        dev = x.device
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_gate is None:
        topk_gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    nws = 0 if logits_in else moe_route_workspace(T, d, E, k, dt)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _contig(x, w_router, logit_bias, select_bias, logits, topk_idx, topk_gate, ws)
    _check(_L.moe_route(_ptr(x), _ptr(w_router), dt, T, d, E, k, _ptr(logit_bias),
                        _ptr(select_bias),
                        (MOE_ROUTE_LOGITS_IN if logits_in else 0) |
                        (MOE_ROUTE_BIAS_ON_PROBS if bias_on_probs else 0) |
                        (MOE_ROUTE_RELU if relu else 0),
                        _ptr(logits), _ptr(topk_idx), _ptr(topk_gate), _ptr(ws), ws.numel(),
                        _stream(stream)))
    return logits, topk_idx, topk_gate


def moe_permute_workspace(T, k, E) -> int:
    return _L.moe_permute_workspace(T, k, E)


def moe_permute(topk_idx, E, capacity=-1, x=None, *, expert_count=None, expert_offset=None,
                pair_row=None, row_pair=None, x_perm=None, ws=None, stream=None):
    """Expert counts, kept offsets, the pair/row permutation and (if ``x`` is
    given) the expert-ordered copy of the token rows."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    R = T * k
    if expert_count is None:
        expert_count = torch.empty(E, dtype=torch.int32, device=dev)
    if expert_offset is None:
        expert_offset = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pair_row is None:
        pair_row = torch.empty(R, dtype=torch.int32, device=dev)
    if row_pair is None:
        row_pair = torch.empty(R, dtype=torch.int32, device=dev)
    dt, d = MOE_F32, 0
    if x is not None:
        dt, d = _dt(x), x.shape[1]
        if x_perm is None:
            x_perm = torch.empty((R, d), dtype=x.dtype, device=dev)
    nws = moe_permute_workspace(T, k, E)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _contig(topk_idx, x, expert_count, expert_offset, pair_row, row_pair, x_perm, ws)
    _check(_L.moe_permute(_ptr(topk_idx), T, k, E, int(capacity), _ptr(x), dt, d,
                          _ptr(expert_count), _ptr(expert_offset), _ptr(pair_row),
                          _ptr(row_pair), _ptr(x_perm), _ptr(ws), ws.numel(), _stream(stream)))
    return expert_count, expert_offset, pair_row, row_pair, x_perm


def moe_permute_noalloc(topk_idx, E, capacity=-1, x=None, *, expert_count=None,
                        expert_offset=None, pair_row=None, row_pair=None, x_perm=None,
                        stream=None):
    """moe_permute with the library's static scratch instead of a workspace
    (the call allocates no device memory; outputs not given are allocated
    here, before it)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    R = T * k
    if expert_count is None:
        expert_count = torch.empty(E, dtype=torch.int32, device=dev)
    if expert_offset is None:
        expert_offset = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pair_row is None:
        pair_row = torch.empty(R, dtype=torch.int32, device=dev)
    if row_pair is None:
        row_pair = torch.empty(R, dtype=torch.int32, device=dev)
    dt, d = MOE_F32, 0
    if x is not None:
        dt, d = _dt(x), x.shape[1]
        if x_perm is None:
            x_perm = torch.empty((R, d), dtype=x.dtype, device=dev)
    _contig(topk_idx, x, expert_count, expert_offset, pair_row, row_pair, x_perm)
    _check(_L.moe_permute_noalloc(_ptr(topk_idx), T, k, E, int(capacity), _ptr(x), dt, d,
                                  _ptr(expert_count), _ptr(expert_offset), _ptr(pair_row),
                                  _ptr(row_pair), _ptr(x_perm), _stream(stream)))
    return expert_count, expert_offset, pair_row, row_pair, x_perm


def moe_permute_budgets(topk_idx, E, expert_capacity, x=None, *, expert_count=None,
                        expert_offset=None, pair_row=None, row_pair=None, x_perm=None, ws=None,
                        stream=None):
    """moe_permute with a per-expert budget (expert_capacity [E] int32 on the device)."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    R = T * k
    if expert_count is None:
        expert_count = torch.empty(E, dtype=torch.int32, device=dev)
    if expert_offset is None:
        expert_offset = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if pair_row is None:
        pair_row = torch.empty(R, dtype=torch.int32, device=dev)
    if row_pair is None:
        row_pair = torch.empty(R, dtype=torch.int32, device=dev)
    dt, d = MOE_F32, 0
    if x is not None:
        dt, d = _dt(x), x.shape[1]
        if x_perm is None:
            x_perm = torch.empty((R, d), dtype=x.dtype, device=dev)
    nws = moe_permute_workspace(T, k, E)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _contig(topk_idx, expert_capacity, x, expert_count, expert_offset, pair_row, row_pair, x_perm,
            ws)
    _check(_L.moe_permute_budgets(_ptr(topk_idx), T, k, E, _ptr(expert_capacity), _ptr(x), dt, d,
                                  _ptr(expert_count), _ptr(expert_offset), _ptr(pair_row),
                                  _ptr(row_pair), _ptr(x_perm), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return expert_count, expert_offset, pair_row, row_pair, x_perm


def moe_balance_update(expert_count, T, k, load_ema, *, select_bias=None, bias_step=0.0,
                       ema_decay=0.0, cf_base=1.0, gamma=0.0, expert_capacity=None,
                       want_capacity=True, stream=None):
    """Per-step updates (in place on select_bias and load_ema); returns the
    per-expert budgets (int32 [E]) when ``want_capacity``."""
    E = expert_count.numel()
    if want_capacity and expert_capacity is None:
        expert_capacity = torch.empty(E, dtype=torch.int32, device=expert_count.device)
    _contig(expert_count, load_ema, select_bias, expert_capacity)
    _check(_L.moe_balance_update(_ptr(expert_count), T, k, E, _ptr(select_bias), float(bias_step),
                                 _ptr(load_ema), float(ema_decay), float(cf_base), float(gamma),
                                 _ptr(expert_capacity), _stream(stream)))
    return expert_capacity


def moe_expert_swiglu_workspace(max_rows, d, h, G, dt) -> int:
    return _L.moe_expert_swiglu_workspace(max_rows, d, h, G, dt)


def moe_expert_swiglu(a, group_offset, max_rows, w_gate, w_up, w_down, *, a_rows=None,
                      a_rows_div=1, y=None, y_dtype=None, ws=None, stream=None, max_cus=0):
    """G SwiGLU experts over contiguous row groups: y[r] = SwiGLU_g(a_r), with
    a_r = a[a_rows[r] // a_rows_div] when ``a_rows`` is given
    (moe_expert_swiglu_gather), else a[r] (moe_expert_swiglu).  ``max_cus`` > 0
    limits the tiled GEMMs' persistent launches to that many workgroups
    (moe_expert_swiglu_cus; same results)."""
    G, h, d = w_gate.shape
    dt = _dt(a)
    dev = a.device
    if y is None:
        y = torch.empty((max_rows, d), dtype=y_dtype or a.dtype, device=dev)
    nws = moe_expert_swiglu_workspace(max_rows, d, h, G, dt)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    _contig(a, group_offset, a_rows, w_gate, w_up, w_down, y, ws)
    if max_cus > 0:
        _check(_L.moe_expert_swiglu_cus(_ptr(a), dt, d, h, G, _ptr(group_offset), max_rows,
                                        _ptr(a_rows), a_rows_div if a_rows is not None else 1,
                                        _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _dt(y),
                                        _ptr(ws), ws.numel(), int(max_cus), _stream(stream)))
    elif a_rows is None:
        _check(_L.moe_expert_swiglu(_ptr(a), dt, d, h, G, _ptr(group_offset), max_rows,
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y), _dt(y),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(_L.moe_expert_swiglu_gather(_ptr(a), dt, d, h, G, _ptr(group_offset), max_rows,
                                           _ptr(a_rows), a_rows_div, _ptr(w_gate), _ptr(w_up),
                                           _ptr(w_down), _ptr(y), _dt(y), _ptr(ws), ws.numel(),
                                           _stream(stream)))
    return y


def moe_expert_group_workspace(G) -> int:
    return _L.moe_expert_group_workspace(G)


def moe_expert_down_workspace(G) -> int:
    return _L.moe_expert_down_workspace(G)


def moe_expert_gate_up(a, group_offset, max_rows, w_gate, w_up, *, a_rows=None, a_rows_div=1,
                       hid=None, ws=None, stream=None):
    """hid[r] = SiLU(a_r W_gate[g]^T) * (a_r W_up[g]^T) for the rows of each group."""
    G, h, d = w_gate.shape
    dev = a.device
    if hid is None:
        hid = torch.empty((max_rows, h), dtype=a.dtype, device=dev)
    if ws is None:
        ws = torch.empty(moe_expert_group_workspace(G), dtype=torch.uint8, device=dev)
    _contig(a, group_offset, a_rows, w_gate, w_up, hid, ws)
    _check(_L.moe_expert_gate_up(_ptr(a), _dt(a), d, h, G, _ptr(group_offset), max_rows,
                                 _ptr(a_rows), a_rows_div, _ptr(w_gate), _ptr(w_up), _ptr(hid),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return hid


def moe_expert_down(hid, group_offset, max_rows, w_down, *, y=None, y_dtype=None, ws=None,
                    stream=None):
    """y[r] = hid[r] W_down[g]^T for the rows of each group."""
    G, d, h = w_down.shape
    dev = hid.device
    if y is None:
        y = torch.empty((max_rows, d), dtype=y_dtype or hid.dtype, device=dev)
    if ws is None:
        ws = torch.empty(moe_expert_down_workspace(G), dtype=torch.uint8, device=dev)
    _contig(hid, group_offset, w_down, y, ws)
    _check(_L.moe_expert_down(_ptr(hid), _dt(hid), d, h, G, _ptr(group_offset), max_rows,
                              _ptr(w_down), _ptr(y), _dt(y), _ptr(ws), ws.numel(),
                              _stream(stream)))
    return y


def moe_combine(y_perm, pair_row, topk_gate, shared_y=None, *, out=None, out_dtype=None,
                k=None, stream=None):
    """out[t] = shared_y[t] + sum of kept g[t, j] * y_perm[pair_row[t k + j]];
    with topk_gate None every gate is 1 (then ``k`` must be given)."""
    if topk_gate is not None:
        T, k = topk_gate.shape
    else:
        T = pair_row.numel() // k
    d = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype or y_perm.dtype, device=y_perm.device)
    _contig(y_perm, pair_row, topk_gate, shared_y, out)
    if shared_y is not None and shared_y.dtype != y_perm.dtype:
        raise TypeError("shared_y must have the dtype of y_perm")
    _check(_L.moe_combine(_ptr(y_perm), _dt(y_perm), _ptr(pair_row), _ptr(topk_gate), T, k, d,
                          _ptr(shared_y), _ptr(out), _dt(out), _stream(stream)))
    return out


def moe_combine_bypass(y_perm, pair_row, topk_idx, topk_gate, e_ffn, n_zero, n_copy, x=None,
                       const_rows=None, shared_y=None, *, out=None, out_dtype=None, stream=None):
    """moe_combine with zero-computation experts after the first ``e_ffn``
    router experts: ``n_zero`` zero, ``n_copy`` copy (add g x[t]) and
    ``const_rows.shape[0]`` constant experts (add g const_rows[c])."""
    T, k = topk_gate.shape
    d = y_perm.shape[1]
    n_const = 0 if const_rows is None else const_rows.shape[0]
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype or y_perm.dtype, device=y_perm.device)
    _contig(y_perm, pair_row, topk_idx, topk_gate, x, const_rows, shared_y, out)
    for t in (x, const_rows, shared_y):
        if t is not None and (t.dtype != y_perm.dtype or t.shape[-1] != d):
            raise TypeError("x, const_rows and shared_y need the dtype and width of y_perm")
    _check(_L.moe_combine_bypass(_ptr(y_perm), _dt(y_perm), _ptr(pair_row), _ptr(topk_idx),
                                 _ptr(topk_gate), T, k, d, e_ffn, n_zero, n_copy, n_const, _ptr(x),
                                 _ptr(const_rows), _ptr(shared_y), _ptr(out), _dt(out),
                                 _stream(stream)))
    return out


def moe_balance_stats_workspace(T, E) -> int:
    return _L.moe_balance_stats_workspace(T, E)


def moe_balance_stats(logits, expert_count, k, alpha=0.01, *, f=None, P=None, loss=None,
                      zloss=None, ws=None, stream=None):
    """Switch balance statistics f, P, alpha*E*sum(f*P) and the router z-loss
    (moe_balance_stats_z; with ``zloss=False``, moe_balance_stats and no z-loss)."""
    T, E = logits.shape
    dev = logits.device
    f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
    P = torch.empty(E, dtype=torch.float32, device=dev) if P is None else P
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    nws = moe_balance_stats_workspace(T, E)
    if ws is None:
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    if zloss is False:
        _contig(logits, expert_count, f, P, loss, ws)
        _check(_L.moe_balance_stats(_ptr(logits), _ptr(expert_count), T, E, k, float(alpha),
                                    _ptr(f), _ptr(P), _ptr(loss), _ptr(ws), ws.numel(),
                                    _stream(stream)))
        return f, P, loss, None
    zloss = torch.empty(1, dtype=torch.float32, device=dev) if zloss is None else zloss
    _contig(logits, expert_count, f, P, loss, zloss, ws)
    _check(_L.moe_balance_stats_z(_ptr(logits), _ptr(expert_count), T, E, k, float(alpha),
                                  _ptr(f), _ptr(P), _ptr(loss), _ptr(zloss), _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return f, P, loss, zloss


# ---------------------------------------------------------------------------
# Backward pass
# ---------------------------------------------------------------------------
def moe_expert_gate_up_train(a, group_offset, max_rows, w_gate, w_up, *, a_rows=None,
                             a_rows_div=1, hid=None, uv=None, ws=None, stream=None):
    """moe_expert_gate_up that also keeps uv = [a W_gate^T | a W_up^T] (bf16)."""
    G, h, d = w_gate.shape
    dev = a.device
    if hid is None:
        hid = torch.empty((max_rows, h), dtype=a.dtype, device=dev)
    if uv is None:
        uv = torch.empty((max_rows, 2 * h), dtype=a.dtype, device=dev)
    if ws is None:
        ws = torch.empty(moe_expert_group_workspace(G), dtype=torch.uint8, device=dev)
    _contig(a, group_offset, a_rows, w_gate, w_up, hid, uv, ws)
    _check(_L.moe_expert_gate_up_train(_ptr(a), _dt(a), d, h, G, _ptr(group_offset), max_rows,
                                       _ptr(a_rows), a_rows_div, _ptr(w_gate), _ptr(w_up),
                                       _ptr(hid), _ptr(uv), _ptr(ws), ws.numel(),
                                       _stream(stream)))
    return hid, uv


def moe_expert_swiglu_backward_workspace(max_rows, d, h, G, dt, gather=False) -> int:
    return _L.moe_expert_swiglu_backward_workspace(max_rows, d, h, G, dt, 1 if gather else 0)


def moe_expert_swiglu_backward(a, group_offset, max_rows, dout, uv, hid, w_gate, w_up, w_down, *,
                               a_rows=None, a_rows_div=1, da=None, dw_gate=None, dw_up=None,
                               dw_down=None, ws=None, stream=None):
    """Gradients of the grouped SwiGLU experts: da [max_rows, d] and dw_gate,
    dw_up [G, h, d], dw_down [G, d, h] (all fp32)."""
    G, h, d = w_gate.shape
    dev = a.device
    f32 = torch.float32
    da = torch.empty((max_rows, d), dtype=f32, device=dev) if da is None else da
    dw_gate = torch.empty((G, h, d), dtype=f32, device=dev) if dw_gate is None else dw_gate
    dw_up = torch.empty((G, h, d), dtype=f32, device=dev) if dw_up is None else dw_up
    dw_down = torch.empty((G, d, h), dtype=f32, device=dev) if dw_down is None else dw_down
    if ws is None:
        n = moe_expert_swiglu_backward_workspace(max_rows, d, h, G, _dt(a), a_rows is not None)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    _contig(a, group_offset, dout, uv, hid, w_gate, w_up, w_down, a_rows, da, dw_gate, dw_up,
            dw_down, ws)
    _check(_L.moe_expert_swiglu_backward(_ptr(a), _dt(a), d, h, G, _ptr(group_offset), max_rows,
                                         _ptr(a_rows), a_rows_div, _ptr(dout), _ptr(uv),
                                         _ptr(hid), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                         _ptr(da), _ptr(dw_gate), _ptr(dw_up), _ptr(dw_down),
                                         _ptr(ws), ws.numel(), _stream(stream)))
    return da, dw_gate, dw_up, dw_down


def moe_combine_backward(dy, y_perm, pair_row, k, topk_gate=None, *, dgate=None, dout=None,
                         want_dout=False, stream=None):
    """dgate[t, j] = <dy[t], y_perm[pair_row[t k + j]]> (0 for dropped pairs) and,
    with ``want_dout`` (or a given dout), dout[pair_row[t k + j]] = g[t, j] dy[t]."""
    T, d = dy.shape
    if dgate is None:
        dgate = torch.empty((T, k), dtype=torch.float32, device=dy.device)
    if want_dout and dout is None:
        dout = torch.empty((T * k, d), dtype=dy.dtype, device=dy.device)
    _contig(dy, y_perm, pair_row, topk_gate, dgate, dout)
    _check(_L.moe_combine_backward(_ptr(dy), _dt(dy), _ptr(y_perm), _dt(y_perm), _ptr(pair_row),
                                   _ptr(topk_gate), T, k, d, _ptr(dgate), _ptr(dout),
                                   _stream(stream)))
    return dgate, dout


def moe_route_backward(logits, topk_idx, topk_gate, dgate, expert_count, alpha=0.01,
                       coef_balance=0.0, coef_z=0.0, *, relu=False, dlogits=None, stream=None):
    """dJ/dlogits through the renormalised gates (or, with ``relu``, the ReLU
    gates), the balance loss and the z-loss."""
    T, E = logits.shape
    k = topk_idx.shape[1]
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=logits.device)
    _contig(logits, topk_idx, topk_gate, dgate, expert_count, dlogits)
    _check(_L.moe_route_backward(_ptr(logits), _ptr(topk_idx), _ptr(topk_gate), _ptr(dgate),
                                 _ptr(expert_count), T, E, k, MOE_ROUTE_RELU if relu else 0,
                                 float(alpha), float(coef_balance),
                                 float(coef_z), _ptr(dlogits), _stream(stream)))
    return dlogits


def moe_combine_backward_bypass(dy, y_perm, pair_row, topk_idx, topk_gate, e_ffn, n_zero, n_copy,
                                x=None, const_rows=None, *, dgate=None, dout=None, stream=None):
    """Gate gradients of every slot (FFN rows, copy = x, constant rows) and
    the gated row gradients dout of the FFN slots that ran."""
    T, k = topk_idx.shape
    d = dy.shape[1]
    n_const = 0 if const_rows is None else const_rows.shape[0]
    if dgate is None:
        dgate = torch.empty((T, k), dtype=torch.float32, device=dy.device)
    _contig(dy, y_perm, pair_row, topk_idx, topk_gate, x, const_rows, dgate, dout)
    _check(_L.moe_combine_backward_bypass(
        _ptr(dy), _dt(dy), _ptr(y_perm), _dt(y_perm), _ptr(pair_row), _ptr(topk_idx),
        _ptr(topk_gate), T, k, d, e_ffn, n_zero, n_copy, n_const, _ptr(x), _ptr(const_rows),
        _ptr(dgate), _ptr(dout), _stream(stream)))
    return dgate, dout


def moe_bypass_backward_workspace(T, d, n_const) -> int:
    return _L.moe_bypass_backward_workspace(T, d, n_const)


def moe_bypass_backward(dy, topk_idx, topk_gate, e_ffn, n_zero, n_copy, n_const, *, dx_acc=None,
                        dconst=None, ws=None, stream=None):
    """dx_acc += (sum of the copy slots' gates) dy; dconst = the constant rows' gradient."""
    T, k = topk_idx.shape
    d = dy.shape[1]
    if dconst is None and n_const:
        dconst = torch.empty((n_const, d), dtype=torch.float32, device=dy.device)
    if ws is None:
        ws = torch.empty(max(1, moe_bypass_backward_workspace(T, d, n_const)), dtype=torch.uint8,
                         device=dy.device)
    _contig(dy, topk_idx, topk_gate, dx_acc, dconst, ws)
    _check(_L.moe_bypass_backward(_ptr(dy), _dt(dy), _ptr(topk_idx), _ptr(topk_gate), T, k, d,
                                  e_ffn, n_zero, n_copy, n_const, _ptr(dx_acc), _ptr(dconst),
                                  _ptr(ws), ws.numel(), _stream(stream)))
    return dx_acc, dconst


def moe_router_backward_workspace(T, d, E) -> int:
    return _L.moe_router_backward_workspace(T, d, E)


def moe_router_backward(x, w_router, dlogits, *, dw_router=None, dlogit_bias=None, dx=None,
                        accumulate_dx=False, want=("dw", "db", "dx"), ws=None, stream=None):
    """Gradients of the linear router: dw_router [E, d], dlogit_bias [E] and
    dx [T, d] (added to the given dx with ``accumulate_dx``); fp32."""
    T, E = dlogits.shape
    d = w_router.shape[1]
    dev = dlogits.device
    f32 = torch.float32
    if "dw" in want and dw_router is None:
        dw_router = torch.empty((E, d), dtype=f32, device=dev)
    if "db" in want and dlogit_bias is None:
        dlogit_bias = torch.empty(E, dtype=f32, device=dev)
    if "dx" in want and dx is None:
        dx = torch.empty((T, d), dtype=f32, device=dev)
    if ws is None:
        ws = torch.empty(max(moe_router_backward_workspace(T, d, E), 1), dtype=torch.uint8,
                         device=dev)
    _contig(x, w_router, dlogits, dw_router, dlogit_bias, dx, ws)
    _check(_L.moe_router_backward(_ptr(x), _ptr(w_router), _dt(w_router), _ptr(dlogits), T, d, E,
                                  _ptr(dw_router), _ptr(dlogit_bias), _ptr(dx),
                                  1 if accumulate_dx else 0, _ptr(ws), ws.numel(),
                                  _stream(stream)))
    return dw_router, dlogit_bias, dx


def moe_probe_mfma_bf16(src, blocks, iters, *, out=None, stream=None):
    """MFMA-only loop on register-resident bf16 operands loaded from src
    (blocks*256*64 bf16); returns out [blocks*256] fp32.  FLOP per call:
    blocks*4*iters*16*32768."""
    if src.dtype != torch.bfloat16 or src.numel() < blocks * 256 * 64:
        raise ValueError("src must hold blocks*256*64 bf16")
    out = torch.empty(blocks * 256, dtype=torch.float32, device=src.device) if out is None else out
    _contig(src, out)
    _check(_L.moe_probe_mfma_bf16(_ptr(src), blocks, iters, _ptr(out), _stream(stream)))
    return out


def moe_probe_read(buf, blocks, *, out=None, stream=None):
    """Streaming read of every byte of buf; returns out [blocks*256] int32
    (each lane's XOR of its words)."""
    nbytes = buf.numel() * buf.element_size()
    out = torch.empty(blocks * 256, dtype=torch.int32, device=buf.device) if out is None else out
    _contig(buf, out)
    _check(_L.moe_probe_read(_ptr(buf), nbytes, blocks, _ptr(out), _stream(stream)))
    return out
