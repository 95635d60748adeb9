"""Plain float64 oracle of two routing variants of the sparse MoE layer:
ReLU routing and zero-computation (zero, copy and constant) experts.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source: "Zen MoDE: Mixture of Diverse Experts", section
"Router" (the router adopts ReLU gating, which gives each token an adaptive
number of experts instead of a fixed top-K, and zero-computation experts, of
three kinds: zero, copy and constant, which let a token skip the FFN
compute), and the same page's "Related Work" (both taken from earlier
published work).  The page names the mechanisms without equations; the
readings used are stated in each function.
"""

from __future__ import annotations

import numpy as np

from .moe_oracle import UNLIMITED, balance_stats, dispatch, gates, moe_output, router_logits, top_k


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# ReLU routing
# ---------------------------------------------------------------------------
def relu_route(logits, k_max):
    """ReLU gating: (topk_idx int32 [T, k_max], topk_gate float64 [T, k_max]).

    Reading used: the gate of expert e is max(l_e, 0), so a token uses exactly
    the experts whose logit is positive (a zero logit gives a zero gate and is
    not used), with no renormalisation.  The token's slots hold its positive
    experts in descending logit order (equal logits: lower index first); at
    most ``k_max`` of them are kept (the largest), and unused slots hold
    expert -1 with gate 0.
    """
    l = _f64(logits)
    T, E = l.shape
    if not 1 <= k_max <= E:
        raise ValueError("need 1 <= k_max <= E")
    idx = np.full((T, k_max), -1, dtype=np.int32)
    g = np.zeros((T, k_max), dtype=np.float64)
    for t in range(T):
        pos = [e for e in range(E) if l[t, e] > 0]
        pos.sort(key=lambda e: (-l[t, e], e))
        for j, e in enumerate(pos[:k_max]):
            idx[t, j] = e
            g[t, j] = l[t, e]
    return idx, g


def forward_relu(x, w_router, w_gate, w_up, w_down, k_max, shared=(), logit_bias=None,
                 cap=UNLIMITED, alpha=0.01, logits=None, tokens=None):
    """The layer with ReLU routing: y = shared + sum over used slots g_j E_j(x).

    Dispatch and capacity are the plain layer's (an unused slot is never
    routed, so it takes no budget); the balance statistics keep their plain
    definitions with f_e = count_e / (T k_max).
    """
    if logits is None:
        logits = router_logits(x, w_router, logit_bias)
    idx, g = relu_route(logits, k_max)
    E = np.asarray(w_router).shape[0]
    disp = dispatch(idx, E, cap)
    y = moe_output(x, idx, g, disp["pair_row"], w_gate, w_up, w_down, shared, tokens)
    f, P, loss = balance_stats(logits, disp["count"], k_max, alpha)
    return dict(logits=logits, topk_idx=idx, topk_gate=g, y=y, f=f, P=P, loss=loss, **disp)


# ---------------------------------------------------------------------------
# Zero-computation experts
# ---------------------------------------------------------------------------
def bypass_kind(e, E_ffn, n_zero, n_copy, n_const):
    """Kind of router expert e: ("ffn", e), ("zero", i), ("copy", i) or ("const", i).

    Reading used for the numbering: the router scores E_ffn FFN experts
    followed by n_zero zero experts, n_copy copy experts and n_const constant
    experts, in that order.
    """
    if 0 <= e < E_ffn:
        return "ffn", e
    i = e - E_ffn
    if 0 <= i < n_zero:
        return "zero", i
    i -= n_zero
    if 0 <= i < n_copy:
        return "copy", i
    i -= n_copy
    if 0 <= i < n_const:
        return "const", i
    raise ValueError(f"expert {e} out of range")


def bypass_output(x, idx, gate, E_ffn, n_zero, n_copy, const_rows, tokens=None):
    """The zero-computation experts' share of the output, float64 [len(tokens), d].

    Readings used: a zero expert outputs the zero vector, a copy expert outputs
    its input token x_t unchanged, and constant expert c outputs a fixed
    (trainable) vector v_c of width d, whatever the token.  Each enters the
    gate-weighted sum like any other selected expert.
    """
    x = _f64(x)
    T, d = x.shape
    idx = np.asarray(idx, dtype=np.int64)
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    const_rows = _f64(const_rows).reshape(-1, d)
    n_const = const_rows.shape[0]
    g = _f64(gate)
    y = np.zeros((tokens.size, d), dtype=np.float64)
    for i, t in enumerate(tokens):
        for j in range(idx.shape[1]):
            kind, c = bypass_kind(int(idx[t, j]), E_ffn, n_zero, n_copy, n_const)
            if kind == "copy":
                y[i] += g[t, j] * x[t]
            elif kind == "const":
                y[i] += g[t, j] * const_rows[c]
    return y


def forward_bypass(x, w_router, w_gate, w_up, w_down, k, n_zero, n_copy, const_rows,
                   shared=(), logit_bias=None, cap=UNLIMITED, alpha=0.01, logits=None,
                   tokens=None):
    """The layer with zero-computation experts after its E_ffn FFN experts.

    Routing is the plain top-k over all E = E_ffn + n_zero + n_copy + n_const
    router experts with softmax gates renormalised over the k selected.
    Readings used: only the FFN experts run on rows, so only they have a token
    budget (``cap`` applies to them; a zero-computation expert never drops a
    pair), and the balance statistics are taken over all E router experts
    (count_e before any drop).
    """
    if logits is None:
        logits = router_logits(x, w_router, logit_bias)
    E = np.asarray(w_router).shape[0]
    E_ffn = np.asarray(w_gate).shape[0]
    n_const = _f64(const_rows).reshape(-1, np.asarray(x).shape[1]).shape[0]
    if E_ffn + n_zero + n_copy + n_const != E:
        raise ValueError("router rows must be E_ffn + n_zero + n_copy + n_const")
    idx = top_k(logits, k)
    g = gates(logits, idx)
    caps = np.zeros(E, dtype=np.int64)
    ffn_cap = np.iinfo(np.int64).max if cap is UNLIMITED else int(cap)
    caps[:E_ffn] = ffn_cap
    disp = dispatch(idx, E, caps)
    y = moe_output(x, idx, g, disp["pair_row"], w_gate, w_up, w_down, shared, tokens)
    y = y + bypass_output(x, idx, g, E_ffn, n_zero, n_copy, const_rows, tokens)
    f, P, loss = balance_stats(logits, disp["count"], k, alpha)
    return dict(logits=logits, topk_idx=idx, topk_gate=g, y=y, f=f, P=P, loss=loss, **disp)


# ---------------------------------------------------------------------------
# ReLU routing: backward
# ---------------------------------------------------------------------------
def relu_gate_logit_grad(logits, idx, dgate):
    """dJ/dlogits [T, E] through ReLU gates.

    A used slot's gate is the logit itself (positive), so dl_e = dgate for
    the expert in that slot; an expert a token does not use gets nothing
    (reading: the ReLU's derivative is taken as 0 at a zero logit, which is
    never used; an expert with a positive logit that the k_max limit left out
    is off, like an unselected expert of top-k routing).
    """
    idx = np.asarray(idx, dtype=np.int64)
    dg = _f64(dgate)
    dl = np.zeros(np.asarray(logits).shape)
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            if idx[t, j] >= 0:
                dl[t, idx[t, j]] += dg[t, j]
    return dl


def backward_relu(x, w_router, w_gate, w_up, w_down, k_max, dy, shared=(), logit_bias=None,
                  cap=UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0, logits=None):
    """dJ of the ReLU-routed layer, J = <dy, y> + c_bal loss + c_z zloss, in
    reverse order of ``forward_relu``: the combine, the experts on their kept
    rows, the ReLU gates, the auxiliary losses, the linear router.  Returns
    the dict of ``moe_backward.backward``."""
    from .moe_backward import (balance_logit_grad, gate_grad, router_linear_backward,
                               swiglu_backward, z_loss_logit_grad)
    x, dy = _f64(x), _f64(dy)
    fw = forward_relu(x, w_router, w_gate, w_up, w_down, k_max, shared=shared,
                      logit_bias=logit_bias, cap=cap, alpha=alpha, logits=logits)
    idx, g, pr = fw["topk_idx"], fw["topk_gate"], fw["pair_row"]
    T, d = x.shape
    E = np.asarray(w_router).shape[0]
    dgate = gate_grad(dy, x, idx, pr, w_gate, w_up, w_down)
    dx = np.zeros((T, d))
    dwg, dwu, dwd = (np.zeros(np.shape(w)) for w in (w_gate, w_up, w_down))
    prk = np.asarray(pr, dtype=np.int64).reshape(T, k_max)
    for e in range(E):
        rows, slots = np.nonzero((idx == e) & (prk >= 0))
        if rows.size == 0:
            continue
        dout = g[rows, slots][:, None] * dy[rows]
        dxs, dwg[e], dwu[e], dwd[e] = swiglu_backward(x[rows], w_gate[e], w_up[e], w_down[e], dout)
        np.add.at(dx, rows, dxs)
    dshared = []
    for (sg, su, sd) in shared:
        dxs, a, b, c = swiglu_backward(x, sg, su, sd, dy)
        dx += dxs
        dshared.append((a, b, c))
    lg = fw["logits"]
    dlogits = relu_gate_logit_grad(lg, idx, dgate)
    if c_bal:
        dlogits = dlogits + c_bal * balance_logit_grad(lg, fw["count"], k_max, alpha)
    if c_z:
        dlogits = dlogits + c_z * z_loss_logit_grad(lg)
    dxr, dwr, dlb = router_linear_backward(x, w_router, dlogits)
    dx += dxr
    return dict(dx=dx, dw_router=dwr, dlogit_bias=dlb, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                dshared=dshared, dgate=dgate, dlogits=dlogits, fwd=fw)


def objective_relu(x, w_router, w_gate, w_up, w_down, k_max, dy, shared=(), logit_bias=None,
                   cap=UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0):
    """J = sum(dy * y) + c_bal * loss + c_z * zloss of the ReLU-routed layer
    from its forward alone, and the selection it used."""
    from .moe_oracle import router_z_loss
    fw = forward_relu(x, w_router, w_gate, w_up, w_down, k_max, shared=shared,
                      logit_bias=logit_bias, cap=cap, alpha=alpha)
    J = (float(np.sum(_f64(dy) * fw["y"])) + c_bal * fw["loss"] +
         c_z * router_z_loss(fw["logits"]))
    return J, fw["topk_idx"]


# ---------------------------------------------------------------------------
# Zero-computation experts: backward
# ---------------------------------------------------------------------------
def bypass_gate_grad(dy, x, idx, E_ffn, n_zero, n_copy, const_rows):
    """dJ/d(gate) [T, k] of the zero-computation slots (0 on FFN slots):
    <dy_t, x_t> for a copy expert, <dy_t, v_c> for constant expert c, 0 for
    a zero expert (y = sum_j g_j out_j, so dJ/dg_j = <dy, out_j>)."""
    dy, x = _f64(dy), _f64(x)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    const_rows = _f64(const_rows).reshape(-1, x.shape[1])
    dg = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            kind, c = bypass_kind(int(idx[t, j]), E_ffn, n_zero, n_copy, const_rows.shape[0])
            if kind == "copy":
                dg[t, j] = float(dy[t] @ x[t])
            elif kind == "const":
                dg[t, j] = float(dy[t] @ const_rows[c])
    return dg


def backward_bypass(x, w_router, w_gate, w_up, w_down, k, n_zero, n_copy, const_rows, dy,
                    shared=(), logit_bias=None, cap=UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0,
                    logits=None):
    """dJ of the layer with zero-computation experts, in reverse order of
    ``forward_bypass``.  Besides the plain layer's gradients: a copy slot
    passes g dy_t to dx_t, constant expert c collects dconst[c] = sum over
    its slots of g dy_t, and every slot's gate gradient enters the softmax
    over all router experts.  Returns the dict of ``moe_backward.backward``
    plus ``dconst`` [n_const, d]."""
    from .moe_backward import (balance_logit_grad, gate_grad, gate_logit_grad,
                               router_linear_backward, swiglu_backward, z_loss_logit_grad)
    x, dy = _f64(x), _f64(dy)
    fw = forward_bypass(x, w_router, w_gate, w_up, w_down, k, n_zero, n_copy, const_rows,
                        shared=shared, logit_bias=logit_bias, cap=cap, alpha=alpha, logits=logits)
    idx, g, pr = fw["topk_idx"], fw["topk_gate"], fw["pair_row"]
    T, d = x.shape
    E_ffn = np.asarray(w_gate).shape[0]
    cr = _f64(const_rows).reshape(-1, d)
    dgate = gate_grad(dy, x, idx, pr, w_gate, w_up, w_down)  # FFN slots (pair_row >= 0)
    dgate = dgate + bypass_gate_grad(dy, x, idx, E_ffn, n_zero, n_copy, cr)
    dx = np.zeros((T, d))
    dwg, dwu, dwd = (np.zeros(np.shape(w)) for w in (w_gate, w_up, w_down))
    prk = np.asarray(pr, dtype=np.int64).reshape(T, k)
    for e in range(E_ffn):
        rows, slots = np.nonzero((idx == e) & (prk >= 0))
        if rows.size == 0:
            continue
        dout = g[rows, slots][:, None] * dy[rows]
        dxs, dwg[e], dwu[e], dwd[e] = swiglu_backward(x[rows], w_gate[e], w_up[e], w_down[e], dout)
        np.add.at(dx, rows, dxs)
    dconst = np.zeros_like(cr)
    for t in range(T):
        for j in range(k):
            kind, c = bypass_kind(int(idx[t, j]), E_ffn, n_zero, n_copy, cr.shape[0])
            if kind == "copy":
                dx[t] += g[t, j] * dy[t]
            elif kind == "const":
                dconst[c] += g[t, j] * dy[t]
    dshared = []
    for (sg, su, sd) in shared:
        dxs, a, b, c = swiglu_backward(x, sg, su, sd, dy)
        dx += dxs
        dshared.append((a, b, c))
    lg = fw["logits"]
    dlogits = gate_logit_grad(lg, idx, dgate)
    if c_bal:
        dlogits = dlogits + c_bal * balance_logit_grad(lg, fw["count"], k, alpha)
    if c_z:
        dlogits = dlogits + c_z * z_loss_logit_grad(lg)
    dxr, dwr, dlb = router_linear_backward(x, w_router, dlogits)
    dx += dxr
    return dict(dx=dx, dw_router=dwr, dlogit_bias=dlb, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                dconst=dconst, dshared=dshared, dgate=dgate, dlogits=dlogits, fwd=fw)


def objective_bypass(x, w_router, w_gate, w_up, w_down, k, n_zero, n_copy, const_rows, dy,
                     shared=(), logit_bias=None, cap=UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0):
    """J = sum(dy * y) + c_bal * loss + c_z * zloss of the layer with
    zero-computation experts, and the selection it used."""
    from .moe_oracle import router_z_loss
    fw = forward_bypass(x, w_router, w_gate, w_up, w_down, k, n_zero, n_copy, const_rows,
                        shared=shared, logit_bias=logit_bias, cap=cap, alpha=alpha)
    J = (float(np.sum(_f64(dy) * fw["y"])) + c_bal * fw["loss"] +
         c_z * router_z_loss(fw["logits"]))
    return J, fw["topk_idx"]
