"""Plain float64 oracle of the sparse MoE feed-forward layer's backward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is differentiated.  The scalar objective is

    J = sum(dy * y) + c_bal * loss + c_z * zloss

with y the layer output of ``moe_oracle.forward`` (no residual), ``dy`` the
upstream gradient of y, ``loss`` the Switch balance loss and ``zloss`` the
router z-loss; the functions below return dJ/d(every input that carries a
gradient), applying the chain rule to the forward definition step by step in
reverse order.

Sources, cited by page title and section:
  [Every]  "Every parameter, every token", section "The gating network": the
           choice of experts is discrete; training holds the selected set
           fixed, sends gradient to the router only through the gate weights
           of the experts that ran, and an expert that was off for a token
           gets no gradient from it.  Section "A balance penalty": the router
           is trained on the task and on the penalty together.  Section "A
           budget": a dropped pair skips its expert update.
  [MoDE]   "Zen MoDE: Mixture of Distilled Experts Architecture", section
           "Auxiliary Load Balancing Loss" (the penalty).
  [Max]    "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
           sections "Fine-Grained Expert Architecture" (the SwiGLU expert),
           "Auxiliary-Loss-Free Load Balancing" (the selection bias) and
           "MoE-Specific Training Stability" (the z-loss).

Readings (the pages give the rule, not every derivative):
  * The selected set, the capacity drop and f (a count) are piecewise
    constant in the parameters: no gradient flows through them, nor into the
    selection bias.  The balance loss reaches the router through P alone.
  * A dropped pair has no expert output, so its gate gets zero gradient from
    the output; its gate still sits in the renormalising softmax over the
    selected set, so the kept gates' gradients reach its logit.
  * logit_bias is part of the logits (it gets the column sums of dJ/dlogits).

Layouts are those of ``moe_oracle`` (weights stored transposed: w_gate and
w_up [E, h, d], w_down [E, d, h], w_router [E, d]).
"""

from __future__ import annotations

import numpy as np

from . import moe_oracle as mo


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------
def silu_grad(z):
    """d SiLU(z) / dz = s (1 + z (1 - s)), s = sigmoid(z) = 1 / (1 + exp(-z)).

    The derivative of the [Max] "Fine-Grained Expert Architecture" activation;
    for z below about -709 exp(-z) overflows, s = 0 and the result is the
    correct limit 0.
    """
    z = _f64(z)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def swiglu_backward(xs, w_gate, w_up, w_down, dout):
    """Gradients of sum(dout * Expert(xs)) for one SwiGLU expert.

    [Max] "Fine-Grained Expert Architecture": Expert(x) = (SiLU(x Wg) * x Wu)
    Wd, here with the stored transposes: u = xs Wg^T, v = xs Wu^T,
    hid = SiLU(u) v, out = hid Wd^T.  Reverse order:
      d Wd  = dout^T hid                       [d, h]
      d hid = dout Wd                          [n, h]
      d u   = d hid * v * SiLU'(u),  d v = d hid * SiLU(u)
      d Wg  = du^T xs,  d Wu = dv^T xs         [h, d]
      d xs  = du Wg + dv Wu                    [n, d]
    Returns (d_xs, d_w_gate, d_w_up, d_w_down).
    """
    xs, wg, wu, wd, dout = _f64(xs), _f64(w_gate), _f64(w_up), _f64(w_down), _f64(dout)
    u = xs @ wg.T
    v = xs @ wu.T
    hid = mo.silu(u) * v
    d_wd = dout.T @ hid
    d_hid = dout @ wd
    du = d_hid * v * silu_grad(u)
    dv = d_hid * mo.silu(u)
    return du @ wg + dv @ wu, du.T @ xs, dv.T @ xs, d_wd


# ---------------------------------------------------------------------------
# Combine and gates
# ---------------------------------------------------------------------------
def gate_grad(dy, x, idx, pair_row, w_gate, w_up, w_down):
    """dJ/d(gate) [T, k]: the inner product of the token's upstream gradient
    with the output of the expert that ran for that slot, zero for a dropped
    pair.

    [Every] "The gating network": y = sum_j g_j Expert_j(x), so dJ/dg_j =
    <dy, Expert_j(x)>; "A budget": a dropped pair has no expert output.
    """
    dy, x = _f64(dy), _f64(x)
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    pr = np.asarray(pair_row, dtype=np.int64).reshape(T, k)
    dg = np.zeros((T, k))
    for e in np.unique(idx[pr >= 0]):
        rows, slots = np.nonzero((idx == e) & (pr >= 0))
        out_e = mo.swiglu(x[rows], w_gate[e], w_up[e], w_down[e])
        dg[rows, slots] = np.sum(dy[rows] * out_e, axis=1)
    return dg


def gate_logit_grad(logits, idx, dgate):
    """dJ/dlogits [T, E] through the renormalised gates.

    [Every] "The gating network": g_j = exp(l_j) / sum_{i in S} exp(l_i) over
    the selected set S, so dg_j/dl_i = g_j (delta_ij - g_i) for i in S and 0
    for i outside S (the experts that were off get nothing).  Hence
    dl_i = g_i (dg_i - sum_j g_j dg_j) on S.
    """
    idx = np.asarray(idx, dtype=np.int64)
    g = mo.gates(logits, idx)
    dg = _f64(dgate)
    inner = np.sum(g * dg, axis=1, keepdims=True)
    dl = np.zeros(np.asarray(logits).shape)
    np.put_along_axis(dl, idx, g * (dg - inner), axis=1)
    return dl


# ---------------------------------------------------------------------------
# Auxiliary losses
# ---------------------------------------------------------------------------
def balance_logit_grad(logits, count, k, alpha=0.01):
    """d loss / dlogits [T, E] of the Switch balance loss.

    [MoDE] "Auxiliary Load Balancing Loss" / [Every] "A balance penalty":
    loss = alpha N sum_e f_e P_e with P_e = (1/T) sum_t p_te, p_t the full
    softmax of logits[t]; f is a count (no gradient).  With dp_te/dl_ti =
    p_te (delta_ei - p_ti):
      dloss/dl_ti = (alpha N / T) p_ti (f_i - sum_e f_e p_te).
    """
    l = _f64(logits)
    T, E = l.shape
    f = _f64(count) / (T * k)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    fp = p @ f
    return (alpha * E / T) * p * (f[None, :] - fp[:, None])


def z_loss_logit_grad(logits):
    """d zloss / dlogits [T, E] of the router z-loss (1/T) sum_t lse_t^2.

    [Max] "MoE-Specific Training Stability".  d lse_t / dl_ti = p_ti, so the
    gradient is (2/T) lse_t p_ti.
    """
    l = _f64(logits)
    T = l.shape[0]
    m = l.max(axis=1, keepdims=True)
    ex = np.exp(l - m)
    s = ex.sum(axis=1, keepdims=True)
    lse = m + np.log(s)
    return (2.0 / T) * lse * (ex / s)


def router_linear_backward(x, w_router, dlogits):
    """Gradients of the linear router logits = x W_r^T (+ logit_bias).

    [Every] "The gating network" / [MoDE] "Router Architecture".  Returns
    (dx [T, d], dw_router [E, d], dlogit_bias [E]).
    """
    dl = _f64(dlogits)
    return dl @ _f64(w_router), dl.T @ _f64(x), dl.sum(axis=0)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def backward(x, w_router, w_gate, w_up, w_down, k, dy, shared=(), logit_bias=None,
             select_bias=None, cap=mo.UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0, logits=None,
             topk_idx=None):
    """dJ for the whole layer, in reverse order of ``moe_oracle.forward``.

    If ``logits`` is given (e.g. float32 logits another implementation
    produced) the routing and every logit-dependent term use them, as in the
    forward; ``topk_idx``, if given, is the selection (as in the forward: the
    selection key moves only the chosen set, so the gradient is the same
    function of that set).  Returns a dict: dx, dw_router, dlogit_bias, dw_gate, dw_up,
    dw_down, dshared (a list of (dwg, dwu, dwd)), and the intermediates
    dgate [T, k] and dlogits [T, E], plus ``fwd`` (the forward's dict).
    """
    x, dy = _f64(x), _f64(dy)
    fw = mo.forward(x, w_router, w_gate, w_up, w_down, k, shared=shared, logit_bias=logit_bias,
                    select_bias=select_bias, cap=cap, alpha=alpha, logits=logits,
                    topk_idx=topk_idx)
    idx, g, pr = fw["topk_idx"], fw["topk_gate"], fw["pair_row"]
    T, d = x.shape
    E = np.asarray(w_router).shape[0]
    # combine: y = sum over kept slots g * Expert(x) + shared
    dgate = gate_grad(dy, x, idx, pr, w_gate, w_up, w_down)
    dx = np.zeros((T, d))
    dwg = np.zeros(np.shape(w_gate))
    dwu = np.zeros(np.shape(w_up))
    dwd = np.zeros(np.shape(w_down))
    prk = np.asarray(pr, dtype=np.int64).reshape(T, k)
    for e in range(E):
        rows, slots = np.nonzero((idx == e) & (prk >= 0))
        if rows.size == 0:
            continue  # an expert that ran for no token gets no gradient
        dout = g[rows, slots][:, None] * dy[rows]
        dxs, dwg[e], dwu[e], dwd[e] = swiglu_backward(x[rows], w_gate[e], w_up[e], w_down[e], dout)
        np.add.at(dx, rows, dxs)
    dshared = []
    for (sg, su, sd) in shared:
        dxs, a, b, c = swiglu_backward(x, sg, su, sd, dy)
        dx += dxs
        dshared.append((a, b, c))
    # router: the gates, then the auxiliary losses, then the linear map
    lg = fw["logits"]
    dlogits = gate_logit_grad(lg, idx, dgate)
    if c_bal:
        dlogits = dlogits + c_bal * balance_logit_grad(lg, fw["count"], k, alpha)
    if c_z:
        dlogits = dlogits + c_z * z_loss_logit_grad(lg)
    dxr, dwr, dlb = router_linear_backward(x, w_router, dlogits)
    dx += dxr
    return dict(dx=dx, dw_router=dwr, dlogit_bias=dlb, dw_gate=dwg, dw_up=dwu, dw_down=dwd,
                dshared=dshared, dgate=dgate, dlogits=dlogits, fwd=fw)


def objective(x, w_router, w_gate, w_up, w_down, k, dy, shared=(), logit_bias=None,
              select_bias=None, cap=mo.UNLIMITED, alpha=0.01, c_bal=0.0, c_z=0.0):
    """J = sum(dy * y) + c_bal * loss + c_z * zloss from the forward alone, and
    the selection it used (for finite-difference checks of ``backward``)."""
    fw = mo.forward(x, w_router, w_gate, w_up, w_down, k, shared=shared, logit_bias=logit_bias,
                    select_bias=select_bias, cap=cap, alpha=alpha)
    J = float(np.sum(_f64(dy) * fw["y"])) + c_bal * fw["loss"] + c_z * mo.router_z_loss(fw["logits"])
    return J, fw["topk_idx"]
