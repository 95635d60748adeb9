"""Plain float64 oracle of the sparse MoE feed-forward forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources, cited by page title and section:
  [Every]  "Every parameter, every token", sections "The gating network",
           "A balance penalty", "A budget", "A shared expert".
  [MoDE]   "Zen MoDE: Mixture of Distilled Experts Architecture", section
           "Router Architecture" (the standard router equation) and section
           "Load Balancing" (the balance-loss and capacity equations).
  [Max]    "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
           sections "Fine-Grained Expert Architecture" (the SwiGLU expert
           equation and the shared-expert paragraph),
           "Auxiliary-Loss-Free Load Balancing" (the per-expert selection bias)
           and "MoE-Specific Training Stability" (the router z-loss).

Layout conventions (shared with the library only by agreement, not by code):
  x        [T, d]        token activations
  w_router [E, d]        one row per expert, so logits = x @ w_router.T
  w_gate   [E, h, d]     expert e's gate projection, stored as the transpose of
  w_up     [E, h, d]     the page's right-multiplied x W_gate form
  w_down   [E, d, h]
  shared   sequence of (w_gate [h_s, d], w_up [h_s, d], w_down [d, h_s])
  Pair p = t*k + j is slot j of token t.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

UNLIMITED = None  # capacity value meaning "no token is ever dropped"


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------
def router_logits(x, w_router, logit_bias=None):
    """One score per expert from a linear map of the token.

    [Every] "The gating network": the gate is a linear layer giving one score
    per expert.  [MoDE] "Router Architecture", standard router equation: the
    scores are W_r x.  No bias term appears in either; ``logit_bias`` is an
    optional per-expert additive offset that becomes part of the logits (it is
    seen by the gates and by the balance probabilities).
    Returns float64 [T, E].
    """
    l = _f64(x) @ _f64(w_router).T
    if logit_bias is not None:
        l = l + _f64(logit_bias)[None, :]
    return l


def selection_keys_on_probs(logits, select_bias=None):
    """The selection key as [Max] "Auxiliary-Loss-Free Load Balancing" writes
    it: s_j = softmax(x W_g)_j + b_j, the routing probability over all experts
    plus the per-expert bias.  The probabilities are computed in float64,
    rounded to float32, and the bias is added in float32 (the precision of
    the decision, as for ``selection_keys``)."""
    l = _f64(logits)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    if select_bias is None:
        return p
    return (p + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)


def selection_keys(logits, select_bias=None):
    """The value that decides expert membership.

    [Max] "Auxiliary-Loss-Free Load Balancing": a per-expert bias b_j shifts
    the selection score; overloaded experts get a negative bias.  Reading used
    here: the bias is added to the logits and affects only which experts are
    chosen, never the gate values.  With no bias the key is the logit itself.
    When ``logits`` are float32 the addition is one IEEE float32 add (round to
    nearest even), the precision in which the selection decision is taken.
    """
    logits = np.asarray(logits)
    if select_bias is None:
        return logits.copy()
    if logits.dtype == np.float32:
        return (logits + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    return _f64(logits) + _f64(select_bias)[None, :]


def top_k(keys, k):
    """Indices of the k largest keys per token, as an int32 [T, k] array.

    [Every] "The gating network": sparse routing keeps the top k scores.
    [MoDE] "Router Architecture": TopK(., K).  The pages are silent on ties and
    on slot order; reading used: slots are in descending key order and equal
    keys go to the lower expert index, for membership and for order.  A stable
    sort of the negated keys gives exactly that (comparison is by value, so
    -0.0 and +0.0 tie).
    """
    keys = np.asarray(keys)
    T, E = keys.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(logits, idx):
    """Renormalised gate weights of the selected experts, float64 [T, k].

    [Every] "The gating network": a softmax over the top-k logits, i.e. the
    kept scores renormalised to sum to one.  [MoDE] "Router Architecture"
    writes TopK(softmax(W_r x)); renormalising that over the kept set is the
    same number.  Computed as exp(l_i - m) / sum over the selected set of
    exp(l_j - m), m the largest selected logit.  The logits used are the
    unbiased ones (the selection bias never reaches the gates).
    """
    l = _f64(logits)
    sel = np.take_along_axis(l, np.asarray(idx, dtype=np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    w = np.exp(sel - m)
    return w / w.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Capacity and dispatch
# ---------------------------------------------------------------------------
def capacity(cf, T, k, E):
    """Per-expert token budget C = ceil(cf * T * k / E), or UNLIMITED.

    [MoDE] "Adaptive Capacity Factors": capacity_e = C * tokens / N_E (the
    page's C is the capacity factor).  [Every] "A budget": a factor above 1
    leaves slack.  Reading used: the count of routed pairs T*k replaces the
    token count (so that cf = 1 is exactly the mean load) and the result is
    rounded up.  ``cf`` is read as the shortest decimal that round-trips to
    the given double (what a user writes: 1.1 means 11/10), and the product is
    rounded up exactly.  None or cf <= 0 means unlimited.
    """
    if cf is None or cf <= 0:
        return UNLIMITED
    q = Fraction(repr(float(cf))) * T * k / E
    return int(math.ceil(q))


def dispatch(idx, E, cap=UNLIMITED):
    """Group routed pairs by expert and apply the capacity drop.

    [Every] "A budget": each expert takes at most ``cap`` tokens of the batch;
    pairs past the budget are dropped.  [Every] "What you still pay for": a
    token travels to the expert it was assigned.  Reading used: an expert's
    pairs are ranked in token order and its first ``cap`` pairs are kept.
    ``cap`` is UNLIMITED, one budget for every expert, or a sequence of E
    per-expert budgets ([MoDE] "Adaptive Capacity Factors": capacity per
    expert).

    Returns a dict of int64 arrays:
      count    [E]    routed pairs per expert, before the drop
      kept     [E]    min(count, cap)
      offset   [E+1]  exclusive prefix sum of kept
      rank     [T*k]  r(p): pairs of the same expert with a smaller token index
      pair_row [T*k]  row of pair p in the expert-sorted order, -1 if dropped
      row_pair [T*k]  inverse of pair_row on rows < offset[E], -1 after
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    R = flat.size
    count = np.zeros(E, dtype=np.int64)
    kept = np.zeros(E, dtype=np.int64)
    rank = np.zeros(R, dtype=np.int64)
    pair_row = np.full(R, -1, dtype=np.int64)
    members = []
    per_expert = cap is not UNLIMITED and np.ndim(cap) == 1
    for e in range(E):
        pairs_e = np.nonzero(flat == e)[0]  # ascending pair id == ascending token id
        count[e] = pairs_e.size
        rank[pairs_e] = np.arange(pairs_e.size)
        cap_e = int(cap[e]) if per_expert else cap
        keep_e = pairs_e if cap_e is UNLIMITED else pairs_e[:cap_e]
        kept[e] = keep_e.size
        members.append(keep_e)
    offset = np.zeros(E + 1, dtype=np.int64)
    offset[1:] = np.cumsum(kept)
    row_pair = np.full(R, -1, dtype=np.int64)
    for e in range(E):
        rows = offset[e] + np.arange(kept[e])
        pair_row[members[e]] = rows
        row_pair[rows] = members[e]
    return dict(count=count, kept=kept, offset=offset, rank=rank,
                pair_row=pair_row, row_pair=row_pair)


# ---------------------------------------------------------------------------
# Experts
# ---------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)).

    [Max] "Fine-Grained Expert Architecture" names SiLU inside the SwiGLU
    expert; the function itself is the standard one.  For z below about -709
    exp(-z) overflows to inf and the quotient is the correct limit -0.
    """
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(xs, w_gate, w_up, w_down):
    """One SwiGLU expert on a batch of rows, float64 [n, d].

    [Max] "Fine-Grained Expert Architecture", expert equation:
    Expert(x) = (SiLU(x W_gate) * x W_up) W_down.  With the stored transposes
    ([h, d], [h, d], [d, h]) that is (silu(x Wg^T) * (x Wu^T)) Wd^T.
    """
    xs = _f64(xs)
    u = xs @ _f64(w_gate).T
    v = xs @ _f64(w_up).T
    return (silu(u) * v) @ _f64(w_down).T


def moe_output(x, idx, gate, pair_row, w_gate, w_up, w_down, shared=(), tokens=None):
    """The layer output y (no residual), float64 [len(tokens), d].

    [Every] "The gating network": y = sum over kept slots of g_j * Expert_j(x);
    the result has the residual width and is added to the residual outside the
    layer.  [Every] "A budget": a dropped pair contributes nothing; the
    remaining gates are not renormalised.  [Max] "Fine-Grained Expert
    Architecture" and [Every] "A shared expert": shared experts run on every
    token and are added with weight one.

    ``tokens`` selects the output rows to compute (all tokens by default); only
    the experts those tokens reach are evaluated.
    """
    x = np.asarray(x)
    T = x.shape[0]
    idx = np.asarray(idx, dtype=np.int64)
    k = idx.shape[1]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    pr = np.asarray(pair_row, dtype=np.int64).reshape(T, k)[tokens]
    sel = idx[tokens]
    g = _f64(gate)[tokens]
    xs = _f64(x[tokens])
    y = np.zeros((tokens.size, x.shape[1]), dtype=np.float64)
    for e in np.unique(sel[pr >= 0]):
        rows, slots = np.nonzero((sel == e) & (pr >= 0))
        out_e = swiglu(xs[rows], w_gate[e], w_up[e], w_down[e])
        y[rows] += g[rows, slots][:, None] * out_e
    for (sg, su, sd) in shared:
        y += swiglu(xs, sg, su, sd)
    return y


# ---------------------------------------------------------------------------
# Balance statistics
# ---------------------------------------------------------------------------
def balance_stats(logits, count, k, alpha=0.01):
    """Switch balance statistics (f, P, loss).

    [MoDE] "Auxiliary Load Balancing Loss": L = alpha * N * sum_e f_e P_e with
    f_e the fraction of tokens routed to e (an indicator of e in TopK, i.e.
    before any capacity drop), P_e the mean routing probability of e, and
    alpha = 0.01.  [Every] "A balance penalty": the same loss with N experts.
    Readings used: f_e = count_e / (T*k) so that f sums to one and uniform
    routing gives L = alpha for every k; P_e averages the full softmax over all
    E experts of the logits (logit bias included, selection bias excluded);
    N = E, the number of routed experts.
    """
    l = _f64(logits)
    T, E = l.shape
    count = _f64(count)
    f = count / (T * k)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    P = p.mean(axis=0)
    loss = alpha * E * float(np.sum(f * P))
    return f, P, loss


def router_z_loss(logits):
    """Router z-loss (1/T) sum_t (log sum_j exp l_tj)^2.

    [Max] "MoE-Specific Training Stability": the z-loss penalises large router
    logits; the page applies it with coefficient 1e-3 (the caller scales).
    """
    l = _f64(logits)
    m = l.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(l - m).sum(axis=1, keepdims=True)))[:, 0]
    return float(np.mean(lse * lse))


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def forward(x, w_router, w_gate, w_up, w_down, k, shared=(), logit_bias=None,
            select_bias=None, cap=UNLIMITED, alpha=0.01, logits=None, tokens=None,
            topk_idx=None):
    """The whole forward pass in the pages' order.

    If ``logits`` is given (e.g. the float32 logits another implementation
    produced) the routing, dispatch, output and statistics are computed from
    them; otherwise from this oracle's own float64 logits.  If ``topk_idx`` is
    given, it is the selection (a selection made on other keys, such as the
    routing probability plus the bias, whose validity the caller checks); the
    gates, dispatch, output and statistics follow from it as usual.  Returns a
    dict with every intermediate.
    """
    if logits is None:
        logits = router_logits(x, w_router, logit_bias)
    keys = selection_keys(logits, select_bias)
    idx = top_k(keys, k) if topk_idx is None else np.asarray(topk_idx, dtype=np.int32)
    g = gates(logits, idx)
    E = np.asarray(w_router).shape[0]
    disp = dispatch(idx, E, cap)
    y = moe_output(x, idx, g, disp["pair_row"], w_gate, w_up, w_down, shared, tokens)
    f, P, loss = balance_stats(logits, disp["count"], k, alpha)
    return dict(logits=logits, keys=keys, topk_idx=idx, topk_gate=g, y=y,
                f=f, P=P, loss=loss, **disp)
