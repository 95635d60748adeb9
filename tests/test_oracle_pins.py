"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it follows.  None of them re-types an oracle
formula: they use closed forms worked by hand, special cases that reduce to a
library routine (PyTorch / SciPy), invariants, and brute force from
``tests/brute.py`` on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings, strategies as st

import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def rand_layer(rng, T, d, E, h, n_shared=0, hs=4):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    wg = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, h)) / math.sqrt(h)
    shared = [(rng.standard_normal((hs, d)) / math.sqrt(d), rng.standard_normal((hs, d)) / math.sqrt(d),
               rng.standard_normal((d, hs)) / math.sqrt(hs)) for _ in range(n_shared)]
    return x, wr, wg, wu, wd, shared


def torch_swiglu(x, wg, wu, wd):
    """Library form of the SwiGLU expert ([ZenMax] "Fine-Grained Expert Architecture")."""
    F = torch.nn.functional
    X = torch.as_tensor(np.asarray(x, dtype=np.float64))
    a = F.silu(F.linear(X, torch.as_tensor(np.asarray(wg, np.float64)))) * \
        F.linear(X, torch.as_tensor(np.asarray(wu, np.float64)))
    return F.linear(a, torch.as_tensor(np.asarray(wd, np.float64))).numpy()


# ---------------------------------------------------------------------------
# Page constants fixture
# ---------------------------------------------------------------------------
def test_page_constants_default_alpha():
    """Balance coefficient alpha = 0.01 ([MoDE] Auxiliary Load Balancing Loss;
    [Every] A balance penalty)."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    E = g["mixtral_routing"]["E"]
    logits = np.zeros((4, E))
    count = np.full(E, 1)
    _, _, loss = oracle.balance_stats(logits, count, k=2)  # default alpha
    # uniform routing: loss equals alpha exactly
    assert loss == pytest.approx(g["balance_alpha"]["value"], rel=1e-15)


# ---------------------------------------------------------------------------
# Worked examples (closed forms derived by hand)
# ---------------------------------------------------------------------------
def test_gates_worked():
    """[Every] The gating network: keep the top k, renormalise to sum to one."""
    l = np.array([[1.0, 3.0, 2.0, 0.5]])
    idx = oracle.top_k(l, 2)
    assert idx.tolist() == [[1, 2]]
    g = oracle.gates(l, idx)
    # m = 3: weights 1 and e^-1, so g = (e/(e+1), 1/(e+1))
    np.testing.assert_allclose(g[0], [sig(1.0), sig(-1.0)], rtol=1e-15)


def test_gates_worked_k_equals_E():
    """k = E keeps every expert: the full softmax ([Every] The gating network)."""
    l = np.array([[0.0, math.log(2.0), math.log(5.0)]])
    idx = oracle.top_k(l, 3)
    assert idx.tolist() == [[2, 1, 0]]
    np.testing.assert_allclose(oracle.gates(l, idx)[0], [5 / 8, 2 / 8, 1 / 8], rtol=1e-14)


def test_ties_lower_index_and_slot_order():
    """Ties go to the lower index, in membership and slot order (reading of a
    point the pages leave open)."""
    l = np.array([[0.5, 0.5, 0.5, 0.5], [-1.0, 7.0, 7.0, 7.0], [0.0, -0.0, 0.0, 1.0]])
    idx = oracle.top_k(l, 3)
    assert idx.tolist() == [[0, 1, 2], [1, 2, 3], [3, 0, 1]]
    g = oracle.gates(l, idx)
    np.testing.assert_allclose(g[0], [1 / 3] * 3, rtol=1e-15)
    assert oracle.gates(l[1:2], oracle.top_k(l[1:2], 1)).tolist() == [[1.0]]


def test_selection_bias_worked():
    """[ZenMax] Auxiliary-Loss-Free Load Balancing: the bias moves the choice;
    reading: gates still come from the unbiased logits."""
    l = np.array([[0.0, 0.5, 1.0]])
    b = np.array([2.0, 0.0, 0.0])
    idx = oracle.top_k(oracle.selection_keys(l, b), 2)
    assert idx.tolist() == [[0, 2]]
    # gates: softmax of the unbiased (0.0, 1.0), not of the keys (2.0, 1.0)
    np.testing.assert_allclose(oracle.gates(l, idx)[0], [sig(-1.0), sig(1.0)], rtol=1e-15)


def test_selection_key_float32_decision():
    """With float32 logits the key is one float32 add: 1 + 2^-24 rounds to 1
    (ties to even), so the two experts tie and the lower index wins; 1 + 2^-23
    is representable and wins."""
    l = np.array([[1.0, 1.0]], dtype=np.float32)
    for eps, want in ((2.0 ** -24, 0), (2.0 ** -23, 1)):
        b = np.array([0.0, eps], dtype=np.float32)
        keys = oracle.selection_keys(l, b)
        assert keys.dtype == np.float32
        assert oracle.top_k(keys, 1).tolist() == [[want]]


def test_swiglu_worked():
    """[ZenMax] Fine-Grained Expert Architecture, expert equation, on d = 2, h = 1:
    x = (1, 2), gate row (1, 0) -> u = 1, up row (0, 1) -> v = 2,
    down column (1, -3): y = 2 silu(1) (1, -3) = 2 e/(1+e) (1, -3)."""
    y = oracle.swiglu(np.array([[1.0, 2.0]]), np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]]),
                      np.array([[1.0], [-3.0]]))
    np.testing.assert_allclose(y[0], [2 * sig(1.0), -6 * sig(1.0)], rtol=1e-15)


def _worked_layer():
    """A 3-token, 3-expert, k = 2, h = 1 layer worked by hand.
    Router rows (1,0), (0,1), (-1,-1); tokens (1,0), (0,1), (-1,-1):
      t0 logits (1, 0, -1) -> experts (0, 1), gates (s(1), s(-1))
      t1 logits (0, 1, -1) -> experts (1, 0), gates (s(1), s(-1))
      t2 logits (-1, -1, 2) -> experts (2, 0) (0 beats 1 on the tie),
                               gates (s(3), s(-3))
    Experts: 0: g (1,0) u (1,0) d (1,0)^T;  1: g (1,1) u (2,0) d (0,1)^T;
             2: g (-1,0) u (0,-1) d (1,1)^T.  Shared: g (1,0) u (1,0) d (0,1)^T.
    """
    x = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, -1.0]])
    wr = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, -1.0]])
    wg = np.array([[[1.0, 0.0]], [[1.0, 1.0]], [[-1.0, 0.0]]])
    wu = np.array([[[1.0, 0.0]], [[2.0, 0.0]], [[0.0, -1.0]]])
    wd = np.array([[[1.0], [0.0]], [[0.0], [1.0]], [[1.0], [1.0]]])
    shared = [(np.array([[1.0, 0.0]]), np.array([[1.0, 0.0]]), np.array([[0.0], [1.0]]))]
    return x, wr, wg, wu, wd, shared


def test_layer_worked_capacity_one():
    """[Every] A budget (capacity 1, token order), The gating network (weighted
    sum), A shared expert (added with weight one)."""
    x, wr, wg, wu, wd, shared = _worked_layer()
    s1, sm1, s3 = sig(1.0), sig(-1.0), sig(3.0)
    r = oracle.forward(x, wr, wg, wu, wd, k=2, shared=shared, cap=1)
    assert r["topk_idx"].tolist() == [[0, 1], [1, 0], [2, 0]]
    assert r["count"].tolist() == [3, 2, 1]
    assert r["kept"].tolist() == [1, 1, 1]
    assert r["offset"].tolist() == [0, 1, 2, 3]
    assert r["pair_row"].tolist() == [0, 1, -1, -1, 2, -1]
    assert r["row_pair"].tolist() == [0, 1, 4, -1, -1, -1]
    want = np.array([[s1 * s1, 2 * sm1 * s1 + s1],
                     [0.0, 0.0],
                     [s3 * s1, s3 * s1 + sm1]])
    np.testing.assert_allclose(r["y"], want, rtol=1e-14, atol=1e-15)
    # balance: f = count / (T k) = (3, 2, 1) / 6
    np.testing.assert_allclose(r["f"], [0.5, 1 / 3, 1 / 6], rtol=1e-15)


def test_layer_worked_no_capacity():
    x, wr, wg, wu, wd, shared = _worked_layer()
    s1, sm1, s3, sm3 = sig(1.0), sig(-1.0), sig(3.0), sig(-3.0)
    r = oracle.forward(x, wr, wg, wu, wd, k=2, shared=shared)
    # t1 = (0,1): expert 1 u = 1, v = 0 -> 0; expert 0 u = 0 -> 0; shared 0
    # t2 = (-1,-1): expert 2 u = 1, v = 1 -> s(1)(1,1); expert 0 u = -1, v = -1 -> s(-1)(1,0)
    want = np.array([[s1 * s1, 2 * sm1 * s1 + s1],
                     [0.0, 0.0],
                     [s3 * s1 + sm3 * sm1, s3 * s1 + sm1]])
    np.testing.assert_allclose(r["y"], want, rtol=1e-14, atol=1e-15)


def test_balance_worked():
    """[MoDE] Auxiliary Load Balancing Loss on T = 2, E = 2, k = 1:
    logits (ln 3, 0) and (0, 0): p = (3/4, 1/4) and (1/2, 1/2), P = (5/8, 3/8);
    both tokens pick expert 0 (the second on a tie), f = (1, 0);
    L = 0.01 * 2 * 5/8 = 0.0125."""
    l = np.array([[math.log(3.0), 0.0], [0.0, 0.0]])
    idx = oracle.top_k(l, 1)
    assert idx.tolist() == [[0], [0]]
    d = oracle.dispatch(idx, 2)
    f, P, loss = oracle.balance_stats(l, d["count"], k=1)
    np.testing.assert_allclose(f, [1.0, 0.0])
    np.testing.assert_allclose(P, [5 / 8, 3 / 8], rtol=1e-15)
    assert loss == pytest.approx(0.0125, rel=1e-14)
    # k = E = 2 on the same logits: f = (1/2, 1/2), L = 0.02 * (5/16 + 3/16) = 0.01
    d2 = oracle.dispatch(oracle.top_k(l, 2), 2)
    _, _, loss2 = oracle.balance_stats(l, d2["count"], k=2)
    assert loss2 == pytest.approx(0.01, rel=1e-14)


def test_capacity_worked():
    """C = ceil(cf * T * k / E) ([MoDE] Adaptive Capacity Factors, with k and
    rounding up), checked on hand-computed cases."""
    assert oracle.capacity(1.25, 16384, 2, 64) == 640
    assert oracle.capacity(1.0, 10, 2, 3) == 7          # ceil(20/3)
    assert oracle.capacity(1.25, 100, 2, 8) == 32       # ceil(31.25)
    assert oracle.capacity(2.0, 3, 1, 2) == 3
    assert oracle.capacity(1.0, 64, 2, 8) == 16         # exact, no rounding up
    assert oracle.capacity(0.5, 1, 1, 8) == 1           # any positive budget is >= 1
    # the factor is the decimal the caller wrote: 0.1 * 10 = 1 and 1.1 * 100 / 10 = 11
    # (the binary doubles nearest 0.1 and 1.1 are slightly larger)
    assert oracle.capacity(0.1, 10, 1, 1) == 1
    assert oracle.capacity(1.1, 100, 1, 10) == 11
    assert oracle.capacity(0.0, 10, 2, 3) is oracle.UNLIMITED
    assert oracle.capacity(None, 10, 2, 3) is oracle.UNLIMITED


def test_router_z_loss_closed_form():
    """[ZenMax] MoE-Specific Training Stability: equal logits c over E experts
    give log-sum-exp c + ln E, so the loss is (c + ln E)^2."""
    E = 16
    for c in (0.0, 2.5, -3.0):
        l = np.full((5, E), c)
        assert oracle.router_z_loss(l) == pytest.approx((c + math.log(E)) ** 2, rel=1e-14)


# ---------------------------------------------------------------------------
# SiLU
# ---------------------------------------------------------------------------
def test_silu_special_values():
    z = np.array([-800.0, -30.0, -1.0, 0.0, 1.0, 30.0, 800.0])
    s = oracle.silu(z)
    assert s[3] == 0.0
    assert s[-1] == 800.0 and s[0] == 0.0 and math.copysign(1, s[0]) == -1.0
    np.testing.assert_allclose(s, z * scipy.special.expit(z), rtol=1e-15, atol=0)
    zz = np.linspace(-20, 20, 4001)
    np.testing.assert_allclose(oracle.silu(zz), zz * scipy.special.expit(zz), rtol=2e-15, atol=1e-300)


# ---------------------------------------------------------------------------
# Special cases that reduce to library routines
# ---------------------------------------------------------------------------
def test_router_one_hot_selects_columns():
    """Router rows that are unit vectors give logits equal to columns of x."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 5))
    cols = [3, 0, 4]
    wr = np.eye(5)[cols]
    np.testing.assert_array_equal(oracle.router_logits(x, wr), x[:, cols])
    lb = np.array([0.25, -1.0, 2.0])
    np.testing.assert_array_equal(oracle.router_logits(x, wr, lb), x[:, cols] + lb)


def test_single_expert_is_plain_swiglu():
    """E = 1, k = 1, no shared: the layer is one SwiGLU FFN (library form)."""
    rng = np.random.default_rng(2)
    x, wr, wg, wu, wd, _ = rand_layer(rng, T=9, d=6, E=1, h=10)
    r = oracle.forward(x, wr, wg, wu, wd, k=1)
    assert (r["topk_gate"] == 1.0).all()
    np.testing.assert_allclose(r["y"], torch_swiglu(x, wg[0], wu[0], wd[0]), rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_soft_mixture():
    """[Every] The gating network: a softmax over every expert is the soft
    mixture y = sum_e softmax(l)_e FFN_e(x)."""
    rng = np.random.default_rng(3)
    x, wr, wg, wu, wd, _ = rand_layer(rng, T=11, d=5, E=4, h=7)
    r = oracle.forward(x, wr, wg, wu, wd, k=4)
    p = scipy.special.softmax(x @ wr.T, axis=1)
    want = sum(p[:, e:e + 1] * torch_swiglu(x, wg[e], wu[e], wd[e]) for e in range(4))
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-14)


def test_identical_experts_reduce_to_one_ffn():
    """Identical experts with no drops: gates sum to one, so y = FFN(x) + shared
    for any router."""
    rng = np.random.default_rng(4)
    x, wr, wg, wu, wd, shared = rand_layer(rng, T=13, d=6, E=5, h=8, n_shared=2, hs=3)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    r = oracle.forward(x, wr, wg, wu, wd, k=3, shared=shared)
    want = torch_swiglu(x, wg[0], wu[0], wd[0]) + sum(torch_swiglu(x, *s) for s in shared)
    np.testing.assert_allclose(r["y"], want, rtol=1e-12, atol=1e-13)


def test_shared_concat_identity():
    """sum_s SwiGLU_s(x) = one SwiGLU whose hidden axis concatenates the shared
    experts (the form the library evaluates)."""
    rng = np.random.default_rng(5)
    x, _, _, _, _, shared = rand_layer(rng, T=6, d=5, E=1, h=2, n_shared=3, hs=4)
    cat = (np.concatenate([s[0] for s in shared]), np.concatenate([s[1] for s in shared]),
           np.concatenate([s[2] for s in shared], axis=1))
    np.testing.assert_allclose(sum(oracle.swiglu(x, *s) for s in shared), torch_swiglu(x, *cat),
                               rtol=1e-12, atol=1e-14)


def test_zero_router_routes_to_first_experts():
    """W_r = 0: every key ties, so each token takes experts 0..k-1 in that
    order with gates 1/k; and P is uniform, so the balance loss is alpha."""
    rng = np.random.default_rng(6)
    x, wr, wg, wu, wd, _ = rand_layer(rng, T=10, d=4, E=6, h=3)
    wr[:] = 0.0
    r = oracle.forward(x, wr, wg, wu, wd, k=3)
    assert r["topk_idx"].tolist() == [[0, 1, 2]] * 10
    np.testing.assert_allclose(r["topk_gate"], 1 / 3, rtol=1e-15)
    np.testing.assert_allclose(r["P"], 1 / 6, rtol=1e-15)
    assert r["loss"] == pytest.approx(0.01, rel=1e-14)


def test_capacity_zero_leaves_shared_only():
    rng = np.random.default_rng(7)
    x, wr, wg, wu, wd, shared = rand_layer(rng, T=8, d=4, E=4, h=3, n_shared=1, hs=5)
    r = oracle.forward(x, wr, wg, wu, wd, k=2, shared=shared, cap=0)
    assert (r["pair_row"] == -1).all() and r["offset"][-1] == 0
    np.testing.assert_allclose(r["y"], torch_swiglu(x, *shared[0]), rtol=1e-12, atol=1e-14)


def test_capacity_at_least_T_drops_nothing():
    rng = np.random.default_rng(8)
    x, wr, wg, wu, wd, _ = rand_layer(rng, T=12, d=4, E=3, h=3)
    a = oracle.forward(x, wr, wg, wu, wd, k=2, cap=12)
    b = oracle.forward(x, wr, wg, wu, wd, k=2)
    assert (a["pair_row"] >= 0).all()
    np.testing.assert_array_equal(a["pair_row"], b["pair_row"])
    np.testing.assert_array_equal(a["y"], b["y"])


def test_uniform_f_gives_alpha():
    """f uniform gives L = alpha whatever P is (sum P = 1)."""
    rng = np.random.default_rng(9)
    E = 5
    l = rng.standard_normal((E, E)) + 10 * np.eye(E)  # token t picks expert t
    idx = oracle.top_k(l, 1)
    assert idx[:, 0].tolist() == list(range(E))
    d = oracle.dispatch(idx, E)
    f, P, loss = oracle.balance_stats(l, d["count"], k=1)
    np.testing.assert_allclose(f, 1 / E)
    assert loss == pytest.approx(0.01, rel=1e-13)


# ---------------------------------------------------------------------------
# Property tests and brute force on tiny inputs
# ---------------------------------------------------------------------------
shapes = st.tuples(st.integers(1, 12), st.integers(1, 5), st.integers(1, 6), st.integers(1, 4))


@settings(max_examples=60, deadline=None)
@given(shapes, st.integers(0, 2 ** 31 - 1), st.booleans())
def test_gates_simplex(shape, seed, ties):
    """[Every] The gating network: gates are non-negative and sum to one."""
    T, _, E, k = shape
    k = min(k, E)
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)) * 5
    if ties:
        l = np.round(l)
    g = oracle.gates(l, oracle.top_k(l, k))
    assert (g >= 0).all()
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)
    if k == 1:
        assert (g == 1.0).all()


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 8), st.integers(1, 3), st.integers(0, 2 ** 31 - 1), st.booleans())
def test_topk_brute_force(E, k, seed, ties):
    """Top-k equals exhaustive subset search (max key sum, lexicographically
    smallest on ties) and the slot order equals repeated max selection."""
    k = min(k, E)
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((6, E))
    if ties:
        keys = np.round(keys)
    idx = oracle.top_k(keys, k)
    for t in range(6):
        kt = keys[t].tolist()
        assert tuple(sorted(idx[t].tolist())) == brute.best_subset(kt, k)
        assert idx[t].tolist() == brute.topk_by_selection(kt, k)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 30), st.integers(1, 7), st.integers(1, 4), st.integers(-1, 12),
       st.integers(0, 2 ** 31 - 1))
def test_dispatch_invariants(T, E, k, cap, seed):
    """[Every] A budget, in token order: bijection, contiguity, ascending token
    order inside each expert, offsets = exclusive scan of min(count, C), and the
    kept set of each expert is its first C tokens (brute-force walk)."""
    k = min(k, E)
    cap = None if cap < 0 else cap
    rng = np.random.default_rng(seed)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    d = oracle.dispatch(idx, E, cap)
    R = T * k
    kept_bf, count_bf = brute.route_and_drop(idx.tolist(), E, cap)
    assert d["count"].tolist() == count_bf
    want_kept = [min(c, cap) if cap is not None else c for c in count_bf]
    assert d["kept"].tolist() == want_kept
    assert d["offset"].tolist() == [0] + list(np.cumsum(want_kept))
    pr, rp = d["pair_row"], d["row_pair"]
    Rk = d["offset"][-1]
    kept_mask = np.array(kept_bf, dtype=bool).reshape(-1) if R else np.zeros(0, bool)
    assert ((pr >= 0) == kept_mask).all()
    assert sorted(pr[pr >= 0].tolist()) == list(range(Rk))
    assert (rp[Rk:] == -1).all()
    for row in range(Rk):
        assert pr[rp[row]] == row
    flat = idx.reshape(-1)
    for e in range(E):
        rows = range(d["offset"][e], d["offset"][e + 1])
        pairs = [rp[r] for r in rows]
        assert all(flat[p] == e for p in pairs)
        assert pairs == sorted(pairs)


@settings(max_examples=25, deadline=None)
@given(st.integers(1, 6), st.integers(1, 3), st.integers(1, 4), st.integers(1, 3), st.integers(-1, 4),
       st.integers(0, 2), st.booleans(), st.booleans(), st.integers(0, 2 ** 31 - 1))
def test_whole_layer_brute_force(T, d, E, h, cap, n_shared, lbias, sbias, seed):
    """The sparse oracle equals the dense evaluation (every expert on every
    token, zero gates for unselected or dropped experts) in pure Python."""
    k = 1 + seed % E
    cap = None if cap < 0 else cap
    rng = np.random.default_rng(seed)
    x, wr, wg, wu, wd, shared = rand_layer(rng, T, d, E, h, n_shared, hs=2)
    lb = rng.standard_normal(E) if lbias else None
    sb = rng.standard_normal(E).astype(np.float32) if sbias else None
    logits = oracle.router_logits(x, wr, lb)
    if sb is not None:
        logits = logits.astype(np.float32)  # the selection decision in float32
    r = oracle.forward(x, wr, wg, wu, wd, k, shared=shared, logit_bias=lb, select_bias=sb,
                       cap=cap, logits=logits)
    want = brute.dense_layer(x.tolist(), wr.tolist(), wg.tolist(), wu.tolist(), wd.tolist(), k,
                             cap=cap, shared=[tuple(a.tolist() for a in s) for s in shared],
                             logit_bias=None if lb is None else lb.tolist(),
                             select_bias=None if sb is None else sb.tolist())
    np.testing.assert_allclose(r["y"], np.array(want), rtol=1e-5 if sb is not None else 1e-12,
                               atol=1e-6 if sb is not None else 1e-13)


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 20), st.integers(1, 9), st.integers(1, 4), st.integers(0, 2 ** 31 - 1))
def test_balance_bounds(T, E, k, seed):
    """Sum f = 1, sum P = 1, 0 <= L <= alpha * E."""
    k = min(k, E)
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)) * 4
    d = oracle.dispatch(oracle.top_k(l, k), E)
    f, P, loss = oracle.balance_stats(l, d["count"], k)
    assert f.sum() == pytest.approx(1.0, rel=1e-14)
    assert P.sum() == pytest.approx(1.0, rel=1e-14)
    assert 0 <= loss <= 0.01 * E * (1 + 1e-14)


def test_tokens_subset_matches_full():
    """Computing a subset of output rows gives the same rows as the full pass."""
    rng = np.random.default_rng(10)
    x, wr, wg, wu, wd, shared = rand_layer(rng, T=20, d=6, E=5, h=4, n_shared=1, hs=3)
    full = oracle.forward(x, wr, wg, wu, wd, k=2, shared=shared, cap=5)
    sub = oracle.forward(x, wr, wg, wu, wd, k=2, shared=shared, cap=5, tokens=[3, 17, 0])
    np.testing.assert_allclose(sub["y"], full["y"][[3, 17, 0]], rtol=1e-13, atol=1e-15)
