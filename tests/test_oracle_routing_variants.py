"""Pins of the routing-variant oracle (ReLU routing, zero-computation
experts) from "Zen MoDE: Mixture of Diverse Experts", section
"Router": worked values, closed forms, special cases that reduce to the plain
layer, and pure-Python brute force from the definitions (``tests/brute.py``
style loops, written here without the oracle's code).  The last test plants
plausible mistakes in the oracle (on the CPU) and checks that a pin fails."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import moe_variants as mv
from tests import brute

E_FFN, D, H = 5, 8, 6


def _layer(seed, E_router, k_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, D))
    wr = rng.standard_normal((E_router, D)) * k_scale
    wg = rng.standard_normal((E_FFN, H, D)) / math.sqrt(D)
    wu = rng.standard_normal((E_FFN, H, D)) / math.sqrt(D)
    wd = rng.standard_normal((E_FFN, D, H)) / math.sqrt(H)
    return rng, x, wr, wg, wu, wd


def _expert(x_row, wg, wu, wd, e):
    return brute.expert(list(x_row), wg[e].tolist(), wu[e].tolist(), wd[e].tolist())


# ---------------------------------------------------------------- ReLU routing
def test_relu_route_worked():
    """Positive logits only, descending, ties to the lower index, -1 padding."""
    logits = np.array([[2.0, -1.0, 0.0, 3.0], [-1.0, -2.0, -3.0, -4.0], [1.0, 1.0, 1.0, 1.0],
                       [0.5, 4.0, 0.25, -0.0]])
    idx, g = oracle.relu_route(logits, 4)
    assert idx.tolist() == [[3, 0, -1, -1], [-1, -1, -1, -1], [0, 1, 2, 3], [1, 0, 2, -1]]
    assert g.tolist() == [[3, 2, 0, 0], [0, 0, 0, 0], [1, 1, 1, 1], [4, 0.5, 0.25, 0]]


def test_relu_route_k_max_keeps_largest():
    idx, g = oracle.relu_route(np.array([[3.0, 5.0, 4.0, 1.0], [2.0, 2.0, 2.0, 7.0]]), 2)
    assert idx.tolist() == [[1, 2], [3, 0]]
    assert g.tolist() == [[5, 4], [7, 2]]


def test_relu_route_closed_forms():
    """With k_max = E every positive expert is used: the used count equals the
    number of positive logits and the gates sum to sum_e max(l_e, 0)."""
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((200, 9))
    idx, g = oracle.relu_route(logits, 9)
    assert np.array_equal((idx >= 0).sum(axis=1), (logits > 0).sum(axis=1))
    np.testing.assert_allclose(g.sum(axis=1), np.maximum(logits, 0).sum(axis=1), rtol=1e-15)
    assert np.all(g[idx < 0] == 0)
    for t in range(200):
        used = idx[t][idx[t] >= 0]
        assert np.all(np.diff(logits[t, used]) <= 0)
        assert np.array_equal(g[t, :used.size], logits[t, used])


def test_forward_relu_brute():
    """y_t = sum over all experts of max(l_te, 0) E_e(x_t) (k_max = E, no
    budget), written as a loop over experts, not over slots."""
    rng, x, wr, wg, wu, wd = _layer(2, E_FFN)
    res = oracle.forward_relu(x, wr, wg, wu, wd, E_FFN)
    logits = x @ wr.T
    for t in range(x.shape[0]):
        want = [0.0] * D
        for e in range(E_FFN):
            if logits[t, e] > 0:
                out = _expert(x[t], wg, wu, wd, e)
                want = [a + logits[t, e] * b for a, b in zip(want, out)]
        np.testing.assert_allclose(res["y"][t], want, rtol=1e-12, atol=1e-12)


def test_forward_relu_budget_and_stats():
    """Unused slots take no budget: the count per expert is the number of
    tokens with a positive logit there (k_max = E); a budget keeps the first
    tokens in token order; f uses T k_max."""
    rng, x, wr, wg, wu, wd = _layer(3, E_FFN)
    logits = x @ wr.T
    res = oracle.forward_relu(x, wr, wg, wu, wd, E_FFN, cap=2)
    assert np.array_equal(res["count"], (logits > 0).sum(axis=0))
    assert np.array_equal(res["kept"], np.minimum((logits > 0).sum(axis=0), 2))
    pr = res["pair_row"].reshape(7, E_FFN)
    for e in range(E_FFN):
        toks = [t for t in range(7) if logits[t, e] > 0]
        kept_toks = sorted(t for t in range(7) for j in range(E_FFN)
                           if res["topk_idx"][t, j] == e and pr[t, j] >= 0)
        assert kept_toks == toks[:2]
    np.testing.assert_allclose(res["f"], res["count"] / (7 * E_FFN))


def test_forward_relu_all_negative_is_shared_only():
    rng, x, wr, wg, wu, wd = _layer(4, E_FFN)
    sh = (rng.standard_normal((4, D)), rng.standard_normal((4, D)), rng.standard_normal((D, 4)))
    logits = -np.abs(rng.standard_normal((7, E_FFN))) - 0.1
    res = oracle.forward_relu(x, wr, wg, wu, wd, 3, shared=[sh], logits=logits)
    assert np.all(res["topk_idx"] == -1) and res["offset"][-1] == 0
    np.testing.assert_allclose(res["y"], oracle.swiglu(x, *sh), rtol=1e-14)


# ------------------------------------------------- zero-computation experts
def test_bypass_numbering():
    kinds = [oracle.bypass_kind(e, 3, 2, 1, 2) for e in range(8)]
    assert kinds == [("ffn", 0), ("ffn", 1), ("ffn", 2), ("zero", 0), ("zero", 1), ("copy", 0),
                     ("const", 0), ("const", 1)]
    with pytest.raises(ValueError):
        oracle.bypass_kind(8, 3, 2, 1, 2)


def _forced_logits(T, E, choice, second=None):
    lg = np.zeros((T, E))
    lg[:, choice] = 5.0
    if second is not None:
        lg[:, second] = 4.0
    return lg


def test_bypass_copy_is_identity():
    """Every token on a copy expert with k = 1: y = x exactly, no FFN rows."""
    rng, x, _, wg, wu, wd = _layer(5, 0)
    n_zero, n_copy, cv = 1, 2, rng.standard_normal((1, D))
    E = E_FFN + n_zero + n_copy + 1
    wr = np.zeros((E, D))
    res = oracle.forward_bypass(x, wr, wg, wu, wd, 1, n_zero, n_copy, cv,
                                logits=_forced_logits(7, E, E_FFN + n_zero + 1))
    assert np.array_equal(res["y"], x)
    assert res["offset"][-1] == 0 and np.all(res["pair_row"] == -1)
    assert res["count"][E_FFN + n_zero + 1] == 7


def test_bypass_constant_and_zero():
    """A constant expert gives its vector; a zero expert gives nothing, and the
    FFN expert beside it keeps its renormalised gate."""
    rng, x, _, wg, wu, wd = _layer(6, 0)
    cv = rng.standard_normal((2, D))
    E = E_FFN + 1 + 1 + 2
    res = oracle.forward_bypass(x, np.zeros((E, D)), wg, wu, wd, 1, 1, 1, cv,
                                logits=_forced_logits(7, E, E - 1))
    np.testing.assert_allclose(res["y"], np.broadcast_to(cv[1], (7, D)), rtol=0, atol=0)
    res = oracle.forward_bypass(x, np.zeros((E, D)), wg, wu, wd, 2, 1, 1, cv,
                                logits=_forced_logits(7, E, 2, second=E_FFN))
    g0 = 1.0 / (1.0 + math.exp(-1.0))
    for t in range(7):
        want = [g0 * v for v in _expert(x[t], wg, wu, wd, 2)]
        np.testing.assert_allclose(res["y"][t], want, rtol=1e-12, atol=1e-14)


def _brute_bypass(x, logits, k, wg, wu, wd, n_zero, n_copy, cv, cap):
    """Per-token definition: softmax over the k best (ties low), kinds by
    position, budget per FFN expert in token order."""
    T, E = logits.shape
    used = [0] * E_FFN
    y = []
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        m = max(logits[t, e] for e in order)
        w = [math.exp(logits[t, e] - m) for e in order]
        s = sum(w)
        acc = [0.0] * D
        for e, wj in zip(order, w):
            g = wj / s
            if e < E_FFN:
                if cap is not None and used[e] >= cap:
                    used[e] += 1
                    continue
                used[e] += 1
                out = _expert(x[t], wg, wu, wd, e)
            elif e < E_FFN + n_zero:
                out = [0.0] * D
            elif e < E_FFN + n_zero + n_copy:
                out = list(x[t])
            else:
                out = list(cv[e - E_FFN - n_zero - n_copy])
            acc = [a + g * b for a, b in zip(acc, out)]
        y.append(acc)
    return np.array(y)


@pytest.mark.parametrize("k,cap,seed", [(1, None, 7), (2, None, 8), (3, 1, 9), (4, 2, 10)])
def test_forward_bypass_brute(k, cap, seed):
    n_zero, n_copy, n_const = 2, 1, 2
    E = E_FFN + n_zero + n_copy + n_const
    rng, x, wr, wg, wu, wd = _layer(seed, E, k_scale=0.8)
    cv = rng.standard_normal((n_const, D))
    res = oracle.forward_bypass(x, wr, wg, wu, wd, k, n_zero, n_copy, cv, cap=cap)
    want = _brute_bypass(x, x @ wr.T, k, wg, wu, wd, n_zero, n_copy, cv, cap)
    np.testing.assert_allclose(res["y"], want, rtol=1e-12, atol=1e-12)
    # statistics over all router experts, counts before any drop
    idx = res["topk_idx"]
    assert np.array_equal(res["count"], np.bincount(idx.ravel(), minlength=E))
    assert math.isclose(res["f"].sum(), 1.0, rel_tol=1e-15)
    assert np.all(res["kept"][E_FFN:] == 0)


def test_forward_bypass_without_bypass_is_plain_layer():
    rng, x, wr, wg, wu, wd = _layer(11, E_FFN)
    a = oracle.forward_bypass(x, wr, wg, wu, wd, 2, 0, 0, np.zeros((0, D)), cap=2)
    b = oracle.forward(x, wr, wg, wu, wd, 2, cap=2)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["pair_row"], b["pair_row"])


# ------------------------------------------------------------- mutations
def _relu_keeps_zero(logits, k_max):
    l = np.asarray(logits, dtype=np.float64)
    idx, g = mv.__dict__["_orig_relu_route"](np.where(l == 0, 1e-300, l), k_max)
    return idx, np.where(idx >= 0, np.take_along_axis(l, np.maximum(idx, 0), 1), 0.0)


def _relu_renormalised(logits, k_max):
    idx, g = mv.__dict__["_orig_relu_route"](logits, k_max)
    s = g.sum(axis=1, keepdims=True)
    return idx, np.where(s > 0, g / np.where(s > 0, s, 1), 0.0)


def _kind_copy_const_swapped(e, E_ffn, n_zero, n_copy, n_const):
    kind, i = mv.__dict__["_orig_bypass_kind"](e, E_ffn, n_zero, n_copy, n_const)
    if kind == "copy" and n_const:
        return "const", 0
    return kind, i


def _bypass_output_no_gate(x, idx, gate, *a, **kw):
    return mv.__dict__["_orig_bypass_output"](x, idx, np.ones_like(np.asarray(gate)), *a, **kw)


MUTATIONS = {
    "relu keeps a zero logit": ("relu_route", _relu_keeps_zero),
    "relu gates renormalised": ("relu_route", _relu_renormalised),
    "copy and constant swapped": ("bypass_kind", _kind_copy_const_swapped),
    "bypass ignores its gate": ("bypass_output", _bypass_output_no_gate),
}

PIN_TESTS = [
    test_relu_route_worked, test_relu_route_closed_forms, test_forward_relu_brute,
    test_bypass_copy_is_identity, test_bypass_constant_and_zero,
    lambda: test_forward_bypass_brute(2, None, 8), lambda: test_forward_bypass_brute(3, 1, 9),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setitem(mv.__dict__, f"_orig_{fn_name}", getattr(mv, fn_name))
    monkeypatch.setattr(mv, fn_name, bad)
    if fn_name == "relu_route":
        monkeypatch.setattr(oracle, "relu_route", bad)
    failed = 0
    for pin in PIN_TESTS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {name}"


# ------------------------------------------------------ ReLU routing backward
RELU_BWD_CASES = [
    # T, d, E, h, k_max, cap, n_shared, c_bal, c_z, seed
    (7, 5, 4, 3, 4, None, 0, 0.0, 0.0, 21),
    (9, 4, 6, 3, 2, 3, 1, 1.0, 0.0, 22),
    (8, 6, 5, 4, 3, 2, 0, 0.5, 0.3, 23),
]


def _relu_setup(case):
    T, d, E, h, k_max, cap, ns, cb, cz, seed = case
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    wg = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, h)) / math.sqrt(h)
    shared = [(rng.standard_normal((4, d)), rng.standard_normal((4, d)),
               rng.standard_normal((d, 4))) for _ in range(ns)]
    lb = 0.5 * rng.standard_normal(E)
    dy = rng.standard_normal((T, d))
    params = dict(x=x, w_router=wr, w_gate=wg, w_up=wu, w_down=wd, logit_bias=lb)
    kw = dict(shared=shared, cap=cap, alpha=0.01, c_bal=cb, c_z=cz)
    return params, k_max, dy, kw


def _relu_J(params, k_max, dy, kw):
    p = params
    return oracle.objective_relu(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], k_max,
                                 dy, logit_bias=p["logit_bias"], **kw)


@pytest.mark.parametrize("case", RELU_BWD_CASES)
def test_relu_backward_finite_differences(case):
    """Every gradient of the ReLU-routed layer equals the central difference
    of its forward objective along random directions (selection fixed)."""
    params, k_max, dy, kw = _relu_setup(case)
    p = params
    g = oracle.backward_relu(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], k_max,
                             dy, logit_bias=p["logit_bias"], **kw)
    _, idx0 = _relu_J(params, k_max, dy, kw)
    assert np.any(idx0 < 0) or case[4] < case[2]  # the case exercises empty or left-out slots
    rng = np.random.default_rng(5)
    eps = 1e-6
    names = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
             "w_down": "dw_down", "logit_bias": "dlogit_bias"}
    for name, gname in names.items():
        for _ in range(2):
            V = rng.standard_normal(params[name].shape)
            Jp, ip = _relu_J(dict(params, **{name: params[name] + eps * V}), k_max, dy, kw)
            Jm, im = _relu_J(dict(params, **{name: params[name] - eps * V}), k_max, dy, kw)
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "selection moved"
            ana = float(np.sum(g[gname] * V))
            assert abs((Jp - Jm) / (2 * eps) - ana) <= 1e-6 * (1.0 + abs(ana)), (name, ana)


def test_relu_backward_autograd():
    """The ReLU-routed layer written in PyTorch as a sum over all experts of
    relu(l) E(x) (k_max = E, no budget), differentiated by autograd."""
    F = torch.nn.functional
    params, k_max, dy, kw = _relu_setup((6, 4, 5, 3, 5, None, 0, 0.0, 0.0, 31))
    p = params
    g = oracle.backward_relu(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], k_max,
                             dy, logit_bias=p["logit_bias"], **kw)
    tp = {n: torch.tensor(v, requires_grad=True) for n, v in params.items()}
    logits = tp["x"] @ tp["w_router"].T + tp["logit_bias"]
    y = torch.zeros_like(tp["x"])
    for e in range(5):
        out = F.linear(F.silu(F.linear(tp["x"], tp["w_gate"][e])) * F.linear(tp["x"], tp["w_up"][e]),
                       tp["w_down"][e])
        y = y + torch.relu(logits[:, e:e + 1]) * out
    torch.sum(torch.as_tensor(dy) * y).backward()
    for n, gn in (("x", "dx"), ("w_router", "dw_router"), ("logit_bias", "dlogit_bias"),
                  ("w_gate", "dw_gate"), ("w_down", "dw_down")):
        np.testing.assert_allclose(g[gn], tp[n].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_relu_gate_logit_grad_worked():
    """Used slots pass dgate to their expert's logit; empty slots and unused
    experts get nothing."""
    idx = np.array([[2, 0, -1], [-1, -1, -1]])
    dg = np.array([[0.5, -2.0, 7.0], [1.0, 1.0, 1.0]])
    dl = oracle.relu_gate_logit_grad(np.zeros((2, 4)), idx, dg)
    assert dl.tolist() == [[-2.0, 0.0, 0.5, 0.0], [0.0, 0.0, 0.0, 0.0]]


def _relu_grad_through_softmax(logits, idx, dgate):
    from oracle.moe_backward import gate_logit_grad
    idx = np.asarray(idx, dtype=np.int64)
    safe = np.where(idx >= 0, idx, np.argmax(np.asarray(logits), axis=1)[:, None])
    return gate_logit_grad(logits, safe, np.where(idx >= 0, dgate, 0.0))


def _relu_grad_counts_empty_slots(logits, idx, dgate):
    dl = mv.__dict__["_orig_relu_gate_logit_grad"](logits, idx, dgate)
    dl[:, 0] += np.sum(np.where(np.asarray(idx) < 0, 1.0, 0.0), axis=1)
    return dl


MUTATIONS["relu backward through a softmax"] = ("relu_gate_logit_grad", _relu_grad_through_softmax)
MUTATIONS["relu backward feeds empty slots"] = ("relu_gate_logit_grad",
                                                _relu_grad_counts_empty_slots)
PIN_TESTS += [lambda: test_relu_backward_finite_differences(RELU_BWD_CASES[1]),
              lambda: test_relu_backward_finite_differences(RELU_BWD_CASES[2]),
              test_relu_gate_logit_grad_worked]


@pytest.mark.parametrize("name", ["relu backward through a softmax",
                                  "relu backward feeds empty slots"])
def test_backward_mutation_is_caught(name, monkeypatch):
    test_mutation_is_caught(name, monkeypatch)


# ------------------------------------------- zero-computation experts backward
BYPASS_BWD_CASES = [
    # T, d, E_ffn, h, k, n_zero, n_copy, n_const, cap, n_shared, c_bal, c_z, seed
    (7, 5, 4, 3, 2, 1, 1, 2, None, 0, 0.0, 0.0, 41),
    (9, 4, 3, 3, 3, 2, 1, 1, 2, 1, 1.0, 0.0, 42),
    (8, 6, 2, 4, 2, 0, 2, 2, 3, 0, 0.5, 0.3, 43),
]


def _bypass_setup(case):
    T, d, E_ffn, h, k, nz, nc, nk, cap, ns, cb, cz, seed = case
    rng = np.random.default_rng(seed)
    E = E_ffn + nz + nc + nk
    params = dict(x=rng.standard_normal((T, d)), w_router=rng.standard_normal((E, d)),
                  w_gate=rng.standard_normal((E_ffn, h, d)) / math.sqrt(d),
                  w_up=rng.standard_normal((E_ffn, h, d)) / math.sqrt(d),
                  w_down=rng.standard_normal((E_ffn, d, h)) / math.sqrt(h),
                  const_rows=rng.standard_normal((nk, d)))
    shared = [(rng.standard_normal((4, d)), rng.standard_normal((4, d)),
               rng.standard_normal((d, 4))) for _ in range(ns)]
    dy = rng.standard_normal((T, d))
    kw = dict(shared=shared, cap=cap, alpha=0.01, c_bal=cb, c_z=cz)
    return params, (k, nz, nc), dy, kw


def _bypass_J(params, kk, dy, kw):
    p = params
    k, nz, nc = kk
    return oracle.objective_bypass(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], k,
                                   nz, nc, p["const_rows"], dy, **kw)


@pytest.mark.parametrize("case", BYPASS_BWD_CASES)
def test_bypass_backward_finite_differences(case):
    """Every gradient of the layer with zero-computation experts, the
    constant rows' included, equals the central difference of its forward
    objective along random directions (selection fixed)."""
    params, kk, dy, kw = _bypass_setup(case)
    p = params
    g = oracle.backward_bypass(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], kk[0],
                               kk[1], kk[2], p["const_rows"], dy, **kw)
    _, idx0 = _bypass_J(params, kk, dy, kw)
    assert np.any(idx0 >= p["w_gate"].shape[0])  # some slots reach zero-computation experts
    rng = np.random.default_rng(6)
    eps = 1e-6
    names = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
             "w_down": "dw_down", "const_rows": "dconst"}
    for name, gname in names.items():
        for _ in range(2):
            V = rng.standard_normal(params[name].shape)
            Jp, ip = _bypass_J(dict(params, **{name: params[name] + eps * V}), kk, dy, kw)
            Jm, im = _bypass_J(dict(params, **{name: params[name] - eps * V}), kk, dy, kw)
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "selection moved"
            ana = float(np.sum(g[gname] * V))
            assert abs((Jp - Jm) / (2 * eps) - ana) <= 1e-6 * (1.0 + abs(ana)), (name, ana)


def test_bypass_backward_autograd():
    """The layer written in PyTorch per token from the definitions (copy =
    x, constant = v_c, zero = 0; softmax over the k selected), with the
    selection fixed, differentiated by autograd."""
    params, kk, dy, kw = _bypass_setup(BYPASS_BWD_CASES[0])
    k, nz, nc = kk
    p = params
    g = oracle.backward_bypass(p["x"], p["w_router"], p["w_gate"], p["w_up"], p["w_down"], k, nz,
                               nc, p["const_rows"], dy, **kw)
    idx = g["fwd"]["topk_idx"]
    F = torch.nn.functional
    tp = {n: torch.tensor(v, requires_grad=True) for n, v in params.items()}
    E_ffn = p["w_gate"].shape[0]
    logits = tp["x"] @ tp["w_router"].T
    J = 0.0
    for t in range(p["x"].shape[0]):
        sel = torch.as_tensor(idx[t].astype(np.int64))
        gt = torch.softmax(logits[t, sel], dim=0)
        for j, e in enumerate(idx[t]):
            if e < E_ffn:
                out = F.linear(F.silu(F.linear(tp["x"][t], tp["w_gate"][e])) *
                               F.linear(tp["x"][t], tp["w_up"][e]), tp["w_down"][e])
            elif e < E_ffn + nz:
                continue
            elif e < E_ffn + nz + nc:
                out = tp["x"][t]
            else:
                out = tp["const_rows"][e - E_ffn - nz - nc]
            J = J + gt[j] * torch.dot(torch.as_tensor(dy[t]), out)
    J.backward()
    for n, gn in (("x", "dx"), ("w_router", "dw_router"), ("const_rows", "dconst"),
                  ("w_gate", "dw_gate"), ("w_down", "dw_down")):
        np.testing.assert_allclose(g[gn], tp[n].grad.numpy(), rtol=1e-10, atol=1e-12)


def _bypass_gate_grad_no_copy(dy, x, idx, E_ffn, n_zero, n_copy, const_rows):
    return mv.__dict__["_orig_bypass_gate_grad"](dy, x, idx, E_ffn, n_zero + n_copy, 0, const_rows)


MUTATIONS["bypass backward drops the copy gate gradient"] = ("bypass_gate_grad",
                                                             _bypass_gate_grad_no_copy)
PIN_TESTS += [lambda: test_bypass_backward_finite_differences(BYPASS_BWD_CASES[0]),
              test_bypass_backward_autograd]


def test_bypass_backward_mutation_is_caught(monkeypatch):
    test_mutation_is_caught("bypass backward drops the copy gate gradient", monkeypatch)
