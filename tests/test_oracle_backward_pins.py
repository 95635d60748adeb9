"""Pins of the backward oracle against what the mathematics fixes.

The backward pass is the derivative of the forward, whose own pins live in
``test_oracle_pins``.  These tests pin ``oracle.backward`` and its parts to
that derivative without re-typing any of the oracle's formulas:

  * central finite differences of the pinned forward objective, parameter by
    parameter, with the selection checked to stay fixed;
  * PyTorch autograd (float64, CPU) of a forward written here from the layer's
    definition, on the oracle's own routing decisions (which are integers the
    forward pins already fix);
  * closed forms worked by hand and invariants (softmax Jacobian rows sum to
    zero; uniform load gives no balance gradient).

Sources: "Every parameter, every token", sections "The gating network" (the
selected set is held fixed, gradient flows through the gates of the experts
that ran), "A balance penalty" and "A budget"; "Zen MoDE: Mixture of Distilled Experts
Architecture", section "Auxiliary
Load Balancing Loss"; Zen-Max, sections "Fine-Grained Expert Architecture"
and "MoE-Specific Training Stability".
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _layer(rng, T, d, E, h, n_shared=0, hs=4):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    wg = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, h, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, h)) / math.sqrt(h)
    shared = [(rng.standard_normal((hs, d)) / math.sqrt(d), rng.standard_normal((hs, d)) / math.sqrt(d),
               rng.standard_normal((d, hs)) / math.sqrt(hs)) for _ in range(n_shared)]
    return x, wr, wg, wu, wd, shared


CASES = [
    # T, d, E, h, k, cap, n_shared, logit_bias, select_bias, c_bal, c_z, seed
    (7, 5, 4, 3, 2, None, 0, False, False, 0.0, 0.0, 1),
    (9, 4, 5, 3, 2, 3, 1, True, False, 1.0, 0.0, 2),
    (8, 6, 4, 4, 3, 4, 0, False, True, 0.0, 1e-3 * 100, 3),
    (6, 3, 3, 2, 1, 2, 2, True, True, 2.0, 0.5, 4),
    (5, 4, 4, 3, 4, None, 0, False, False, 1.0, 1.0, 5),  # k = E: the soft mixture
]


def _setup(case):
    T, d, E, h, k, cap, ns, lb, sb, cb, cz, seed = case
    rng = np.random.default_rng(seed)
    x, wr, wg, wu, wd, shared = _layer(rng, T, d, E, h, ns)
    lbias = rng.standard_normal(E) if lb else None
    sbias = 0.3 * rng.standard_normal(E) if sb else None
    dy = rng.standard_normal((T, d))
    kw = dict(shared=shared, logit_bias=lbias, select_bias=sbias, cap=cap, alpha=0.01,
              c_bal=cb, c_z=cz)
    params = dict(x=x, w_router=wr, w_gate=wg, w_up=wu, w_down=wd)
    return params, k, dy, kw


def _objective(params, k, dy, kw):
    return oracle.objective(params["x"], params["w_router"], params["w_gate"], params["w_up"],
                            params["w_down"], k, dy, **kw)


@pytest.mark.parametrize("case", CASES)
def test_finite_differences(case):
    """Every gradient equals the central difference of the forward objective
    along random directions (the selection stays fixed at +-eps)."""
    params, k, dy, kw = _setup(case)
    g = oracle.backward(params["x"], params["w_router"], params["w_gate"], params["w_up"],
                        params["w_down"], k, dy, **kw)
    _, idx0 = _objective(params, k, dy, kw)
    rng = np.random.default_rng(99)
    eps = 1e-5
    targets = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
               "w_down": "dw_down"}
    for name, gname in targets.items():
        for _ in range(2):
            V = rng.standard_normal(params[name].shape)
            Jp, ip = _objective(dict(params, **{name: params[name] + eps * V}), k, dy, kw)
            Jm, im = _objective(dict(params, **{name: params[name] - eps * V}), k, dy, kw)
            assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), "selection moved"
            num = (Jp - Jm) / (2 * eps)
            ana = float(np.sum(g[gname] * V))
            assert abs(num - ana) <= 1e-6 * (1.0 + abs(ana)), (name, num, ana)
    if kw["logit_bias"] is not None:
        V = rng.standard_normal(kw["logit_bias"].shape)
        Jp, _ = _objective(params, k, dy, dict(kw, logit_bias=kw["logit_bias"] + eps * V))
        Jm, _ = _objective(params, k, dy, dict(kw, logit_bias=kw["logit_bias"] - eps * V))
        ana = float(np.sum(g["dlogit_bias"] * V))
        assert abs((Jp - Jm) / (2 * eps) - ana) <= 1e-6 * (1.0 + abs(ana))
    for s, (sg, su, sd) in enumerate(kw["shared"]):
        for j, W in enumerate((sg, su, sd)):
            V = rng.standard_normal(W.shape)
            def with_w(delta):
                sh = [list(t) for t in kw["shared"]]
                sh[s][j] = W + delta
                return dict(kw, shared=[tuple(t) for t in sh])
            Jp, _ = _objective(params, k, dy, with_w(eps * V))
            Jm, _ = _objective(params, k, dy, with_w(-eps * V))
            ana = float(np.sum(g["dshared"][s][j] * V))
            assert abs((Jp - Jm) / (2 * eps) - ana) <= 1e-6 * (1.0 + abs(ana))


def _torch_objective(params, k, dy, kw, idx, pair_row, count):
    """The layer written directly in PyTorch from its definition, with the
    routing decisions (idx, kept pairs, counts) as fixed integers."""
    F = torch.nn.functional
    x, wr, wg, wu, wd = (params[n] for n in ("x", "w_router", "w_gate", "w_up", "w_down"))
    T, E = x.shape[0], wr.shape[0]
    logits = x @ wr.T
    if kw["lbias"] is not None:
        logits = logits + kw["lbias"]
    idx_t = torch.as_tensor(np.asarray(idx, dtype=np.int64))
    g = torch.softmax(torch.gather(logits, 1, idx_t), dim=1)
    kept = torch.as_tensor(np.asarray(pair_row).reshape(T, k) >= 0)
    y = torch.zeros_like(x)
    for t in range(T):
        for j in range(k):
            if kept[t, j]:
                e = int(idx_t[t, j])
                out = F.linear(F.silu(F.linear(x[t], wg[e])) * F.linear(x[t], wu[e]), wd[e])
                y[t] = y[t] + g[t, j] * out
    for (sg, su, sd) in kw["shared"]:
        y = y + F.linear(F.silu(F.linear(x, sg)) * F.linear(x, su), sd)
    J = torch.sum(torch.as_tensor(dy) * y)
    p = torch.softmax(logits, dim=1)
    f = torch.as_tensor(np.asarray(count, dtype=np.float64)) / (T * k)
    J = J + kw["c_bal"] * 0.01 * E * torch.sum(f * p.mean(0))
    J = J + kw["c_z"] * torch.mean(torch.logsumexp(logits, dim=1) ** 2)
    return J


@pytest.mark.parametrize("case", CASES)
def test_autograd(case):
    """The oracle's gradients equal PyTorch autograd of the layer written from
    its definition (float64) on the same routing decisions."""
    params, k, dy, kw = _setup(case)
    g = oracle.backward(params["x"], params["w_router"], params["w_gate"], params["w_up"],
                        params["w_down"], k, dy, **kw)
    fw = g["fwd"]
    tp = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True) for n, v in params.items()}
    lb = None if kw["logit_bias"] is None else torch.tensor(kw["logit_bias"], requires_grad=True)
    sh = [tuple(torch.tensor(w, requires_grad=True) for w in s) for s in kw["shared"]]
    J = _torch_objective(tp, k, dy, dict(lbias=lb, shared=sh, c_bal=kw["c_bal"], c_z=kw["c_z"]),
                         fw["topk_idx"], fw["pair_row"], fw["count"])
    J.backward()
    names = {"x": "dx", "w_router": "dw_router", "w_gate": "dw_gate", "w_up": "dw_up",
             "w_down": "dw_down"}
    for n, gn in names.items():
        np.testing.assert_allclose(g[gn], tp[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)
    if lb is not None:
        np.testing.assert_allclose(g["dlogit_bias"], lb.grad.numpy(), rtol=1e-10, atol=1e-12)
    for s, ts in enumerate(sh):
        for j in range(3):
            np.testing.assert_allclose(g["dshared"][s][j], ts[j].grad.numpy(), rtol=1e-10, atol=1e-12)


def test_silu_grad_closed_forms():
    """SiLU'(0) = 1/2; SiLU'(z) -> 1 for large z and -> 0 for very negative z;
    at z = ln 3 (sigmoid 3/4) it is 3/4 (1 + ln3 / 4)."""
    z = np.array([0.0, 40.0, -800.0, math.log(3.0)])
    got = oracle.silu_grad(z)
    assert got[0] == 0.5
    assert abs(got[1] - 1.0) < 1e-15
    assert got[2] == 0.0
    assert abs(got[3] - 0.75 * (1 + math.log(3.0) / 4)) < 1e-15


def test_silu_grad_autograd():
    z = torch.linspace(-30, 30, 241, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.silu(z).sum().backward()
    np.testing.assert_allclose(oracle.silu_grad(z.detach().numpy()), z.grad.numpy(), rtol=1e-13,
                               atol=1e-300)


def test_gate_grad_rows_sum_to_zero():
    """Renormalised gates sum to one, so their logit gradients sum to zero per
    token; experts outside the selected set get exactly zero."""
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((11, 6))
    idx = oracle.top_k(logits, 3)
    dl = oracle.gate_logit_grad(logits, idx, rng.standard_normal((11, 3)))
    assert np.max(np.abs(dl.sum(axis=1))) < 1e-14
    mask = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~mask] == 0.0)


def test_single_expert_has_no_gate_gradient():
    """With k = 1 the one gate is identically 1: no gradient reaches the
    logits through it, whatever dgate is."""
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((5, 4))
    idx = oracle.top_k(logits, 1)
    dl = oracle.gate_logit_grad(logits, idx, rng.standard_normal((5, 1)))
    assert np.all(dl == 0.0)


def test_balance_grad_worked():
    """T = 1, E = 2, logits (0, 0), one pair on expert 0 (k = 1): p = (1/2,
    1/2), f = (1, 0), so dloss/dl = alpha * 2 * (1/2) * (f - 1/2) =
    (alpha/2, -alpha/2)."""
    got = oracle.balance_logit_grad(np.zeros((1, 2)), np.array([1, 0]), k=1, alpha=0.01)
    np.testing.assert_allclose(got, [[0.005, -0.005]], rtol=1e-15)


def test_balance_grad_uniform_load_is_zero():
    """With f uniform (every expert gets T k / E pairs) the loss is alpha for
    any logits, so its gradient vanishes."""
    rng = np.random.default_rng(7)
    got = oracle.balance_logit_grad(rng.standard_normal((6, 4)), np.array([3, 3, 3, 3]), k=2)
    assert np.max(np.abs(got)) < 1e-18


def test_z_loss_grad_worked():
    """T = 1, logits (0, 0): lse = ln 2, p = (1/2, 1/2), so the gradient is
    2 ln2 * (1/2, 1/2) = (ln 2, ln 2)."""
    got = oracle.z_loss_logit_grad(np.zeros((1, 2)))
    np.testing.assert_allclose(got, [[math.log(2.0), math.log(2.0)]], rtol=1e-15)


def test_dropped_pair_gets_no_expert_gradient():
    """Capacity 0 drops every pair: only the router (through the dropped gates,
    which stay in the softmax) and the shared experts see gradient; the routed
    experts' weights get none."""
    rng = np.random.default_rng(8)
    x, wr, wg, wu, wd, shared = _layer(rng, 5, 4, 3, 2, n_shared=1)
    dy = rng.standard_normal((5, 4))
    g = oracle.backward(x, wr, wg, wu, wd, 2, dy, shared=shared, cap=0)
    assert np.all(g["dw_gate"] == 0) and np.all(g["dw_up"] == 0) and np.all(g["dw_down"] == 0)
    assert np.all(g["dgate"] == 0) and np.all(g["dlogits"] == 0)
    assert np.any(g["dshared"][0][0] != 0)
