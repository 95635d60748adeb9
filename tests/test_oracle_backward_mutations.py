"""The backward pins catch plausible mistakes: each mutation plants one mistake
in the backward oracle (on the CPU, in this process only) and at least one pin
of ``test_oracle_backward_pins`` must fail against it."""

import numpy as np
import pytest

import oracle
from oracle import moe_backward as mb
from oracle import moe_oracle as mo
from tests import test_oracle_backward_pins as pins

PIN_TESTS = []
for _n in dir(pins):
    _t = getattr(pins, _n)
    if not _n.startswith("test_"):
        continue
    marks = getattr(_t, "pytestmark", [])
    params = [m for m in marks if m.name == "parametrize"]
    if params:
        for _v in params[0].args[1]:
            PIN_TESTS.append(lambda _t=_t, _v=_v: _t(_v))
    else:
        PIN_TESTS.append(_t)


def _silu_grad_no_second_term(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _gate_logit_grad_uncentred(logits, idx, dgate):
    g = mo.gates(logits, idx)
    dl = np.zeros(np.asarray(logits).shape)
    np.put_along_axis(dl, np.asarray(idx, dtype=np.int64), g * np.asarray(dgate), axis=1)
    return dl


def _balance_sign(logits, count, k, alpha=0.01):
    return -mb.__dict__["_orig_balance_grad"](logits, count, k, alpha)


def _z_half(logits):
    return 0.5 * mb.__dict__["_orig_z_grad"](logits)


def _swiglu_backward_dv_from_u(xs, wg, wu, wd, dout):
    xs, wg, wu, wd, dout = (np.asarray(a, np.float64) for a in (xs, wg, wu, wd, dout))
    u, v = xs @ wg.T, xs @ wu.T
    hid = mo.silu(u) * v
    d_hid = dout @ wd
    du = d_hid * v * mb.silu_grad(u)
    dv = d_hid * u  # the gate's pre-activation instead of SiLU of it
    return du @ wg + dv @ wu, du.T @ xs, dv.T @ xs, dout.T @ hid


def _swiglu_backward_dxs_transposed(xs, wg, wu, wd, dout):
    dxs, a, b, c = mb.__dict__["_orig_swiglu_backward"](xs, wg, wu, wd, dout)
    # gate and up weights swapped in the input gradient
    xs, wg, wu, wd, dout = (np.asarray(t, np.float64) for t in (xs, wg, wu, wd, dout))
    u, v = xs @ wg.T, xs @ wu.T
    d_hid = dout @ wd
    du = d_hid * v * mb.silu_grad(u)
    dv = d_hid * mo.silu(u)
    return du @ wu + dv @ wg, a, b, c


def _router_no_bias_grad(x, w_router, dlogits):
    dx, dw, db = mb.__dict__["_orig_router_linear"](x, w_router, dlogits)
    return dx, dw, np.zeros_like(db)


def _gate_grad_ignores_drop(dy, x, idx, pair_row, wg, wu, wd):
    return mb.__dict__["_orig_gate_grad"](dy, x, idx, np.zeros_like(np.asarray(pair_row)), wg, wu, wd)


MUTATIONS = {
    "silu_grad_missing_term": ("silu_grad", _silu_grad_no_second_term),
    "gate_grad_uncentred": ("gate_logit_grad", _gate_logit_grad_uncentred),
    "balance_grad_sign": ("balance_logit_grad", _balance_sign),
    "z_grad_missing_two": ("z_loss_logit_grad", _z_half),
    "dv_from_preactivation": ("swiglu_backward", _swiglu_backward_dv_from_u),
    "dx_gate_up_swapped": ("swiglu_backward", _swiglu_backward_dxs_transposed),
    "logit_bias_grad_dropped": ("router_linear_backward", _router_no_bias_grad),
    "dropped_pairs_get_gate_grad": ("gate_grad", _gate_grad_ignores_drop),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_pins_catch_mutation(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setitem(mb.__dict__, "_orig_balance_grad", mb.balance_logit_grad)
    monkeypatch.setitem(mb.__dict__, "_orig_z_grad", mb.z_loss_logit_grad)
    monkeypatch.setitem(mb.__dict__, "_orig_swiglu_backward", mb.swiglu_backward)
    monkeypatch.setitem(mb.__dict__, "_orig_router_linear", mb.router_linear_backward)
    monkeypatch.setitem(mb.__dict__, "_orig_gate_grad", mb.gate_grad)
    monkeypatch.setattr(mb, fn_name, bad)
    monkeypatch.setattr(oracle, fn_name, bad)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"
