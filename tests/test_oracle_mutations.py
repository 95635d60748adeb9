"""The pins catch plausible mistakes: each mutation below plants one mistake
in the oracle (on the CPU, in this process only) and at least one pin of
``test_oracle_pins`` must fail against it."""

import math

import numpy as np
import pytest

import oracle
from oracle import moe_oracle as mo
from tests import test_oracle_pins as pins

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _gates_from_keys(logits, idx):  # softmax over all experts, not renormalised
    l = np.asarray(logits, dtype=np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)


def _silu_wrong_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _swiglu_transposed_down(xs, wg, wu, wd):
    xs = np.asarray(xs, dtype=np.float64)
    a = mo.silu(xs @ np.asarray(wg, np.float64).T) * (xs @ np.asarray(wu, np.float64).T)
    wd = np.asarray(wd, np.float64)
    # the stored [d, h] matrix used without its transpose (reshaped when d != h)
    return a @ wd.reshape(a.shape[1], -1)


def _swiglu_gate_up_swapped(xs, wg, wu, wd):
    return mo.__dict__["_orig_swiglu"](xs, wu, wg, wd)


def _topk_high_index_ties(keys, k):
    keys = np.asarray(keys)
    E = keys.shape[1]
    order = np.argsort(-keys[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _capacity_floor(cf, T, k, E):
    if cf is None or cf <= 0:
        return None
    return int(math.floor(cf * T * k / E))


def _capacity_no_k(cf, T, k, E):
    if cf is None or cf <= 0:
        return None
    return int(math.ceil(cf * T / E))


def _dispatch_slot_order(idx, E, cap=None):
    # drops by slot rank first (all slot-0 pairs before slot-1 pairs), not token order
    idx = np.asarray(idx)
    T, k = idx.shape
    order = np.argsort(np.repeat(np.arange(k)[None, :], T, 0).reshape(-1), kind="stable")
    perm_idx = idx.reshape(-1)[order]
    d = mo.__dict__["_orig_dispatch"](perm_idx.reshape(-1, 1), E, cap)
    pr = np.full(T * k, -1, dtype=np.int64)
    pr[order] = d["pair_row"]
    rp = np.where(d["row_pair"] >= 0, order[np.maximum(d["row_pair"], 0)], -1)
    return dict(d, pair_row=pr, row_pair=rp)


def _balance_f_over_T(logits, count, k, alpha=0.01):
    f, P, _ = mo.__dict__["_orig_balance"](logits, count, k, alpha)
    f = f * k
    return f, P, alpha * len(P) * float(np.sum(f * P))


def _balance_gate_prob(logits, count, k, alpha=0.01):
    # P from the renormalised top-k gates instead of the full softmax
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    idx = mo.top_k(l, k)
    g = mo.gates(l, idx)
    P = np.zeros(E)
    for t in range(T):
        P[idx[t]] += g[t]
    P /= T
    f = np.asarray(count, np.float64) / (T * k)
    return f, P, alpha * E * float(np.sum(f * P))


def _moe_output_no_shared(x, idx, gate, pair_row, wg, wu, wd, shared=(), tokens=None):
    return mo.__dict__["_orig_output"](x, idx, gate, pair_row, wg, wu, wd, (), tokens)


def _moe_output_renorm_after_drop(x, idx, gate, pair_row, wg, wu, wd, shared=(), tokens=None):
    g = np.array(gate, dtype=np.float64)
    T, k = g.shape
    kept = np.asarray(pair_row).reshape(T, k) >= 0
    s = (g * kept).sum(axis=1, keepdims=True)
    g = np.where(s > 0, g / np.where(s > 0, s, 1), g)
    return mo.__dict__["_orig_output"](x, idx, g, pair_row, wg, wu, wd, shared, tokens)


def _keys_bias_in_f64(logits, select_bias=None):
    if select_bias is None:
        return np.asarray(logits).copy()
    return np.asarray(logits, np.float64) + np.asarray(select_bias, np.float64)[None, :]


def _gates_biased(logits, idx):
    # gates taken from the keys (the caller passes keys for logits) is modelled by
    # adding a constant ramp, i.e. the gate sees a per-expert offset
    l = np.asarray(logits, np.float64) + np.arange(np.asarray(logits).shape[1])[None, :] * 0.5
    return mo.__dict__["_orig_gates"](l, idx)


MUTATIONS = {
    "gates_not_renormalised": ("gates", _gates_from_keys),
    "gates_see_offset": ("gates", _gates_biased),
    "silu_wrong_sign": ("silu", _silu_wrong_sign),
    "down_projection_transposed": ("swiglu", _swiglu_transposed_down),
    "gate_up_swapped": ("swiglu", _swiglu_gate_up_swapped),
    "ties_to_higher_index": ("top_k", _topk_high_index_ties),
    "capacity_floor": ("capacity", _capacity_floor),
    "capacity_without_k": ("capacity", _capacity_no_k),
    "drop_in_slot_order": ("dispatch", _dispatch_slot_order),
    "f_divided_by_T": ("balance_stats", _balance_f_over_T),
    "P_from_topk_gates": ("balance_stats", _balance_gate_prob),
    "shared_expert_dropped": ("moe_output", _moe_output_no_shared),
    "renormalise_after_drop": ("moe_output", _moe_output_renorm_after_drop),
    "selection_key_in_f64": ("selection_keys", _keys_bias_in_f64),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    fn_name, bad = MUTATIONS[name]
    monkeypatch.setitem(mo.__dict__, "_orig_swiglu", mo.swiglu)
    monkeypatch.setitem(mo.__dict__, "_orig_dispatch", mo.dispatch)
    monkeypatch.setitem(mo.__dict__, "_orig_balance", mo.balance_stats)
    monkeypatch.setitem(mo.__dict__, "_orig_output", mo.moe_output)
    monkeypatch.setitem(mo.__dict__, "_orig_gates", mo.gates)
    monkeypatch.setattr(mo, fn_name, bad)
    monkeypatch.setattr(oracle, fn_name, bad)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"
