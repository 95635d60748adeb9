"""The balancing-update pins catch plausible mistakes planted in the oracle
(on the CPU, in this process only)."""

import math

import numpy as np
import pytest

import oracle
from oracle import moe_balance as mb
from oracle import moe_oracle as mo
from tests import test_oracle_balance_pins as pins

PIN_TESTS = []
for _n in dir(pins):
    _t = getattr(pins, _n)
    if not _n.startswith("test_"):
        continue
    marks = [m for m in getattr(_t, "pytestmark", []) if m.name == "parametrize"]
    if marks:
        for _v in marks[0].args[1]:
            PIN_TESTS.append(lambda _t=_t, _v=_v: _t(_v))
    else:
        PIN_TESTS.append(_t)


def _bias_sign_flipped(b, count, T, k, step):
    return mb.__dict__["_orig_bias"](b, count, T, k, -step)


def _bias_float64(b, count, T, k, step):
    c = np.asarray(count, dtype=np.int64)
    s = np.sign(np.int64(T) * k - c.size * c)
    return (np.asarray(b, np.float64) + step * s).astype(np.float32)


def _ema_swapped(fb, count, T, k, decay):
    return mb.__dict__["_orig_ema"](fb, count, T, k, 1.0 - decay)


def _cap_tokens_not_pairs(fb, cf, gamma, T, k):
    return mb.__dict__["_orig_cap"](fb, cf, gamma, T, 1)


def _cap_floor(fb, cf, gamma, T, k):
    fbv = np.asarray(fb, np.float32).astype(np.float64)
    E = fbv.size
    return np.array([min(max(math.floor((cf + gamma * (f - 1.0 / E)) * T * k / E), 0), T)
                     for f in fbv], dtype=np.int64)


def _dispatch_first_cap_only(idx, E, cap=None):
    if cap is not None and np.ndim(cap) == 1:
        cap = int(cap[0])
    return mo.__dict__["_orig_dispatch"](idx, E, cap)


MUTATIONS = {
    "bias_sign_flipped": (mb, "selection_bias_update", _bias_sign_flipped),
    "bias_added_in_float64": (mb, "selection_bias_update", _bias_float64),
    "ema_weights_swapped": (mb, "load_ema", _ema_swapped),
    "capacity_over_tokens": (mb, "adaptive_capacity", _cap_tokens_not_pairs),
    "capacity_floor": (mb, "adaptive_capacity", _cap_floor),
    "dispatch_one_budget": (mo, "dispatch", _dispatch_first_cap_only),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_balance_pins_catch_mutation(name, monkeypatch):
    mod, fn_name, bad = MUTATIONS[name]
    monkeypatch.setitem(mb.__dict__, "_orig_bias", mb.selection_bias_update)
    monkeypatch.setitem(mb.__dict__, "_orig_ema", mb.load_ema)
    monkeypatch.setitem(mb.__dict__, "_orig_cap", mb.adaptive_capacity)
    monkeypatch.setitem(mo.__dict__, "_orig_dispatch", mo.dispatch)
    monkeypatch.setattr(mod, fn_name, bad)
    monkeypatch.setattr(oracle, fn_name, bad)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"
