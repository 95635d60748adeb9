"""Pins of the load-balancing update oracle ([Max] "Auxiliary-Loss-Free Load
Balancing"; [MoDE] "Adaptive Capacity Factors"): worked examples, exact
rational brute force on inputs that are exact in binary, and the per-expert
dispatch against a plain loop."""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_bias_worked():
    """T = 2, k = 2, E = 2: target 2 pairs; expert 0 holds 3 (overloaded: its
    bias falls by the step), expert 1 holds 1 (rises)."""
    got = oracle.selection_bias_update([0.5, -0.25], [3, 1], T=2, k=2, step=0.125)
    assert got.dtype == np.float32
    assert got.tolist() == [0.375, -0.125]


def test_bias_at_target_unchanged():
    b = np.array([0.1, -0.7, 3.0], dtype=np.float32)
    got = oracle.selection_bias_update(b, [4, 4, 4], T=6, k=2, step=0.5)
    assert np.array_equal(got, b)


def test_bias_is_a_float32_addition():
    """The step is taken as a float32 and added in float32: with step =
    2^-24 + 2^-50 (float32: 2^-24), 1 + 2^-24 is a tie that rounds to 1,
    while the sum in float64 rounded afterwards would give 1 + 2^-23.  (The
    overloaded expert: 1 - 2^-24 is exact either way.)"""
    step = 2.0 ** -24 + 2.0 ** -50
    got = oracle.selection_bias_update([1.0, 1.0], [0, 2], T=1, k=2, step=step)
    assert got.tolist() == [1.0, 1.0 - 2.0 ** -24]


@pytest.mark.parametrize("seed", range(5))
def test_bias_direction_brute(seed):
    rng = np.random.default_rng(seed)
    E, T, k = 7, 50, 3
    count = rng.multinomial(T * k, np.ones(E) / E)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.selection_bias_update(b, count, T, k, 0.25)
    for e in range(E):
        load, target = Fraction(int(count[e])), Fraction(T * k, E)
        want = b[e] + (np.float32(0.25) if load < target else
                       (np.float32(-0.25) if load > target else np.float32(0.0)))
        assert got[e] == np.float32(want)


def test_ema_worked():
    """fbar 0.5, f = 1/4 (one pair of T k = 4), beta 1/2: 0.25 + 0.125."""
    got = oracle.load_ema([0.5, 0.5], [1, 3], T=2, k=2, decay=0.5)
    assert got.tolist() == [0.375, 0.625]


def test_ema_extremes():
    fb = np.array([0.3, 0.7], dtype=np.float32)
    assert np.array_equal(oracle.load_ema(fb, [1, 2], T=3, k=1, decay=1.0), fb)
    f_now = oracle.load_ema(fb, [1, 2], T=3, k=1, decay=0.0)
    assert f_now.tolist() == [np.float32(1 / 3), np.float32(2 / 3)]


def test_capacity_gamma_zero_matches_capacity():
    """With gamma = 0 and a factor exact in binary, the adaptive budget is
    moe_capacity's budget for every expert."""
    for cf, T, k, E in [(1.25, 16384, 2, 64), (1.0, 1000, 8, 128), (2.5, 37, 3, 5)]:
        got = oracle.adaptive_capacity(np.full(E, 0.123, np.float32), cf, 0.0, T, k)
        want = min(oracle.capacity(cf, T, k, E), T)
        assert (got == want).all(), (cf, T, k, E)


def test_capacity_worked():
    """E = 2, T k = 8, cf_base 1, gamma 2, fbar (3/4, 1/4): C = (3/2, 1/2),
    budgets ceil(C * 8 / 2) = (6, 2)."""
    got = oracle.adaptive_capacity([0.75, 0.25], 1.0, 2.0, T=4, k=2)
    assert got.tolist() == [4, 2]  # 6 clamps to T = 4
    got = oracle.adaptive_capacity([0.75, 0.25], 1.0, 2.0, T=8, k=1)
    assert got.tolist() == [6, 2]


@pytest.mark.parametrize("seed", range(5))
def test_capacity_exact_rationals(seed):
    """Dyadic fbar, factor and gamma: the float64 evaluation is exact, so the
    budget is the ceiling of the exact rational, clamped to [0, T]."""
    rng = np.random.default_rng(seed)
    E, T, k = 8, 1024, 2
    fb = (rng.integers(0, 256, E) / 256).astype(np.float32)
    cf, gamma = 1.25, float(rng.integers(-8, 9)) / 2
    got = oracle.adaptive_capacity(fb, cf, gamma, T, k)
    for e in range(E):
        c = Fraction(cf) + Fraction(gamma) * (Fraction(float(fb[e])) - Fraction(1, E))
        q = c * T * k / E
        want = min(max(math.ceil(q), 0), T)
        assert got[e] == want


def test_capacity_monotone_in_load():
    fb = np.linspace(0.0, 0.5, 9).astype(np.float32)
    caps = oracle.adaptive_capacity(fb, 1.0, 3.0, T=4096, k=2)
    assert all(a <= b for a, b in zip(caps[:-1], caps[1:]))


@pytest.mark.parametrize("seed", range(4))
def test_dispatch_per_expert_caps(seed):
    """Per-expert budgets keep each expert's first cap_e pairs in token order;
    equal budgets give the scalar budget's dispatch."""
    rng = np.random.default_rng(seed)
    T, E, k = 40, 6, 2
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    caps = rng.integers(0, 12, E)
    d = oracle.dispatch(idx, E, caps)
    flat = idx.reshape(-1)
    seen = [0] * E
    for p, e in enumerate(flat):
        kept = seen[e] < caps[e]
        seen[e] += 1
        assert (d["pair_row"][p] >= 0) == kept
    assert d["kept"].tolist() == [min(int(c), int(n)) for c, n in zip(caps, d["count"])]
    s = oracle.dispatch(idx, E, 5)
    u = oracle.dispatch(idx, E, np.full(E, 5))
    for key in ("pair_row", "row_pair", "offset"):
        assert np.array_equal(s[key], u[key])
