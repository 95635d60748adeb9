"""Pins of the selection-key variant that adds the bias to the routing
probability ("Zen-Max: Maximum Capability via Mixture-of-Experts
Architecture", section "Auxiliary-Loss-Free Load Balancing": s_ij =
softmax(x_i W_g)_j + b_j)."""

import math

import numpy as np
import scipy.special

import oracle


def test_prob_keys_worked():
    """Logits (0, ln 3): probabilities (1/4, 3/4); bias (0.6, 0): keys (0.85,
    0.75), so top-1 is expert 0 -- where bias on the logits (0.6 vs ln 3)
    would pick expert 1."""
    logits = np.array([[0.0, math.log(3.0)]])
    bias = np.array([0.6, 0.0], dtype=np.float32)
    keys = oracle.selection_keys_on_probs(logits, bias)
    assert keys.dtype == np.float32
    np.testing.assert_allclose(keys, [[0.85, 0.75]], rtol=1e-7)
    assert oracle.top_k(keys, 1)[0, 0] == 0
    assert oracle.top_k(oracle.selection_keys(logits, bias), 1)[0, 0] == 1


def test_prob_keys_without_bias_are_softmax():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((50, 13)) * 3
    keys = oracle.selection_keys_on_probs(logits)
    want = scipy.special.softmax(logits, axis=1).astype(np.float32)
    assert np.array_equal(keys, want)
    np.testing.assert_allclose(keys.sum(axis=1), 1.0, rtol=1e-6)


def test_prob_keys_bias_shift():
    """A constant bias moves every key of a token equally."""
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((20, 6))
    base = oracle.selection_keys_on_probs(logits)
    shifted = oracle.selection_keys_on_probs(logits, np.full(6, 0.5, np.float32))
    assert np.array_equal(shifted, (base + np.float32(0.5)).astype(np.float32))


def test_given_selection_equals_own_selection():
    """Passing the oracle's own selection as ``topk_idx`` changes nothing, and
    a selection on probability keys flows through the forward and backward."""
    rng = np.random.default_rng(8)
    T, d, E, h, k = 6, 5, 4, 3, 2
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    wg = rng.standard_normal((E, h, d))
    wu = rng.standard_normal((E, h, d))
    wd = rng.standard_normal((E, d, h))
    dy = rng.standard_normal((T, d))
    sb = 0.4 * rng.standard_normal(E)
    a = oracle.backward(x, wr, wg, wu, wd, k, dy, select_bias=sb, c_bal=1.0, c_z=0.1)
    b = oracle.backward(x, wr, wg, wu, wd, k, dy, select_bias=sb, c_bal=1.0, c_z=0.1,
                        topk_idx=a["fwd"]["topk_idx"])
    for key in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dlogits"):
        assert np.array_equal(a[key], b[key])
    pk = oracle.top_k(oracle.selection_keys_on_probs(x @ wr.T, sb.astype(np.float32)), k)
    c = oracle.backward(x, wr, wg, wu, wd, k, dy, c_bal=1.0, topk_idx=pk)
    assert np.array_equal(c["fwd"]["topk_idx"], pk)
    assert np.allclose(c["fwd"]["topk_gate"].sum(axis=1), 1.0)
