"""Oracle of the per-step load-balancing updates (test infrastructure only;
see the package docstring).

Sources, cited by page title and section:
  [Max]   "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
          section "Auxiliary-Loss-Free Load Balancing": a per-expert bias b_j
          is updated after each training step from the deviation of the
          expert's load from the target; overloaded experts get a negative
          bias, underloaded ones a positive bias.
  [MoDE]  "Zen MoDE: Mixture of Distilled Experts Architecture", section
          "Adaptive Capacity Factors": C_e(t) = C_base + gamma (fbar_e - 1/N_E)
          with fbar_e a rolling load statistic; capacity_e = C_e * tokens / N_E.

Readings (the pages leave these open; each becomes an argument or a stated
choice):
  * load_e = count_e, the pre-drop routed pairs of expert e (moe_permute's
    counts); target = T k / E.  The bias moves by a fixed step in the
    direction of the sign of target - load_e (zero at the target): b_e +=
    step * sign(T k - E count_e), decided in exact integer arithmetic, added
    as one float32 addition.
  * fbar is an exponential moving average with decay beta: f_e =
    float32(count_e / (T k)) (one rounding from the exact quotient), then
    fbar = float32(beta * fbar) + float32((1 - beta) * f), each product and
    the sum rounded to float32 (beta = 0 keeps this step's f only).
  * C_e is evaluated in float64 in the formula's order, and capacity_e =
    ceil(C_e * (T k) / E) in float64 (T k pairs, as moe_capacity reads
    "tokens"), clamped to [0, T] (an expert receives at most one pair per
    token).  Unlike moe_capacity, which reads a user-written factor exactly as
    a decimal, C_e is a computed binary value and is used as such.
"""

from __future__ import annotations

import math

import numpy as np


def selection_bias_update(select_bias, count, T, k, step):
    """[Max] "Auxiliary-Loss-Free Load Balancing": b_e + step * sign(T k -
    E count_e) in float32 (see the module readings)."""
    b = np.asarray(select_bias, dtype=np.float32)
    c = np.asarray(count, dtype=np.int64)
    E = c.size
    dev = np.int64(T) * np.int64(k) - np.int64(E) * c
    sgn = np.sign(dev).astype(np.float32)
    return (b + np.float32(step) * sgn).astype(np.float32)


def load_ema(f_bar, count, T, k, decay):
    """Rolling load statistic fbar (float32, see the module readings)."""
    c = np.asarray(count, dtype=np.int64)
    f = np.array([float(v) / float(T * k) for v in c], dtype=np.float64).astype(np.float32)
    beta = np.float32(decay)
    one_minus = np.float32(1.0) - beta
    a = (beta * np.asarray(f_bar, dtype=np.float32)).astype(np.float32)
    b = (one_minus * f).astype(np.float32)
    return (a + b).astype(np.float32)


def adaptive_capacity(f_bar, cf_base, gamma, T, k):
    """[MoDE] "Adaptive Capacity Factors": per-expert budgets (int64 [E])."""
    fb = np.asarray(f_bar, dtype=np.float32).astype(np.float64)
    E = fb.size
    out = np.empty(E, dtype=np.int64)
    inv_e = 1.0 / E
    pairs = float(T * k)
    for e in range(E):
        c_e = float(cf_base) + float(gamma) * (float(fb[e]) - inv_e)
        q = (c_e * pairs) / E
        cap = math.ceil(q) if q > 0 else 0
        out[e] = min(max(cap, 0), T)
    return out


def balance_update(select_bias, f_bar, count, T, k, step, decay, cf_base, gamma):
    """One per-step update: new selection bias, new fbar, and the capacities
    the next step uses (computed from the new fbar)."""
    b = selection_bias_update(select_bias, count, T, k, step) if select_bias is not None else None
    fb = load_ema(f_bar, count, T, k, decay)
    return b, fb, adaptive_capacity(fb, cf_base, gamma, T, k)
