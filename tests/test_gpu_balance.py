"""GPU parity of the per-step load-balancing updates and of the per-expert
budgets against the CPU oracle (needs an MI355X).  Everything here is integer
or an exactly specified float sequence: the comparisons are bit-exact.

Sources: "Zen-Max: Maximum Capability via Mixture-of-Experts Architecture",
section "Auxiliary-Loss-Free Load Balancing"; "Zen MoDE: Mixture of Distilled
Experts Architecture", section "Adaptive Capacity Factors"; "Every parameter,
every token", section "A budget".
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import generate, small_case
from tests.gpu_helpers import build_layer, host, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_moe_amd._lib as lib
    return lib


def _bits(a):
    return np.asarray(a, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("E,T,k,decay,cf,gamma,step,seed", [
    (1, 10, 1, 0.0, 1.0, 0.0, 0.01, 0),
    (8, 4096, 2, 0.9, 1.25, 2.0, 1e-3, 1),
    (64, 16384, 2, 0.5, 1.0, 8.0, 0.1, 2),
    (128, 8192, 8, 1.0, 1.5, -3.0, 2.0 ** -24 + 2.0 ** -50, 3),
    (200, 1 << 20, 8, 0.99, 1.1, 40.0, 0.0, 4),
    (256, 64, 8, 0.25, 0.5, 1e6, 1.0, 5),
])
def test_balance_update_bit_exact(L, E, T, k, decay, cf, gamma, step, seed):
    _say(f"[case] balance update E={E} T={T} k={k} decay={decay} gamma={gamma}")
    rng = np.random.default_rng(seed)
    count = rng.multinomial(T * k, rng.dirichlet(np.ones(E) * 0.7)).astype(np.int32)
    if E > 2:
        count[0] = T * k // E  # one expert exactly at the mean load when it divides
    b0 = rng.standard_normal(E).astype(np.float32)
    fb0 = rng.uniform(0, 2.0 / E, E).astype(np.float32)
    dc = torch.from_numpy(count).cuda()
    db = torch.from_numpy(b0.copy()).cuda()
    dfb = torch.from_numpy(fb0.copy()).cuda()
    caps = L.moe_balance_update(dc, T, k, dfb, select_bias=db, bias_step=step, ema_decay=decay,
                                cf_base=cf, gamma=gamma)
    torch.cuda.synchronize()
    rb, rfb, rcap = oracle.balance_update(b0, fb0, count, T, k, step, decay, cf, gamma)
    assert np.array_equal(_bits(host(db)), _bits(rb))
    assert np.array_equal(_bits(host(dfb)), _bits(rfb))
    assert np.array_equal(host(caps).astype(np.int64), rcap)


@pytest.mark.parametrize("T,E,k,seed", [(1000, 8, 2, 0), (4099, 64, 8, 1), (333, 256, 3, 2),
                                        (1, 4, 4, 3)])
def test_permute_budgets(L, T, E, k, seed):
    _say(f"[case] permute budgets T={T} E={E} k={k}")
    rng = np.random.default_rng(seed)
    w = rng.dirichlet(np.ones(E) * 0.5)
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w) for _ in range(T)]).astype(np.int32)
    caps = rng.integers(0, 2 * T * k // E + 2, E).astype(np.int32)
    caps[0] = 0
    d = 64
    x = rng.standard_normal((T, d)).astype(np.float32)
    dx = torch.from_numpy(x).cuda()
    res = L.moe_permute_budgets(torch.from_numpy(idx).cuda(), E, torch.from_numpy(caps).cuda(),
                                dx)
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E, caps)
    count, offset, pair_row, row_pair, x_perm = (host(t) for t in res)
    assert np.array_equal(count, ref["count"])
    assert np.array_equal(offset, ref["offset"])
    assert np.array_equal(pair_row, ref["pair_row"])
    assert np.array_equal(row_pair, ref["row_pair"])
    R = int(ref["offset"][-1])
    assert np.array_equal(x_perm[:R], x[ref["row_pair"][:R] // k])


def test_layer_balance_steps(L):
    """Five training-style steps of a layer with the selection-bias update and
    adaptive per-expert budgets: after every step the GPU's routing, bias,
    rolling load and budgets equal the oracle's, which replays the same steps
    on the GPU's logits."""
    cfg = small_case("capacity_balance_bf16", T=1024, d=128, h=128)
    inp = generate(cfg)
    bal = dict(bias_step=0.05, ema_decay=0.8, cf_base=1.0, gamma=4.0)
    layer = build_layer(inp)
    layer = type(layer)(layer.w_router, layer.w_gate, layer.w_up, layer.w_down, cfg.k,
                        select_bias=layer.select_bias, alpha=cfg.alpha, balance=bal)
    x = to_device(inp["x"])
    T, E, k = cfg.T, cfg.E, cfg.k
    b = np.asarray(inp["select_bias"], dtype=np.float32).copy()
    fb = np.full(E, 1.0 / E, dtype=np.float32)
    caps = np.full(E, min(oracle.capacity(bal["cf_base"], T, k, E), T), dtype=np.int64)
    for step in range(5):
        res = layer.forward(x)
        torch.cuda.synchronize()
        gl = host(res["logits"])
        idx = oracle.top_k(oracle.selection_keys(gl, b), k)
        disp = oracle.dispatch(idx, E, caps)
        assert np.array_equal(host(res["topk_idx"]), idx), step
        assert np.array_equal(host(res["pair_row"]), disp["pair_row"]), step
        assert np.array_equal(host(res["expert_count"]), disp["count"]), step
        layer.update_balance()
        torch.cuda.synchronize()
        b, fb, caps = oracle.balance_update(b, fb, disp["count"], T, k, bal["bias_step"],
                                            bal["ema_decay"], bal["cf_base"], bal["gamma"])
        assert np.array_equal(_bits(host(layer.select_bias)), _bits(b)), step
        got_fb = host(layer.load_ema)
        bad = np.nonzero(_bits(got_fb) != _bits(fb))[0]
        assert bad.size == 0, (step, bad[:4].tolist(), got_fb[bad[:4]].tolist(),
                               fb[bad[:4]].tolist(), disp["count"][bad[:4]].tolist())
        assert np.array_equal(host(layer.expert_capacity).astype(np.int64), caps), step
        _say(f"[ok] step {step}: dropped {T * k - int(disp['offset'][-1])}, "
             f"max load {int(disp['count'].max())}, caps {caps.min()}..{caps.max()}")
