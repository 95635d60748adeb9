"""GPU parity of the backward pass against the CPU oracle (needs an MI355X).

The objective is <dy, y> + c_bal * loss + c_z * zloss ("Every parameter,
every token", sections "The gating network" and "A balance penalty"; Zen-Max,
section "MoE-Specific Training Stability").  The oracle runs on the GPU's own
float32 logits, so both sides route identically.

Tolerances:
  * routing-side kernels on identical inputs (the GPU's dgate and dlogits fed
    to the oracle's formulas): 1e-5 max-abs relative (fp32 arithmetic);
  * everything downstream of the bf16 expert GEMMs (dgate, dlogits, dx and
    the expert weight gradients, per expert): 2e-2 max-abs relative, the bf16
    output bar; u, v, [du | dv] and the gated hidden activation are rounded
    to bf16 between the GEMMs (relative 2^-9 each);
  * the kept pre-activations uv: 1e-2; the gated row gradients dout: 4e-3
    (one bf16 rounding);
  * fp32 layers (fp32 intermediates, fp32 accumulation): 1e-4 for every
    gradient, 1e-5 for uv, 1e-6 for dout;
  * experts without rows: exactly zero weight gradients.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from dataclasses import replace

from moe_inputs import WORKLOADS, Bf16, as_f32, generate, generate_dy, small_case
from tests.gpu_helpers import build_layer, check_layer, host, normwise, shared_list, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "mixtral_small": (small_case("mixtral_bf16", T=1600, d=256, h=320, cid_offset=300), 1.0, 0.1),
    "finegrained_small": (small_case("finegrained_shared_bf16", T=512, d=128, h=128, h_shared=64),
                          1.0, 0.1),
    "capacity_small": (small_case("capacity_balance_bf16", T=2048, d=192, h=256), 1.0, 0.0),
    "decode_small": (small_case("decode_bf16", T=64, d=256, h=128, h_shared=512), 0.0, 0.1),
    "tiny_f32": (WORKLOADS["tiny_f32"], 1.0, 0.1),
    "finegrained_f32": (replace(small_case("finegrained_shared_bf16", T=300, d=96, h=80,
                                           h_shared=48), dtype="f32"), 1.0, 0.1),
}


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_mixture_experts_moe_amd import _lib  # noqa: F401  (fails loudly if not built)


def _split_shared(g, inp):
    """Concatenated shared-expert gradients -> per shared expert (gate, up, down)."""
    ns, hs = inp["shared_gate"].shape[0], inp["shared_gate"].shape[1]
    out = []
    for s in range(ns):
        sl = slice(s * hs, (s + 1) * hs)
        out.append((g[0][0, sl], g[1][0, sl], g[2][0][:, sl]))
    return out


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer_backward(name):
    cfg, c_bal, c_z = CASES[name]
    _say(f"[case] {name} {cfg} c_bal={c_bal} c_z={c_z}")
    inp = generate(cfg)
    dy_h = generate_dy(cfg)
    layer = build_layer(inp)
    x = to_device(inp["x"])
    dy = to_device(dy_h)
    res = layer.forward(x, train=True)
    layer.backward(dy, c_bal, c_z)
    torch.cuda.synchronize()
    check_layer(inp, res)  # the training forward's output

    T, E, k = cfg.T, cfg.E, cfg.k
    xf, wr = as_f32(inp["x"]), as_f32(inp["w_router"])
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    dyf = as_f32(dy_h)
    gl = host(res["logits"])
    cap = oracle.capacity(cfg.cf, T, k, E)
    ref = oracle.backward(xf, wr, wg, wu, wd, k, dyf, shared=shared_list(inp),
                          logit_bias=inp["logit_bias"], select_bias=inp["select_bias"], cap=cap,
                          alpha=cfg.alpha, c_bal=c_bal, c_z=c_z, logits=gl)
    fw = ref["fwd"]
    errs = {}

    # kept pre-activations of the routed rows
    R = int(fw["offset"][-1])
    rp = fw["row_pair"][:R]
    u_ref = np.concatenate([xf[rp[r] // k][None] @ wg[e].T for e in range(E)
                            for r in range(fw["offset"][e], fw["offset"][e + 1])], axis=0) if R else None
    if R:
        v_ref = np.concatenate([xf[rp[r] // k][None] @ wu[e].T for e in range(E)
                                for r in range(fw["offset"][e], fw["offset"][e + 1])], axis=0)
        uv = host(res["uv"])[:R]
        errs["uv"] = max(normwise(uv[:, 0::2], u_ref), normwise(uv[:, 1::2], v_ref))
        assert errs["uv"] <= (1e-5 if cfg.dtype == "f32" else 1e-2), errs

    # gated upstream gradient of every kept row: dout[pair_row[p]] = g_p dy_t
    if R:
        g_gpu = host(res["topk_gate"]).reshape(-1)
        want = g_gpu[rp][:, None] * dyf[rp // k]
        errs["dout"] = normwise(host(res["dout"])[:R], want)
        assert errs["dout"] <= (1e-6 if cfg.dtype == "f32" else 4e-3), errs

    # routing side on identical inputs (fp32 kernels)
    gdg = host(res["dgate"])
    gdl = host(res["dlogits"])
    dl_same = oracle.gate_logit_grad(gl, fw["topk_idx"], gdg)
    if c_bal:
        dl_same = dl_same + c_bal * oracle.balance_logit_grad(gl, fw["count"], k, cfg.alpha)
    if c_z:
        dl_same = dl_same + c_z * oracle.z_loss_logit_grad(gl)
    errs["dlogits_same_in"] = normwise(gdl, dl_same)
    assert errs["dlogits_same_in"] <= 1e-5, errs
    _, dwr_same, dlb_same = oracle.router_linear_backward(xf, wr, gdl)
    errs["dw_router_same_in"] = normwise(host(res["dw_router"]), dwr_same)
    assert errs["dw_router_same_in"] <= 1e-5, errs
    if inp["logit_bias"] is not None:
        errs["dlogit_bias_same_in"] = normwise(host(res["dlogit_bias"]), dlb_same)
        assert errs["dlogit_bias_same_in"] <= 1e-5, errs
    dropped = fw["pair_row"].reshape(T, k) < 0
    assert np.all(gdg[dropped] == 0.0)

    # end to end against the float64 oracle
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    for key in ("dgate", "dlogits", "dx", "dw_router"):
        errs[key] = normwise(host(res[key]), ref[key])
        assert errs[key] <= tol, errs
    kept = fw["kept"]
    for key in ("dw_gate", "dw_up", "dw_down"):
        got = host(res[key])
        worst = 0.0
        for e in range(E):
            if kept[e] == 0:
                assert np.all(got[e] == 0.0), (key, e)
                continue
            worst = max(worst, normwise(got[e], ref[key][e]))
        errs[key] = worst
        assert worst <= tol, errs
    if inp["shared_gate"] is not None:
        got = _split_shared((host(res["shared_dw_gate"]), host(res["shared_dw_up"]),
                             host(res["shared_dw_down"])), inp)
        worst = max(normwise(got[s][j], ref["dshared"][s][j])
                    for s in range(len(got)) for j in range(3))
        errs["shared"] = worst
        assert worst <= tol, errs
    _say(f"[ok] {name}: " + ", ".join(f"{a}={b:.2e}" for a, b in errs.items()))


def test_backward_deterministic():
    cfg, c_bal, c_z = CASES["finegrained_small"]
    inp = generate(cfg)
    layer = build_layer(inp)
    x = to_device(inp["x"])
    dy = to_device(generate_dy(cfg))
    outs = []
    for _ in range(2):
        layer.forward(x, train=True)
        b = layer.backward(dy, c_bal, c_z)
        torch.cuda.synchronize()
        outs.append({k: b[k].clone() for k in ("dx", "dw_gate", "dw_up", "dw_down", "dw_router",
                                                "dlogits", "shared_dw_gate")})
    for key in outs[0]:
        assert torch.equal(outs[0][key], outs[1][key]), key


@pytest.mark.parametrize("sizes,d,h,gather,dt", [
    ([60], 128, 64, False, "bf16"),
    ([17, 0, 29, 300], 192, 128, True, "bf16"),
    ([3] * 47 + [0] + [3] * 48, 128, 192, True, "bf16"),
    ([0, 0], 64, 64, False, "bf16"),
    ([257, 1, 64, 128], 256, 320, True, "bf16"),
    ([70, 130], 384, 64, False, "bf16"),
    ([17, 0, 29, 100], 72, 40, True, "f32"),
    ([1, 130], 64, 96, False, "f32"),
])
def test_expert_backward_groups(sizes, d, h, gather, dt):
    """moe_expert_swiglu_backward alone on ragged groups (empty ones included),
    with and without a row gather, against the oracle's expert backward."""
    from sparse_mixture_experts_moe_amd import _lib
    from moe_inputs import bf16_bits_rne
    _say(f"[case] groups {sizes[:6]}{'...' if len(sizes) > 6 else ''} d={d} h={h} gather={gather} {dt}")
    rng = np.random.default_rng(len(sizes) * 1000 + d + h)
    G = len(sizes)
    R = int(sum(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)

    def bf(a):
        if dt == "f32":
            return a.astype(np.float32)
        return Bf16(bf16_bits_rne(a.astype(np.float32)))

    ntok = max(R // 2 + 1, 1)
    div = 2
    src = bf(rng.standard_normal((ntok if gather else max(R, 1), d)))
    rows = rng.integers(0, ntok * div, size=max(R, 1)).astype(np.int32)  # token = rows / div
    wg = bf(rng.standard_normal((G, h, d)) / np.sqrt(d))
    wu = bf(rng.standard_normal((G, h, d)) / np.sqrt(d))
    wd = bf(rng.standard_normal((G, d, h)) / np.sqrt(h))
    dout = bf(rng.standard_normal((max(R, 1), d)))
    A, WG, WU, WD, DOUT = (to_device(t) for t in (src, wg, wu, wd, dout))
    goff = torch.from_numpy(off).cuda()
    a_rows = torch.from_numpy(rows).cuda() if gather else None
    hid, uv = _lib.moe_expert_gate_up_train(A, goff, R, WG, WU, a_rows=a_rows, a_rows_div=div)
    da, dwg, dwu, dwd = _lib.moe_expert_swiglu_backward(A, goff, R, DOUT, uv, hid, WG, WU, WD,
                                                        a_rows=a_rows, a_rows_div=div)
    torch.cuda.synchronize()
    srcf, doutf = as_f32(src), as_f32(dout)
    af = srcf[rows[:R] // div] if gather else srcf[:R]
    wgf, wuf, wdf = as_f32(wg), as_f32(wu), as_f32(wd)
    da_h, dwg_h, dwu_h, dwd_h = host(da), host(dwg), host(dwu), host(dwd)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r0 == r1:
            assert np.all(dwg_h[g] == 0) and np.all(dwu_h[g] == 0) and np.all(dwd_h[g] == 0)
            continue
        ref = oracle.swiglu_backward(af[r0:r1], wgf[g], wuf[g], wdf[g], doutf[r0:r1])
        for name, got, want in (("da", da_h[r0:r1], ref[0]), ("dw_gate", dwg_h[g], ref[1]),
                                ("dw_up", dwu_h[g], ref[2]), ("dw_down", dwd_h[g], ref[3])):
            err = normwise(got, want)
            assert err <= (1e-4 if dt == "f32" else 2e-2), (g, name, err)


@pytest.mark.parametrize("name,variant", [("mixtral_bf16", None), ("finegrained_shared_bf16", None),
                                          ("capacity_balance_bf16", None),
                                          ("mixtral_bf16", "relu"), ("mixtral_bf16", "bypass")])
def test_backward_full_size(name, variant):
    """The training step at a workload's full size, in the bench's launch
    configuration (two streams; for a routing variant, the one of
    ``bench.py --backward --variant``), against the oracle's whole backward
    on the GPU's own logits: every token's gate and input gradients, every
    logit and router-weight gradient, and every entry of every expert's (and
    the shared experts') weight gradients, so that every tile of every
    backward GEMM is compared."""
    from bench import BYPASS_COUNTS, RELU_K_MUL
    from moe_inputs import WORKLOADS, generate_bypass, relu_logit_offset
    from sparse_mixture_experts_moe_amd.workload import (bypass_layer_from_inputs,
                                                         relu_layer_from_inputs, relu_logit_bias)
    cfg = WORKLOADS[name]
    c_bal, c_z = 1.0, 1e-3
    _say(f"[case] full-size backward {name} {variant}: generating inputs")
    inp = generate(cfg)
    dy_h = generate_dy(cfg)
    nz = nc = nk = 0
    if variant == "relu":
        k_run = min(cfg.E, RELU_K_MUL * cfg.k)
        lb = relu_logit_bias(inp, relu_logit_offset(cfg, cfg.k))
        layer = relu_layer_from_inputs(inp, k_run, relu_logit_offset(cfg, cfg.k))
    elif variant == "bypass":
        k_run = cfg.k
        nz, nc, nk = BYPASS_COUNTS
        rows, const = generate_bypass(cfg, nz, nc, nk)
        layer = bypass_layer_from_inputs(inp, rows, const, nz, nc)
    else:
        k_run = cfg.k
        layer = build_layer(inp)
    x = to_device(inp["x"])
    dy = to_device(dy_h)
    _say(f"[case] full-size backward {name} {variant}: running")
    res = layer.forward(x, train=True)
    layer.backward(dy, c_bal, c_z)
    torch.cuda.synchronize()
    _say(f"[case] full-size backward {name} {variant}: oracle")
    T, E, k = cfg.T, cfg.E, k_run
    xf, wr = as_f32(inp["x"]), as_f32(inp["w_router"])
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    dyf = as_f32(dy_h)
    gl = host(res["logits"])
    cap = oracle.capacity(cfg.cf, T, cfg.k, E)
    if variant == "relu":
        ref = oracle.backward_relu(xf, wr, wg, wu, wd, k, dyf,
                                   shared=shared_list(inp), logit_bias=lb, cap=cap,
                                   alpha=cfg.alpha, c_bal=c_bal, c_z=c_z, logits=gl)
        glg = oracle.relu_gate_logit_grad
    elif variant == "bypass":
        wr = np.concatenate([wr, as_f32(rows)], 0)
        ref = oracle.backward_bypass(xf, wr, wg, wu, wd, k, nz, nc,
                                     as_f32(const), dyf, shared=shared_list(inp), cap=cap,
                                     alpha=cfg.alpha, c_bal=c_bal, c_z=c_z, logits=gl)
        glg = oracle.gate_logit_grad
    else:
        ref = oracle.backward(xf, wr, wg, wu, wd, k, dyf,
                              shared=shared_list(inp), logit_bias=inp["logit_bias"],
                              select_bias=inp["select_bias"], cap=cap, alpha=cfg.alpha,
                              c_bal=c_bal, c_z=c_z, logits=gl)
        glg = oracle.gate_logit_grad
    fw = ref["fwd"]
    _say(f"[case] full-size backward {name} {variant}: checking")
    # the selection and dispatch the gradients were taken for are the oracle's
    assert np.array_equal(host(res["topk_idx"]), fw["topk_idx"])
    assert np.array_equal(host(res["pair_row"]), fw["pair_row"])
    errs = {}
    # routing side on identical inputs (fp32 kernels)
    gdg = host(res["dgate"])
    gdl = host(res["dlogits"])
    dl_same = glg(gl, fw["topk_idx"], gdg)
    dl_same = dl_same + c_bal * oracle.balance_logit_grad(gl, fw["count"], k, cfg.alpha)
    dl_same = dl_same + c_z * oracle.z_loss_logit_grad(gl)
    errs["dlogits_same_in"] = normwise(gdl, dl_same)
    _, dwr_same, _ = oracle.router_linear_backward(xf, wr, gdl)
    errs["dw_router_same_in"] = normwise(host(res["dw_router"]), dwr_same)
    assert errs["dlogits_same_in"] <= 1e-5 and errs["dw_router_same_in"] <= 1e-5, errs
    # end to end against the float64 oracle, every entry
    tol = 2e-2
    for key in ("dgate", "dlogits", "dx", "dw_router"):
        errs[key] = normwise(host(res[key]), ref[key])
    if nk:
        errs["dconst"] = normwise(host(res["dconst"])[:nk], ref["dconst"])
    kept = fw["kept"]
    for key in ("dw_gate", "dw_up", "dw_down"):
        worst = 0.0
        for e in range(cfg.E):
            got = host(res[key][e])
            if kept[e] == 0:
                assert np.all(got == 0.0), (key, e)
                continue
            worst = max(worst, normwise(got, ref[key][e]))
        errs[key] = worst
    if inp["shared_gate"] is not None:
        got = _split_shared((host(res["shared_dw_gate"]), host(res["shared_dw_up"]),
                             host(res["shared_dw_down"])), inp)
        errs["shared"] = max(normwise(got[s][j], ref["dshared"][s][j])
                             for s in range(len(got)) for j in range(3))
    _say(f"[ok] full-size backward {name} {variant}: " +
         ", ".join(f"{a}={b:.2e}" for a, b in errs.items()))
    for key, v in errs.items():
        if not key.endswith("_same_in"):
            assert v <= tol, (key, errs)


@pytest.mark.parametrize("T,E,k,d,dt,c_bal,c_z", [
    (1, 1, 1, 64, "bf16", 1.0, 1.0),
    (333, 256, 32, 96, "f32", 1.0, 0.01),
    (1000, 200, 7, 160, "bf16", 0.5, 0.0),
    (4099, 8, 2, 256, "bf16", 0.0, 0.001),
])
def test_routing_backward_shapes(T, E, k, d, dt, c_bal, c_z):
    """moe_combine_backward, moe_route_backward and moe_router_backward alone,
    from the smallest to the largest expert count and k, with dropped pairs,
    against the oracle on the same inputs (fp32 arithmetic: 1e-5)."""
    from sparse_mixture_experts_moe_amd import _lib
    from moe_inputs import bf16_bits_rne
    _say(f"[case] routing backward T={T} E={E} k={k} d={d} {dt}")
    rng = np.random.default_rng(T + E + k)

    def cast(a):
        return a.astype(np.float32) if dt == "f32" else Bf16(bf16_bits_rne(a.astype(np.float32)))

    x = cast(rng.standard_normal((T, d)))
    wr = cast(rng.standard_normal((E, d)) / np.sqrt(d))
    dy = cast(rng.standard_normal((T, d)))
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx = oracle.top_k(logits, k)
    gate = oracle.gates(logits, idx).astype(np.float32)
    cap = max(1, (T * k) // (2 * E))
    disp = oracle.dispatch(idx, E, cap)
    R = int(disp["offset"][-1])
    y_rows = cast(rng.standard_normal((max(R, 1), d)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    pair_row = dev(disp["pair_row"].astype(np.int32))
    dgate, dout = _lib.moe_combine_backward(to_device(dy), to_device(y_rows), pair_row, k,
                                            dev(gate), want_dout=True)
    count = dev(disp["count"].astype(np.int32))
    dl = _lib.moe_route_backward(dev(logits), dev(idx.astype(np.int32)), dev(gate), dgate, count,
                                 0.01, c_bal, c_z)
    dw, db, dx = _lib.moe_router_backward(to_device(x), to_device(wr), dl)
    torch.cuda.synchronize()
    xf, wrf, dyf, yf = as_f32(x), as_f32(wr), as_f32(dy), as_f32(y_rows)
    pr = disp["pair_row"].reshape(T, k)
    dg_ref = np.where(pr >= 0, np.einsum("td,tkd->tk", dyf.astype(np.float64),
                                         yf[np.maximum(pr, 0)].astype(np.float64)), 0.0)
    assert normwise(host(dgate), dg_ref) <= 1e-5
    kept_pairs = np.nonzero(disp["pair_row"] >= 0)[0]
    want = gate.reshape(-1)[kept_pairs][:, None].astype(np.float64) * dyf[kept_pairs // k]
    got = host(dout)[disp["pair_row"][kept_pairs]]
    assert normwise(got, want) <= (1e-6 if dt == "f32" else 4e-3)
    gdg = host(dgate)
    dl_ref = oracle.gate_logit_grad(logits, idx, gdg)
    if c_bal:
        dl_ref = dl_ref + c_bal * oracle.balance_logit_grad(logits, disp["count"], k, 0.01)
    if c_z:
        dl_ref = dl_ref + c_z * oracle.z_loss_logit_grad(logits)
    gdl = host(dl)
    assert normwise(gdl, dl_ref) <= 1e-5
    dx_ref, dw_ref, db_ref = oracle.router_linear_backward(xf, wrf, gdl)
    assert normwise(host(dx), dx_ref) <= 1e-5
    assert normwise(host(dw), dw_ref) <= 1e-5
    assert normwise(host(db), db_ref) <= 1e-5


def test_layer_backward_bias_on_probs():
    """A training step whose selection adds the bias to the routing
    probability: the GPU's selection is checked for validity on the
    probability keys, then every gradient against the oracle's backward of
    that selection (the key moves only the chosen set)."""
    cfg = small_case("capacity_balance_bf16", T=2048, d=192, h=256)
    _say(f"[case] backward with bias on probabilities {cfg}")
    inp = generate(cfg)
    dy_h = generate_dy(cfg)
    base = build_layer(inp)
    cap = oracle.capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    layer = type(base)(base.w_router, base.w_gate, base.w_up, base.w_down, cfg.k,
                       select_bias=base.select_bias, capacity=cap, alpha=cfg.alpha,
                       bias_on_probs=True)
    res = layer.forward(to_device(inp["x"]), train=True)
    layer.backward(to_device(dy_h), 1.0, 0.1)
    torch.cuda.synchronize()
    gl = host(res["logits"])
    idx = host(res["topk_idx"]).astype(np.int64)
    keys = oracle.selection_keys_on_probs(gl, inp["select_bias"]).astype(np.float64)
    chosen = np.take_along_axis(keys, idx, axis=1)
    mask = np.ones_like(keys, dtype=bool)
    np.put_along_axis(mask, idx, False, axis=1)
    worst_other = np.where(mask, keys, -np.inf).max(axis=1)
    tol = 4e-7 * np.abs(keys).max()
    assert np.all(chosen.min(axis=1) >= worst_other - tol)
    assert np.all(np.diff(chosen, axis=1) <= tol)
    xf, wr = as_f32(inp["x"]), as_f32(inp["w_router"])
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    ref = oracle.backward(xf, wr, wg, wu, wd, cfg.k, as_f32(dy_h), cap=cap, alpha=cfg.alpha,
                          c_bal=1.0, c_z=0.1, logits=gl, topk_idx=idx)
    fw = ref["fwd"]
    assert np.array_equal(host(res["pair_row"]), fw["pair_row"])
    errs = {}
    for key in ("dgate", "dlogits", "dx", "dw_router"):
        errs[key] = normwise(host(res[key]), ref[key])
        assert errs[key] <= 2e-2, errs
    for key in ("dw_gate", "dw_up", "dw_down"):
        got = host(res[key])
        worst = max(normwise(got[e], ref[key][e]) for e in range(cfg.E) if fw["kept"][e])
        errs[key] = worst
        assert worst <= 2e-2, errs
    _say("[ok] bias on probabilities: " + ", ".join(f"{a}={b:.2e}" for a, b in errs.items()))
