"""GPU parity of the routing variants against the CPU oracle (needs an
MI355X): ReLU routing ("Zen MoDE: Mixture of Diverse Experts",
section "Router": ReLU gating, an adaptive expert count per
token) and zero-computation experts (same section: zero, copy and constant
experts).  Selection, gates and dispatch are compared bit-exactly on the
GPU's own float32 logits; outputs at 1e-4 (fp32) and 2e-2 (bf16) normwise."""

import sys

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import (Bf16, as_f32, bf16_bits_rne, generate, generate_bypass,
                        relu_logit_offset, small_case)
from tests.gpu_helpers import host, normwise, shared_list, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_moe_amd._lib as lib
    return lib


# ------------------------------------------------------------ ReLU routing
@pytest.mark.parametrize("E,k", [(1, 1), (8, 2), (8, 8), (64, 6), (200, 32), (256, 16)])
def test_route_relu_logits_in(L, E, k):
    """Selection and gates bit-exact on adversarial logits: ties, signed
    zeros, rows with no positive logit and rows with more than k."""
    _say(f"[case] relu route logits_in E={E} k={k}")
    rng = np.random.default_rng(E * 7 + k)
    T = 517
    lg = np.round(rng.standard_normal((T, E)) * 2).astype(np.float32) * 0.5
    lg[0] = 0.0
    lg[1] = -1.0
    lg[2, ::2] = -0.0
    lg[3] = 1.0
    lg[4] = np.linspace(1, -1, E)
    _, idx, gate = L.moe_route(None, None, k, logits=torch.from_numpy(lg).cuda(), logits_in=True,
                               relu=True)
    torch.cuda.synchronize()
    ridx, rg = oracle.relu_route(lg, k)
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(gate), rg.astype(np.float32))


def test_route_relu_rejects_selection_bias(L):
    lg = torch.zeros((4, 8), device="cuda")
    with pytest.raises(L.MoEError):
        L.moe_route(None, None, 2, None, torch.zeros(8, device="cuda"), logits=lg,
                    logits_in=True, relu=True)


@pytest.mark.parametrize("T,E,k,cap", [(1000, 8, 2, -1), (4099, 64, 8, 100), (333, 256, 3, 2),
                                       (5, 4, 4, 0)])
def test_permute_skips_empty_slots(L, T, E, k, cap):
    """Slots holding -1 or an id past E are not routed: no count, no budget,
    pair_row -1; everything else as the plain dispatch."""
    _say(f"[case] permute with empty slots T={T} E={E} k={k} cap={cap}")
    rng = np.random.default_rng(T + E)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    holes = rng.random((T, k)) < 0.3
    idx[holes] = -1
    idx[rng.random((T, k)) < 0.02] = E + 3
    d = 64
    x = rng.standard_normal((T, d)).astype(np.float32)
    res = L.moe_permute(torch.from_numpy(idx).cuda(), E, cap, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E, None if cap < 0 else cap)
    count, offset, pair_row, row_pair, x_perm = (host(t) for t in res)
    assert np.array_equal(count, ref["count"])
    assert np.array_equal(offset, ref["offset"])
    assert np.array_equal(pair_row, ref["pair_row"])
    assert np.array_equal(row_pair, ref["row_pair"])
    R = int(ref["offset"][-1])
    assert np.array_equal(x_perm[:R], x[ref["row_pair"][:R] // k])


def _check_relu(inp, res, k_max, lb, tokens=None):
    cfg = inp["cfg"]
    x, wr = as_f32(inp["x"]), as_f32(inp["w_router"])
    gl = host(res["logits"])
    lt = np.arange(cfg.T) if tokens is None else tokens
    assert normwise(gl[lt], oracle.router_logits(x[lt], wr, lb)) <= 1e-5
    idx, g = oracle.relu_route(gl, k_max)
    assert np.array_equal(host(res["topk_idx"]), idx)
    assert np.array_equal(host(res["topk_gate"]), g.astype(np.float32))
    cap = oracle.capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    disp = oracle.dispatch(idx, cfg.E, cap)
    for key in ("count", "offset", "pair_row", "row_pair"):
        want = disp[key]
        got = host(res["expert_" + key] if key in ("count", "offset") else res[key])
        assert np.array_equal(got, want), key
    y = oracle.moe_output(x, idx, g, disp["pair_row"], inp["w_gate"], inp["w_up"], inp["w_down"],
                          shared_list(inp), tokens)
    out = host(res["out"])
    out = out if tokens is None else out[tokens]
    err = normwise(out, y)
    assert err <= (1e-4 if cfg.dtype == "f32" else 2e-2), err
    f, P, loss = oracle.balance_stats(gl, disp["count"], k_max, cfg.alpha)
    assert np.array_equal(host(res["f"]), f.astype(np.float32))
    used = (idx >= 0).sum(axis=1)
    return err, float(used.mean()), int(used.min()), int(used.max())


@pytest.mark.parametrize("name,T,d,h,kmul", [("tiny_f32", 64, 128, 256, 2),
                                             ("mixtral_bf16", 512, 256, 384, 2),
                                             ("finegrained_shared_bf16", 700, 256, 128, 2),
                                             ("capacity_balance_bf16", 1024, 128, 128, 3)])
@pytest.mark.parametrize("gather", ["fused", "copy"])
def test_layer_relu(L, name, T, d, h, kmul, gather):
    from sparse_mixture_experts_moe_amd.workload import relu_layer_from_inputs, relu_logit_bias
    cfg = small_case(name, T=T, d=d, h=h)
    _say(f"[case] relu layer {name} T={T} d={d} h={h} gather={gather}")
    inp = generate(cfg)
    off = relu_logit_offset(cfg, cfg.k)
    k_max = min(cfg.E, kmul * cfg.k)
    layer = relu_layer_from_inputs(inp, k_max, off, gather)
    res = layer(to_device(inp["x"]))
    torch.cuda.synchronize()
    err, mean_used, lo, hi = _check_relu(inp, res, k_max, relu_logit_bias(inp, off))
    _say(f"[ok] {name}: out err {err:.3g}, experts per token {mean_used:.2f} ({lo}..{hi})")


# ---------------------------------------------------- zero-computation experts
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,k,nz,nc,nk,E_ffn", [(300, 128, 2, 1, 1, 2, 8), (65, 72, 4, 0, 2, 0, 5),
                                                  (1500, 256, 8, 3, 0, 5, 60), (7, 8, 1, 0, 0, 3, 0),
                                                  (33, 70, 3, 1, 1, 1, 4), (1100, 70, 2, 0, 1, 1, 3)])
def test_combine_bypass(L, dt, T, d, k, nz, nc, nk, E_ffn):
    """moe_combine_bypass alone against the definition, with dropped FFN
    pairs, every kind of zero-computation expert and ids past the last."""
    _say(f"[case] combine bypass {dt} T={T} d={d} k={k} kinds={nz},{nc},{nk} E_ffn={E_ffn}")
    rng = np.random.default_rng(T + d + k)
    E = E_ffn + nz + nc + nk
    idx = rng.integers(0, E + 1, (T, k)).astype(np.int32)  # E itself: past the last
    gate = rng.random((T, k)).astype(np.float32)
    caps = np.array([max(1, T * k // (2 * max(E_ffn, 1)))] * E_ffn + [0] * (E - E_ffn) + [0])
    disp = oracle.dispatch(idx, E + 1, caps)
    R = max(int(disp["offset"][-1]), 1)

    def cast(a):
        return a.astype(np.float32) if dt == "f32" else Bf16(bf16_bits_rne(a.astype(np.float32)))

    y = cast(rng.standard_normal((R, d)))
    x = cast(rng.standard_normal((T, d)))
    cv = cast(rng.standard_normal((nk, d)))
    sh = cast(rng.standard_normal((T, d)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = L.moe_combine_bypass(to_device(y), dev(disp["pair_row"].astype(np.int32)), dev(idx),
                               dev(gate), E_ffn, nz, nc, to_device(x) if nc else None,
                               to_device(cv) if nk else None, to_device(sh), out_dtype=torch.float32)
    torch.cuda.synchronize()
    yf, xf, cf, shf = as_f32(y), as_f32(x), as_f32(cv), as_f32(sh)
    pr = disp["pair_row"].reshape(T, k)
    want = shf.astype(np.float64).copy()
    ffn = (idx < E_ffn) & (pr >= 0)
    for j in range(k):
        rows = np.nonzero(ffn[:, j])[0]
        want[rows] += gate[rows, j, None] * yf[pr[rows, j]]
    idx_b = np.where(idx < E, idx, -1)
    idx_b[idx < E_ffn] = -1
    for t in range(T):  # the zero-computation part by the oracle, token by token
        sel = idx_b[t] >= 0
        if sel.any():
            want[t] += oracle.bypass_output(xf[t:t + 1], idx_b[t:t + 1, sel], gate[t:t + 1, sel],
                                            E_ffn, nz, nc, cf.reshape(nk, d))[0]
    assert normwise(host(out), want) <= 1e-6


def _bypass_inputs(name, T, d, h, counts):
    cfg = small_case(name, T=T, d=d, h=h)
    inp = generate(cfg)
    rows, const = generate_bypass(cfg, *counts)
    return cfg, inp, rows, const


def _check_bypass(cfg, inp, res, rows, const, nz, nc, tokens=None):
    x = as_f32(inp["x"])
    wr = np.concatenate([as_f32(inp["w_router"]), as_f32(rows)], 0)
    gl = host(res["logits"])
    lt = np.arange(cfg.T) if tokens is None else tokens
    assert normwise(gl[lt], oracle.router_logits(x[lt], wr)) <= 1e-5
    cap = oracle.capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    ref = oracle.forward_bypass(x, wr, inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k, nz, nc,
                                as_f32(const), shared=shared_list(inp), cap=cap, alpha=cfg.alpha,
                                logits=gl, tokens=tokens)
    assert np.array_equal(host(res["topk_idx"]), ref["topk_idx"])
    assert float(np.max(np.abs(host(res["topk_gate"]) - ref["topk_gate"]))) <= 1e-6
    assert np.array_equal(host(res["expert_count"]), ref["count"])
    assert np.array_equal(host(res["expert_offset"]), ref["offset"])
    assert np.array_equal(host(res["pair_row"]), ref["pair_row"])
    out = host(res["out"])
    out = out if tokens is None else out[tokens]
    err = normwise(out, ref["y"])
    assert err <= (1e-4 if cfg.dtype == "f32" else 2e-2), err
    assert np.array_equal(host(res["f"]), ref["f"].astype(np.float32))
    assert abs(float(host(res["loss"])[0]) - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    E = cfg.E
    return err, int(ref["offset"][E]), int(ref["count"][E:].sum())


@pytest.mark.parametrize("name,T,d,h,counts", [
    ("tiny_f32", 64, 128, 256, (1, 1, 2)),
    ("mixtral_bf16", 512, 256, 384, (1, 1, 2)),
    ("finegrained_shared_bf16", 700, 256, 128, (4, 2, 2)),
    ("capacity_balance_bf16", 1024, 128, 128, (0, 3, 1)),
    ("decode_bf16", 64, 256, 128, (2, 0, 0)),
])
@pytest.mark.parametrize("gather", ["fused", "copy"])
def test_layer_bypass(L, name, T, d, h, counts, gather):
    from sparse_mixture_experts_moe_amd.workload import bypass_layer_from_inputs
    cfg, inp, rows, const = _bypass_inputs(name, T, d, h, counts)
    _say(f"[case] bypass layer {name} T={T} d={d} h={h} kinds={counts} gather={gather}")
    layer = bypass_layer_from_inputs(inp, rows, const, counts[0], counts[1], gather)
    res = layer(to_device(inp["x"]))
    torch.cuda.synchronize()
    err, ffn_rows, bypass_pairs = _check_bypass(cfg, inp, res, rows, const, counts[0], counts[1])
    _say(f"[ok] {name}: out err {err:.3g}, FFN rows {ffn_rows}, bypass pairs {bypass_pairs}")


def test_layer_variants_full_size_mixtral(L):
    """Both variants on the full Mixtral-shaped workload in the benchmark's
    configuration (1 zero, 1 copy, 2 constant experts; ReLU with k_max = 2k
    and the offset that makes k experts positive on average), on every
    token."""
    from bench import BYPASS_COUNTS, RELU_K_MUL
    from moe_inputs import WORKLOADS
    from sparse_mixture_experts_moe_amd.workload import (bypass_layer_from_inputs,
                                                         relu_layer_from_inputs, relu_logit_bias)
    cfg = WORKLOADS["mixtral_bf16"]
    inp = generate(cfg)
    tokens = None
    x = to_device(inp["x"])
    rows, const = generate_bypass(cfg, *BYPASS_COUNTS)
    layer = bypass_layer_from_inputs(inp, rows, const, BYPASS_COUNTS[0], BYPASS_COUNTS[1])
    res = layer(x)
    torch.cuda.synchronize()
    err, ffn_rows, bypass_pairs = _check_bypass(cfg, inp, res, rows, const, BYPASS_COUNTS[0],
                                                BYPASS_COUNTS[1], tokens=tokens)
    _say(f"[ok] bypass full size: err {err:.3g}, FFN rows {ffn_rows}, bypass pairs {bypass_pairs}")
    del layer, res
    off = relu_logit_offset(cfg, cfg.k)
    k_max = RELU_K_MUL * cfg.k
    layer = relu_layer_from_inputs(inp, k_max, off)
    res = layer(x)
    torch.cuda.synchronize()
    err, mean_used, lo, hi = _check_relu(inp, res, k_max, relu_logit_bias(inp, off), tokens=tokens)
    _say(f"[ok] relu full size: err {err:.3g}, experts per token {mean_used:.2f} ({lo}..{hi})")


# ------------------------------------------------------ ReLU routing backward
@pytest.mark.parametrize("name,T,d,h,c_bal,c_z", [("tiny_f32", 64, 128, 256, 1.0, 0.1),
                                                  ("mixtral_bf16", 1024, 256, 320, 1.0, 0.1),
                                                  ("finegrained_shared_bf16", 512, 128, 128, 0.0, 0.1),
                                                  ("capacity_balance_bf16", 2048, 192, 256, 1.0, 0.0)])
def test_layer_relu_backward(L, name, T, d, h, c_bal, c_z):
    """A ReLU-routed training step (forward keeping the pre-activations, then
    the backward) against the oracle's backward on the GPU's logits: the
    routing side on identical inputs at 1e-5, everything after the bf16
    GEMMs at 2e-2 (1e-4 in fp32)."""
    from moe_inputs import generate_dy
    from sparse_mixture_experts_moe_amd.workload import relu_layer_from_inputs, relu_logit_bias
    cfg = small_case(name, T=T, d=d, h=h)
    _say(f"[case] relu backward {name} T={T} d={d} h={h} c_bal={c_bal} c_z={c_z}")
    inp = generate(cfg)
    dy_h = generate_dy(cfg)
    off = relu_logit_offset(cfg, cfg.k)
    k_max = min(cfg.E, 2 * cfg.k)
    lb = relu_logit_bias(inp, off)
    layer = relu_layer_from_inputs(inp, k_max, off)
    res = layer.forward(to_device(inp["x"]), train=True)
    layer.backward(to_device(dy_h), c_bal, c_z)
    torch.cuda.synchronize()
    _check_relu(inp, res, k_max, lb)
    xf, wr = as_f32(inp["x"]), as_f32(inp["w_router"])
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    gl = host(res["logits"])
    cap = oracle.capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    ref = oracle.backward_relu(xf, wr, wg, wu, wd, k_max, as_f32(dy_h), shared=shared_list(inp),
                               logit_bias=lb, cap=cap, alpha=cfg.alpha, c_bal=c_bal, c_z=c_z,
                               logits=gl)
    fw = ref["fwd"]
    errs = {}
    gdg, gdl = host(res["dgate"]), host(res["dlogits"])
    assert np.all(gdg[fw["topk_idx"] < 0] == 0.0)
    dl_same = oracle.relu_gate_logit_grad(gl, fw["topk_idx"], gdg)
    if c_bal:
        dl_same = dl_same + c_bal * oracle.balance_logit_grad(gl, fw["count"], k_max, cfg.alpha)
    if c_z:
        dl_same = dl_same + c_z * oracle.z_loss_logit_grad(gl)
    errs["dlogits_same_in"] = normwise(gdl, dl_same)
    assert errs["dlogits_same_in"] <= 1e-5, errs
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    for key in ("dgate", "dlogits", "dx", "dw_router", "dlogit_bias"):
        errs[key] = normwise(host(res[key]), ref[key])
        assert errs[key] <= tol, errs
    for key in ("dw_gate", "dw_up", "dw_down"):
        got = host(res[key])
        worst = 0.0
        for e in range(cfg.E):
            if fw["kept"][e] == 0:
                assert np.all(got[e] == 0.0), (key, e)
                continue
            worst = max(worst, normwise(got[e], ref[key][e]))
        errs[key] = worst
        assert worst <= tol, errs
    _say(f"[ok] relu backward {name}: " + ", ".join(f"{a}={b:.2e}" for a, b in errs.items()))


# --------------------------------------------- zero-computation experts backward
@pytest.mark.parametrize("name,T,d,h,counts,c_bal,c_z", [
    ("tiny_f32", 64, 128, 256, (1, 1, 2), 1.0, 0.1),
    ("mixtral_bf16", 1024, 256, 320, (1, 1, 2), 1.0, 0.1),
    ("finegrained_shared_bf16", 512, 128, 128, (4, 2, 2), 0.0, 0.1),
    ("capacity_balance_bf16", 2048, 192, 256, (0, 3, 1), 1.0, 0.0),
])
def test_layer_bypass_backward(L, name, T, d, h, counts, c_bal, c_z):
    """A training step of the layer with zero-computation experts against the
    oracle's backward on the GPU's logits (the constant rows' gradient
    included): routing side on identical inputs at 1e-5, the rest at 2e-2
    (1e-4 in fp32)."""
    from moe_inputs import generate_dy
    from sparse_mixture_experts_moe_amd.workload import bypass_layer_from_inputs
    cfg, inp, rows, const = _bypass_inputs(name, T, d, h, counts)
    nz, nc, nk = counts
    _say(f"[case] bypass backward {name} T={T} d={d} h={h} kinds={counts}")
    dy_h = generate_dy(cfg)
    layer = bypass_layer_from_inputs(inp, rows, const, nz, nc)
    res = layer.forward(to_device(inp["x"]), train=True)
    layer.backward(to_device(dy_h), c_bal, c_z)
    torch.cuda.synchronize()
    _check_bypass(cfg, inp, res, rows, const, nz, nc)
    xf = as_f32(inp["x"])
    wr = np.concatenate([as_f32(inp["w_router"]), as_f32(rows)], 0)
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    gl = host(res["logits"])
    cap = oracle.capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    ref = oracle.backward_bypass(xf, wr, wg, wu, wd, cfg.k, nz, nc, as_f32(const), as_f32(dy_h),
                                 shared=shared_list(inp), cap=cap, alpha=cfg.alpha, c_bal=c_bal,
                                 c_z=c_z, logits=gl)
    fw = ref["fwd"]
    errs = {}
    gdg, gdl = host(res["dgate"]), host(res["dlogits"])
    dl_same = oracle.gate_logit_grad(gl, fw["topk_idx"], gdg)
    if c_bal:
        dl_same = dl_same + c_bal * oracle.balance_logit_grad(gl, fw["count"], cfg.k, cfg.alpha)
    if c_z:
        dl_same = dl_same + c_z * oracle.z_loss_logit_grad(gl)
    errs["dlogits_same_in"] = normwise(gdl, dl_same)
    assert errs["dlogits_same_in"] <= 1e-5, errs
    tol = 1e-4 if cfg.dtype == "f32" else 2e-2
    for key in ("dgate", "dlogits", "dx", "dw_router"):
        errs[key] = normwise(host(res[key]), ref[key])
        assert errs[key] <= tol, errs
    if nk:
        errs["dconst"] = normwise(host(res["dconst"])[:nk], ref["dconst"])
        assert errs["dconst"] <= tol, errs
    for key in ("dw_gate", "dw_up", "dw_down"):
        got = host(res[key])
        worst = 0.0
        for e in range(cfg.E):
            if fw["kept"][e] == 0:
                assert np.all(got[e] == 0.0), (key, e)
                continue
            worst = max(worst, normwise(got[e], ref[key][e]))
        errs[key] = worst
        assert worst <= tol, errs
    _say(f"[ok] bypass backward {name}: " + ", ".join(f"{a}={b:.2e}" for a, b in errs.items()))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,d,k,nz,nc,nk,E_ffn", [(300, 128, 2, 1, 1, 2, 8), (77, 70, 3, 1, 2, 1, 4),
                                                  (5000, 64, 8, 2, 1, 3, 20), (9, 8, 1, 0, 0, 2, 2)])
def test_bypass_backward_calls(L, dt, T, d, k, nz, nc, nk, E_ffn):
    """moe_combine_backward_bypass and moe_bypass_backward alone against the
    definitions: dgate per slot source, dout on the FFN rows that ran, the
    copy slots' dx added to an accumulator, the constant rows' gradient."""
    _say(f"[case] bypass backward calls {dt} T={T} d={d} k={k} kinds={nz},{nc},{nk} E_ffn={E_ffn}")
    rng = np.random.default_rng(T * 3 + d + k)
    E = E_ffn + nz + nc + nk
    idx = np.stack([rng.choice(E + 1, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = rng.random((T, k)).astype(np.float32)
    caps = np.array([max(1, T * k // (2 * E))] * E_ffn + [0] * (E + 1 - E_ffn))
    disp = oracle.dispatch(idx, E + 1, caps)
    R = max(int(disp["offset"][-1]), 1)

    def cast(a):
        return a.astype(np.float32) if dt == "f32" else Bf16(bf16_bits_rne(a.astype(np.float32)))

    y, x, cv, dy = (cast(rng.standard_normal(s)) for s in ((R, d), (T, d), (nk, d), (T, d)))
    acc0 = rng.standard_normal((T, d)).astype(np.float32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    pr = disp["pair_row"].astype(np.int32)
    dout = torch.zeros((R, d), dtype=torch.float32 if dt == "f32" else torch.bfloat16,
                       device="cuda")
    dgate, _ = L.moe_combine_backward_bypass(to_device(dy), to_device(y), dev(pr), dev(idx),
                                             dev(gate), E_ffn, nz, nc, to_device(x) if nc else None,
                                             to_device(cv) if nk else None, dout=dout)
    dx_acc = dev(acc0)
    _, dconst = L.moe_bypass_backward(to_device(dy), dev(idx), dev(gate), E_ffn, nz, nc, nk,
                                      dx_acc=dx_acc if nc else None)
    torch.cuda.synchronize()
    yf, xf, cf, dyf = (as_f32(a).astype(np.float64) for a in (y, x, cv, dy))
    prk = pr.reshape(T, k)
    want_dg = np.zeros((T, k))
    want_dx = acc0.astype(np.float64).copy()
    want_dc = np.zeros((nk, d))
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if e < E_ffn:
                if prk[t, j] >= 0:
                    want_dg[t, j] = dyf[t] @ yf[prk[t, j]]
                continue
            if e >= E:
                continue
            kind, c = oracle.bypass_kind(e, E_ffn, nz, nc, nk)
            if kind == "copy":
                want_dg[t, j] = dyf[t] @ xf[t]
                want_dx[t] += gate[t, j] * dyf[t]
            elif kind == "const":
                want_dg[t, j] = dyf[t] @ cf[c]
                want_dc[c] += gate[t, j] * dyf[t]
    assert normwise(host(dgate), want_dg) <= 1e-5
    kept = np.nonzero(pr >= 0)[0]
    if kept.size:
        got = host(dout)[pr[kept]]
        want = gate.reshape(-1)[kept][:, None] * dyf[kept // k]
        assert normwise(got, want) <= (1e-6 if dt == "f32" else 4e-3)
    if nc:
        assert normwise(host(dx_acc), want_dx) <= 1e-6
    if nk:
        assert normwise(host(dconst), want_dc) <= 1e-5

