"""The C-ABI library on the host: it loads, exports every declared entry
point, computes the capacity exactly, and rejects bad arguments before it
touches the GPU (no call here launches a kernel)."""

import ctypes
import os
import re
import subprocess

import pytest
from hypothesis import given, settings, strategies as st

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")

L = pytest.importorskip("sparse_mixture_experts_moe_amd._lib",
                        reason="libmoe not built (python -m sparse_mixture_experts_moe_amd.build)")
C = L._L
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(L.EXPORTED) == names  # the binding declares exactly these


def test_version_and_strings():
    assert L.moe_abi_version() == 4
    assert L.moe_status_string(L.MOE_OK) == "ok"
    assert L.moe_status_string(L.MOE_EWORKSPACE) == "workspace too small"
    assert L.moe_status_string(99) == "unknown status"


def test_capacity_worked():
    assert L.moe_capacity(1.25, 16384, 2, 64) == 640
    assert L.moe_capacity(0.1, 10, 1, 1) == 1
    assert L.moe_capacity(1.1, 100, 1, 10) == 11
    assert L.moe_capacity(0.0, 10, 2, 3) == -1
    assert L.moe_capacity(-1.0, 10, 2, 3) == -1
    assert L.moe_capacity(float("nan"), 10, 2, 3) == -1
    assert L.moe_capacity(1.0, -1, 2, 3) == -2
    assert L.moe_capacity(1e-300, 10, 2, 3) == 1
    assert L.moe_capacity(1e300, 10, 2, 3) == 2 ** 63 - 1


@settings(max_examples=400, deadline=None)
@given(st.floats(min_value=1e-6, max_value=1e6, allow_nan=False, allow_infinity=False),
       st.integers(1, 10 ** 7), st.integers(1, 32), st.integers(1, 256))
def test_capacity_matches_oracle(cf, T, k, E):
    assert L.moe_capacity(cf, T, k, E) == oracle.capacity(cf, T, k, E)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 10 ** 6), st.integers(1, 32), st.integers(1, 256),
       st.integers(1, 400).map(lambda n: n / 100))
def test_capacity_two_decimal_factors(T, k, E, cf):
    # factors written with two decimals, as configs write them
    assert L.moe_capacity(cf, T, k, E) == oracle.capacity(cf, T, k, E)


def _err():
    return L.moe_last_error()


def test_route_rejects():
    s = C.moe_route(FAKE, FAKE, L.MOE_BF16, 64, 128, 8, 9, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EINVAL and "k <= E" in _err()
    s = C.moe_route(None, FAKE, L.MOE_BF16, 64, 128, 8, 2, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EINVAL
    s = C.moe_route(FAKE, FAKE, L.MOE_BF16, 64, 128, 300, 2, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EUNSUPPORTED
    s = C.moe_route(FAKE, FAKE, L.MOE_BF16, 64, 100, 8, 2, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EUNSUPPORTED and "d % 32" in _err()
    s = C.moe_route(FAKE, FAKE, 7, 64, 128, 8, 2, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EINVAL
    s = C.moe_route(FAKE, FAKE, L.MOE_F32, 64, 128, 64, 33, None, None, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EUNSUPPORTED
    s = C.moe_route(FAKE, FAKE, L.MOE_F32, 64, 128, 8, 2, None, None, 8, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EINVAL and "flags" in _err()
    # ReLU routing takes no selection bias, on the logits or on the probabilities
    s = C.moe_route(FAKE, FAKE, L.MOE_F32, 64, 128, 8, 2, None, FAKE, L.MOE_ROUTE_RELU, FAKE, FAKE,
                    FAKE, None, 0, None)
    assert s == L.MOE_EINVAL and "ReLU" in _err()
    s = C.moe_route(FAKE, FAKE, L.MOE_F32, 64, 128, 8, 2, None, None,
                    L.MOE_ROUTE_RELU | L.MOE_ROUTE_BIAS_ON_PROBS, FAKE, FAKE, FAKE, None, 0, None)
    assert s == L.MOE_EINVAL and "ReLU" in _err()
    # T = 0 is a no-op that enqueues nothing
    assert C.moe_route(FAKE, FAKE, L.MOE_F32, 0, 128, 8, 2, None, None, 0, FAKE, FAKE, FAKE,
                       None, 0, None) == L.MOE_OK
    assert _err() == ""
    # a small bf16 batch splits the reduction over d and needs a workspace
    need = L.moe_route_workspace(64, 6144, 128, 8, L.MOE_BF16)
    assert need > 0
    s = C.moe_route(FAKE, FAKE, L.MOE_BF16, 64, 6144, 128, 8, None, None, 0, FAKE, FAKE, FAKE,
                    FAKE, need - 1, None)
    assert s == L.MOE_EWORKSPACE
    assert L.moe_route_workspace(64, 6144, 128, 8, L.MOE_F32) == 0


def test_permute_rejects():
    ws = L.moe_permute_workspace(100, 2, 8)
    assert ws > 0
    s = C.moe_permute(FAKE, 100, 2, 8, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 1,
                      None)
    assert s == L.MOE_EWORKSPACE
    s = C.moe_permute(None, 100, 2, 8, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert s == L.MOE_EINVAL
    s = C.moe_permute(FAKE, 100, 2, 8, -1, FAKE, L.MOE_BF16, 64, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                      ws, None)
    assert s == L.MOE_EINVAL and "x_perm" in _err()
    s = C.moe_permute(FAKE, 100, 3, 2, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert s == L.MOE_EINVAL


def test_permute_noalloc_rejects():
    """The no-allocation permute checks its arguments, and the static scratch's
    limit of 2^20 pairs, on the host before it looks up the scratch or
    launches anything."""
    s = C.moe_permute_noalloc(FAKE, 131072 + 1, 8, 8, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE,
                              None, None)
    assert s == L.MOE_EUNSUPPORTED and "scratch" in _err()
    s = C.moe_permute_noalloc(FAKE, 100, 2, 300, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None,
                              None)
    assert s == L.MOE_EUNSUPPORTED
    s = C.moe_permute_noalloc(FAKE, 100, 3, 2, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None)
    assert s == L.MOE_EINVAL
    s = C.moe_permute_noalloc(None, 100, 2, 8, -1, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None, None)
    assert s == L.MOE_EINVAL
    s = C.moe_permute_noalloc(FAKE, 100, 2, 8, -1, FAKE, L.MOE_BF16, 64, FAKE, FAKE, FAKE, FAKE,
                              None, None)
    assert s == L.MOE_EINVAL and "x_perm" in _err()


def test_expert_swiglu_rejects():
    ws = L.moe_expert_swiglu_workspace(1000, 128, 256, 8, L.MOE_BF16)
    assert ws >= 1000 * 256 * 2
    args = dict(a=FAKE, dt=L.MOE_BF16, d=128, h=256, G=8, off=FAKE, mr=1000, rows=None, div=1,
                wg=FAKE, wu=FAKE, wd=FAKE, y=FAKE, ydt=L.MOE_BF16, ws=FAKE, nws=ws)

    def call(**kw):
        a = dict(args, **kw)
        return C.moe_expert_swiglu_gather(a["a"], a["dt"], a["d"], a["h"], a["G"], a["off"],
                                          a["mr"], a["rows"], a["div"], a["wg"], a["wu"], a["wd"],
                                          a["y"], a["ydt"], a["ws"], a["nws"], None)

    assert call(nws=ws - 1) == L.MOE_EWORKSPACE
    assert call(d=100) == L.MOE_EUNSUPPORTED
    assert call(h=96) == L.MOE_EUNSUPPORTED
    # one expert's bf16 weight matrix must fit 32-bit byte offsets
    assert call(d=65536, h=32768, nws=L.moe_expert_swiglu_workspace(1000, 65536, 32768, 8,
                                                                    L.MOE_BF16)) == L.MOE_EUNSUPPORTED
    assert "4 GiB" in _err()
    assert call(wd=None) == L.MOE_EINVAL
    assert call(rows=FAKE, div=0) == L.MOE_EINVAL
    assert call(G=0) == L.MOE_EINVAL
    assert call(ydt=5) == L.MOE_EINVAL
    # no rows: nothing to do
    assert call(mr=0, nws=L.moe_expert_swiglu_workspace(0, 128, 256, 8, L.MOE_BF16)) == L.MOE_OK
    # the plain call without the row index checks the same way
    assert C.moe_expert_swiglu(FAKE, L.MOE_BF16, 128, 256, 8, FAKE, 1000, FAKE, FAKE, FAKE, FAKE,
                               L.MOE_BF16, FAKE, ws - 1, None) == L.MOE_EWORKSPACE
    assert C.moe_expert_swiglu(FAKE, L.MOE_BF16, 100, 256, 8, FAKE, 1000, FAKE, FAKE, FAKE, FAKE,
                               L.MOE_BF16, FAKE, ws, None) == L.MOE_EUNSUPPORTED
    # the workgroup-limited call checks the same way, whatever the limit
    for cus in (-1, 0, 8, 100, 1 << 20):
        assert C.moe_expert_swiglu_cus(FAKE, L.MOE_BF16, 128, 256, 8, FAKE, 1000, None, 1, FAKE,
                                       FAKE, FAKE, FAKE, L.MOE_BF16, FAKE, ws - 1, cus,
                                       None) == L.MOE_EWORKSPACE
        assert C.moe_expert_swiglu_cus(FAKE, L.MOE_BF16, 128, 256, 8, FAKE, 1000, FAKE, 0, FAKE,
                                       FAKE, FAKE, FAKE, L.MOE_BF16, FAKE, ws, cus,
                                       None) == L.MOE_EINVAL
        assert C.moe_expert_swiglu_cus(FAKE, L.MOE_BF16, 128, 256, 8, FAKE, 0, None, 1, FAKE,
                                       FAKE, FAKE, FAKE, L.MOE_BF16, FAKE,
                                       L.moe_expert_swiglu_workspace(0, 128, 256, 8, L.MOE_BF16),
                                       cus, None) == L.MOE_OK


def test_combine_and_stats_reject():
    assert C.moe_combine(None, L.MOE_BF16, FAKE, FAKE, 10, 2, 64, None, FAKE, L.MOE_BF16,
                         None) == L.MOE_EINVAL
    assert C.moe_combine(FAKE, L.MOE_BF16, FAKE, FAKE, 10, 0, 64, None, FAKE, L.MOE_BF16,
                         None) == L.MOE_EINVAL
    assert C.moe_combine(FAKE, L.MOE_BF16, FAKE, FAKE, 0, 2, 64, None, FAKE, L.MOE_BF16,
                         None) == L.MOE_OK
    ws = L.moe_balance_stats_workspace(1000, 64)
    assert C.moe_balance_stats_z(FAKE, FAKE, 1000, 64, 2, 0.01, FAKE, FAKE, FAKE, None, FAKE,
                                 ws - 1, None) == L.MOE_EWORKSPACE
    assert C.moe_balance_stats_z(FAKE, FAKE, 1000, 300, 2, 0.01, FAKE, FAKE, FAKE, None, FAKE, ws,
                                 None) == L.MOE_EUNSUPPORTED
    assert C.moe_balance_stats_z(FAKE, None, 1000, 64, 2, 0.01, FAKE, FAKE, FAKE, None, FAKE, ws,
                                 None) == L.MOE_EINVAL
    # the plain call without the z-loss output
    assert C.moe_balance_stats(FAKE, FAKE, 1000, 64, 2, 0.01, FAKE, FAKE, FAKE, FAKE, ws - 1,
                               None) == L.MOE_EWORKSPACE
    assert C.moe_balance_stats(FAKE, None, 1000, 64, 2, 0.01, FAKE, FAKE, FAKE, FAKE, ws,
                               None) == L.MOE_EINVAL


def test_probes_reject():
    assert C.moe_probe_mfma_bf16(FAKE, 0, 10, FAKE, None) == L.MOE_EINVAL
    assert C.moe_probe_mfma_bf16(FAKE, 4, 0, FAKE, None) == L.MOE_EINVAL
    assert C.moe_probe_mfma_bf16(None, 4, 10, FAKE, None) == L.MOE_EINVAL
    assert C.moe_probe_read(FAKE, 24, 4, FAKE, None) == L.MOE_EINVAL and "multiple of 16" in _err()
    assert C.moe_probe_read(FAKE, 0, 4, FAKE, None) == L.MOE_EINVAL
    assert C.moe_probe_read(FAKE, 1024, 0, FAKE, None) == L.MOE_EINVAL
    assert C.moe_probe_read(FAKE, 1024, 4, None, None) == L.MOE_EINVAL


def test_backward_rejects():
    F32, BF = L.MOE_F32, L.MOE_BF16
    # expert backward: dtype, shapes, pointers, workspace
    ws = L.moe_expert_swiglu_backward_workspace(1000, 128, 256, 4, BF, True)
    assert ws > 0 and L.moe_expert_swiglu_backward_workspace(1000, 128, 256, 4, F32, True) > 0
    assert L.moe_expert_swiglu_backward_workspace(1000, 128, 256, 4, 7, True) == 0
    assert ws > L.moe_expert_swiglu_backward_workspace(1000, 128, 256, 4, BF, False)
    args = [FAKE, BF, 128, 256, 4, FAKE, 1000, FAKE, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    s = C.moe_expert_swiglu_backward(*args[:1], 7, *args[2:])
    assert s == L.MOE_EINVAL
    s = C.moe_expert_swiglu_backward(*args[:2], 100, *args[3:])
    assert s == L.MOE_EUNSUPPORTED and "% 64" in _err()
    s = C.moe_expert_swiglu_backward(*args[:9], None, *args[10:])
    assert s == L.MOE_EINVAL
    s = C.moe_expert_swiglu_backward(*args[:20], ws - 1, None)
    assert s == L.MOE_EWORKSPACE
    s = C.moe_expert_swiglu_backward(*args[:8], 0, *args[9:])
    assert s == L.MOE_EINVAL and "a_rows_div" in _err()
    # training gate/up: uv required
    s = C.moe_expert_gate_up_train(FAKE, BF, 128, 256, 4, FAKE, 100, None, 1, FAKE, FAKE, FAKE,
                                   None, FAKE, 1 << 30, None)
    assert s == L.MOE_EINVAL
    # combine backward: dout needs the gates
    s = C.moe_combine_backward(FAKE, BF, FAKE, BF, FAKE, None, 10, 2, 64, FAKE, FAKE, None)
    assert s == L.MOE_EINVAL
    assert C.moe_combine_backward(FAKE, 7, FAKE, BF, FAKE, FAKE, 10, 2, 64, FAKE, None, None) == L.MOE_EINVAL
    assert C.moe_combine_backward(None, BF, None, BF, None, None, 0, 2, 64, None, None, None) == L.MOE_OK
    # route backward: k <= E, counts needed with the balance term
    assert C.moe_route_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 4, 5, 0, 0.01, 0.0, 0.0, FAKE,
                                None) == L.MOE_EINVAL
    assert C.moe_route_backward(FAKE, FAKE, FAKE, FAKE, None, 10, 8, 2, 0, 0.01, 1.0, 0.0, FAKE,
                                None) == L.MOE_EINVAL
    assert C.moe_route_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 300, 2, 0, 0.01, 1.0, 0.0, FAKE,
                                None) == L.MOE_EUNSUPPORTED
    # the only flag is MOE_ROUTE_RELU
    assert C.moe_route_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 8, 2, L.MOE_ROUTE_LOGITS_IN, 0.01,
                                1.0, 0.0, FAKE, None) == L.MOE_EINVAL
    assert "flags" in _err()
    assert C.moe_route_backward(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 2, L.MOE_ROUTE_RELU, 0.01,
                                1.0, 0.0, FAKE, None) == L.MOE_OK
    # router backward: workspace only with dw_router
    need = L.moe_router_backward_workspace(4096, 1024, 8)
    assert need > 0
    s = C.moe_router_backward(FAKE, FAKE, BF, FAKE, 4096, 1024, 8, FAKE, None, None, 0, FAKE,
                              need - 1, None)
    assert s == L.MOE_EWORKSPACE
    s = C.moe_router_backward(None, FAKE, BF, FAKE, 4096, 1024, 8, FAKE, None, None, 0, FAKE,
                              need, None)
    assert s == L.MOE_EINVAL


def test_balance_rejects():
    # the budgets are required; bad k
    s = C.moe_permute_budgets(FAKE, 100, 2, 8, None, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None,
                              FAKE, 1 << 20, None)
    assert s == L.MOE_EINVAL and "expert_capacity" in _err()
    s = C.moe_permute_budgets(FAKE, 100, 9, 8, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None,
                              FAKE, 1 << 20, None)
    assert s == L.MOE_EINVAL
    ws = L.moe_permute_workspace(100, 2, 8)
    s = C.moe_permute_budgets(FAKE, 100, 2, 8, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, None,
                              FAKE, ws - 1, None)
    assert s == L.MOE_EWORKSPACE
    # update: finite arguments, decay in [0, 1], a rolling-load buffer
    nan = float("nan")
    assert C.moe_balance_update(FAKE, 100, 2, 8, None, 0.1, FAKE, 0.5, nan, 1.0, None,
                                None) == L.MOE_EINVAL
    assert C.moe_balance_update(FAKE, 100, 2, 8, None, 0.1, FAKE, 1.5, 1.0, 1.0, None,
                                None) == L.MOE_EINVAL
    assert C.moe_balance_update(FAKE, 100, 2, 8, None, 0.1, None, 0.5, 1.0, 1.0, None,
                                None) == L.MOE_EINVAL
    assert C.moe_balance_update(FAKE, 0, 2, 8, None, 0.1, FAKE, 0.5, 1.0, 1.0, None,
                                None) == L.MOE_EINVAL
    assert C.moe_balance_update(FAKE, 100, 2, 300, None, 0.1, FAKE, 0.5, 1.0, 1.0, None,
                                None) == L.MOE_EUNSUPPORTED


def test_combine_bypass_rejects():
    f = C.moe_combine_bypass
    args = lambda **kw: dict(dict(y=FAKE, ydt=L.MOE_BF16, pr=FAKE, idx=FAKE, g=FAKE, T=16, k=2,  # noqa: E731
                                  d=64, ef=8, nz=1, nc=1, nk=2, x=FAKE, cr=FAKE, sh=None, out=FAKE,
                                  odt=L.MOE_BF16), **kw)

    def call(**kw):
        a = args(**kw)
        return f(a["y"], a["ydt"], a["pr"], a["idx"], a["g"], a["T"], a["k"], a["d"], a["ef"],
                 a["nz"], a["nc"], a["nk"], a["x"], a["cr"], a["sh"], a["out"], a["odt"], None)
    assert call(k=0) == L.MOE_EINVAL
    assert call(nz=-1) == L.MOE_EINVAL and "negative" in _err()
    assert call(ef=250, nk=7) == L.MOE_EUNSUPPORTED
    assert call(ydt=5) == L.MOE_EINVAL
    assert call(idx=None) == L.MOE_EINVAL
    assert call(x=None) == L.MOE_EINVAL and "x or const_rows" in _err()
    assert call(cr=None) == L.MOE_EINVAL
    assert call(T=0, idx=None, x=None) == L.MOE_OK
    # no copy or constant experts: x and const_rows may be NULL (checked only)
    assert call(T=0, nc=0, nk=0, x=None, cr=None) == L.MOE_OK


def test_bypass_backward_rejects():
    BF = L.MOE_BF16
    f = C.moe_combine_backward_bypass
    assert f(FAKE, BF, FAKE, BF, FAKE, FAKE, FAKE, 16, 0, 64, 8, 1, 1, 2, FAKE, FAKE, FAKE, None,
             None) == L.MOE_EINVAL
    assert f(FAKE, BF, FAKE, BF, FAKE, FAKE, FAKE, 16, 2, 64, 8, 1, 1, 2, None, FAKE, FAKE, None,
             None) == L.MOE_EINVAL and "x or const_rows" in _err()
    assert f(FAKE, BF, FAKE, BF, FAKE, None, FAKE, 16, 2, 64, 8, 1, 1, 2, FAKE, FAKE, FAKE, None,
             None) == L.MOE_EINVAL
    assert f(FAKE, BF, FAKE, BF, FAKE, FAKE, FAKE, 16, 2, 64, 250, 1, 1, 9, FAKE, FAKE, FAKE, None,
             None) == L.MOE_EUNSUPPORTED
    assert f(None, BF, None, BF, None, None, None, 0, 2, 64, 8, 1, 1, 2, None, None, None, None,
             None) == L.MOE_OK
    g = C.moe_bypass_backward
    need = L.moe_bypass_backward_workspace(4096, 1024, 2)
    assert need >= 2 * 1024 * 4
    assert g(FAKE, BF, FAKE, FAKE, 4096, 2, 1024, 8, 1, 1, 2, FAKE, FAKE, FAKE, need - 1,
             None) == L.MOE_EWORKSPACE
    assert g(FAKE, BF, FAKE, FAKE, 4096, 2, 1024, 8, 1, 1, 2, None, FAKE, FAKE, need,
             None) == L.MOE_EINVAL and "dx_acc" in _err()
    assert g(FAKE, BF, FAKE, FAKE, 4096, 2, 1024, 8, 1, 1, 2, FAKE, None, FAKE, need,
             None) == L.MOE_EINVAL
    assert g(FAKE, 9, FAKE, FAKE, 4096, 2, 1024, 8, 1, 1, 2, FAKE, FAKE, FAKE, need,
             None) == L.MOE_EINVAL
    # no copy and no constant experts: nothing to do beyond the checks
    assert g(FAKE, BF, FAKE, FAKE, 0, 2, 1024, 8, 1, 0, 0, None, None, None, 0, None) == L.MOE_OK

