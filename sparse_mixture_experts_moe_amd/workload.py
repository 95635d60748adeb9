"""Builds an MoELayer from host arrays (as ``moe_inputs.generate`` returns
them): uploads the tensors, concatenates the shared experts along the hidden
axis and derives the capacity with the library's moe_capacity."""

from __future__ import annotations

import numpy as np
import torch

from . import _lib
from .layer import MoELayer


def to_device(a, dev="cuda"):
    """float32 array, or an object holding bfloat16 bit patterns in ``.bits``,
    as a device tensor."""
    if a is None:
        return None
    bits = getattr(a, "bits", None)
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


def _rows(a, i, dev):
    bits = getattr(a, "bits", None)
    return to_device(a[i] if bits is None else type(a)(bits[i]), dev)


def concat_shared(inp, dev="cuda"):
    """(gate [n_s h_s, d], up [n_s h_s, d], down [d, n_s h_s]) or None."""
    if inp.get("shared_gate") is None:
        return None
    ns = inp["shared_gate"].shape[0]
    g = torch.cat([_rows(inp["shared_gate"], s, dev) for s in range(ns)], dim=0)
    u = torch.cat([_rows(inp["shared_up"], s, dev) for s in range(ns)], dim=0)
    d = torch.cat([_rows(inp["shared_down"], s, dev) for s in range(ns)], dim=1)
    return g.contiguous(), u.contiguous(), d.contiguous()


def layer_from_inputs(inp, gather="fused", dev="cuda"):
    cfg = inp["cfg"]
    cap = _lib.moe_capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    return MoELayer(to_device(inp["w_router"], dev), to_device(inp["w_gate"], dev),
                    to_device(inp["w_up"], dev), to_device(inp["w_down"], dev), cfg.k,
                    shared=concat_shared(inp, dev), logit_bias=to_device(inp["logit_bias"], dev),
                    select_bias=to_device(inp["select_bias"], dev), capacity=cap,
                    alpha=cfg.alpha, gather=gather)


def relu_logit_bias(inp, offset):
    """The logit bias of the ReLU-routed layer: the workload's own (if any)
    plus a constant ``offset``, float32 [E]."""
    E = inp["cfg"].E
    lb = np.zeros(E, dtype=np.float32) if inp["logit_bias"] is None else inp["logit_bias"]
    return (np.asarray(lb, dtype=np.float32) + np.float32(offset)).astype(np.float32)


def relu_layer_from_inputs(inp, k_max, offset, gather="fused", dev="cuda"):
    """The workload's layer with ReLU routing: at most ``k_max`` experts per
    token, those whose logit (with ``relu_logit_bias(inp, offset)``) is
    positive.  The workload's selection bias is not used."""
    cfg = inp["cfg"]
    cap = _lib.moe_capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    lb = relu_logit_bias(inp, offset)
    return MoELayer(to_device(inp["w_router"], dev), to_device(inp["w_gate"], dev),
                    to_device(inp["w_up"], dev), to_device(inp["w_down"], dev), k_max,
                    shared=concat_shared(inp, dev), logit_bias=to_device(lb, dev), capacity=cap,
                    alpha=cfg.alpha, gather=gather, relu=True)


def bypass_layer_from_inputs(inp, router_rows, const_rows, n_zero, n_copy, gather="fused",
                             dev="cuda"):
    """The workload's layer with zero-computation experts: ``router_rows``
    [n_zero + n_copy + n_const, d] are appended to w_router (zero experts
    first, then copy, then constant), ``const_rows`` [n_const, d] are the
    constant experts' outputs.  The workload's logit and selection biases are
    not used (they have one entry per FFN expert)."""
    cfg = inp["cfg"]
    cap = _lib.moe_capacity(cfg.cf, cfg.T, cfg.k, cfg.E)
    wr = torch.cat([to_device(inp["w_router"], dev), to_device(router_rows, dev)], 0).contiguous()
    cr = to_device(const_rows, dev) if const_rows.shape[0] else None
    return MoELayer(wr, to_device(inp["w_gate"], dev), to_device(inp["w_up"], dev),
                    to_device(inp["w_down"], dev), cfg.k, shared=concat_shared(inp, dev),
                    capacity=cap, alpha=cfg.alpha, gather=gather,
                    bypass=dict(n_zero=n_zero, n_copy=n_copy, const_rows=cr))
