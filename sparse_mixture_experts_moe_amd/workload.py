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
