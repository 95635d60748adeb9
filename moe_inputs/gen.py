"""Seeded synthetic inputs for the MoE layer.

Holds none of the method's arithmetic: it only draws random tensors.  Both the
HIP path (through the tests and the benchmark) and the oracle read the arrays
made here.

Recipe (per workload ``cfg`` and seed):
  every tensor has its own PCG64 stream, SeedSequence([seed, cfg.cid, tensor_id]);
  tensor ids: x = 0, w_router = 1, routed expert e: w_gate 2+3e, w_up 3+3e,
  w_down 4+3e; shared expert s: 2+3E+3s, 3+3E+3s, 4+3E+3s; logit_bias
  2+3E+3n_s; select_bias 3+3E+3n_s.
  values are float32 standard normals times the scale below; for bfloat16
  workloads they are then rounded to bfloat16, round-to-nearest-even.
    x                       N(0, 1)
    w_router, w_gate, w_up  N(0, 1/d)          (fan-in d)
    w_down                  N(0, 1/h)          (fan-in h, or h_shared)
    logit_bias "zipf"       -s * ln(e + 1), e = 0..E-1: the log of a Zipf(s)
                            prior over experts (expert 0 the most popular)
    select_bias "normal"    N(0, select_var), float32
  backward pass (``generate_dy``): the upstream gradient dy [T, d] of the
  layer output, N(0, 1), tensor id 4 + 3E + 3n_s, in the workload's dtype.
Biases always stay float32.

bfloat16 tensors are returned as ``Bf16`` objects holding the uint16 bit
patterns; ``Bf16.f32()`` (or indexing) gives the exact values as float32.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import MoEConfig


def _stream(seed: int, cid: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tid])))


def bf16_bits_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class Bf16:
    """A bfloat16 tensor kept as uint16 bit patterns."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits

    @property
    def shape(self):
        return self.bits.shape

    def f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.bits)

    def __getitem__(self, i):
        return bf16_bits_to_f32(self.bits[i])

    def __len__(self):
        return self.bits.shape[0]


def _draw(seed, cid, tid, shape, scale, dtype):
    z = _stream(seed, cid, tid).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    return bf16_bits_rne(z) if dtype == "bf16" else z


def _workers(threads):
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def generate(cfg: MoEConfig, seed: int = 0, threads: int | None = None) -> dict:
    """All inputs of one layer call for workload ``cfg``.

    Returns a dict: x, w_router, w_gate [E,h,d], w_up [E,h,d], w_down [E,d,h],
    shared_gate/shared_up [n_s, h_s, d], shared_down [n_s, d, h_s] (or None),
    logit_bias [E] / select_bias [E] float32 (or None).
    Tensors are float32 arrays for "f32" workloads and ``Bf16`` for "bf16".
    """
    T, d, E, h, dt = cfg.T, cfg.d, cfg.E, cfg.h, cfg.dtype
    store = np.uint16 if dt == "bf16" else np.float32
    w_gate = np.empty((E, h, d), dtype=store)
    w_up = np.empty((E, h, d), dtype=store)
    w_down = np.empty((E, d, h), dtype=store)
    ns, hs = cfg.n_shared, cfg.h_shared
    sg = np.empty((ns, hs, d), dtype=store) if ns else None
    su = np.empty((ns, hs, d), dtype=store) if ns else None
    sd = np.empty((ns, d, hs), dtype=store) if ns else None

    jobs = []
    for e in range(E):
        jobs.append((w_gate, e, 2 + 3 * e, (h, d), cfg.sigma_in))
        jobs.append((w_up, e, 3 + 3 * e, (h, d), cfg.sigma_in))
        jobs.append((w_down, e, 4 + 3 * e, (d, h), cfg.sigma_down))
    for s in range(ns):
        b = 2 + 3 * E + 3 * s
        jobs.append((sg, s, b, (hs, d), cfg.sigma_in))
        jobs.append((su, s, b + 1, (hs, d), cfg.sigma_in))
        jobs.append((sd, s, b + 2, (d, hs), cfg.sigma_down_shared))

    def run(job):
        dst, i, tid, shape, scale = job
        dst[i] = _draw(seed, cfg.cid, tid, shape, scale, dt)

    with ThreadPoolExecutor(_workers(threads)) as ex:
        list(ex.map(run, jobs))

    x = _draw(seed, cfg.cid, 0, (T, d), 1.0, dt)
    w_router = _draw(seed, cfg.cid, 1, (E, d), cfg.sigma_in, dt)

    lb_tid = 2 + 3 * E + 3 * ns
    logit_bias = None
    if cfg.logit_bias == "zipf":
        logit_bias = (-cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    select_bias = None
    if cfg.select_bias == "normal":
        select_bias = _stream(seed, cfg.cid, lb_tid + 1).standard_normal(E, dtype=np.float32)
        select_bias *= np.float32(math.sqrt(cfg.select_var))

    wrap = (lambda a: Bf16(a)) if dt == "bf16" else (lambda a: a)
    return dict(
        cfg=cfg,
        x=wrap(x), w_router=wrap(w_router),
        w_gate=wrap(w_gate), w_up=wrap(w_up), w_down=wrap(w_down),
        shared_gate=wrap(sg) if ns else None,
        shared_up=wrap(su) if ns else None,
        shared_down=wrap(sd) if ns else None,
        logit_bias=logit_bias, select_bias=select_bias,
    )


def as_f32(a):
    """Exact float32 values of a generated tensor (float32 array or Bf16)."""
    if a is None:
        return None
    return a.f32() if isinstance(a, Bf16) else np.asarray(a, dtype=np.float32)


def generate_dy(cfg: MoEConfig, seed: int = 0):
    """Upstream gradient dy [T, d] of the layer output for the backward pass:
    N(0, 1) in the workload's dtype (``Bf16`` for bf16 workloads)."""
    tid = 4 + 3 * cfg.E + 3 * cfg.n_shared
    z = _draw(seed, cfg.cid, tid, (cfg.T, cfg.d), 1.0, cfg.dtype)
    return Bf16(z) if cfg.dtype == "bf16" else z


def generate_bypass(cfg: MoEConfig, n_zero: int, n_copy: int, n_const: int, seed: int = 0):
    """Inputs of the zero-computation experts added to workload ``cfg``: their
    router rows [n_zero + n_copy + n_const, d] (drawn like w_router, to be
    appended after its E rows) and the constant experts' rows [n_const, d],
    N(0, 1).  Returned in the workload's dtype (``Bf16`` for bf16)."""
    tid = 5 + 3 * cfg.E + 3 * cfg.n_shared
    n = n_zero + n_copy + n_const
    rows = _draw(seed, cfg.cid, tid, (n, cfg.d), cfg.sigma_in, cfg.dtype)
    const = _draw(seed, cfg.cid, tid + 1, (n_const, cfg.d), 1.0, cfg.dtype)
    wrap = (lambda a: Bf16(a)) if cfg.dtype == "bf16" else (lambda a: a)
    return wrap(rows), wrap(const)


def relu_logit_offset(cfg: MoEConfig, k_mean: float) -> float:
    """The constant logit bias -tau that makes k_mean of the E logits of a
    token positive on average, for ReLU routing on untrained random weights:
    a logit of this generator is N(0, d sigma_in^2), so tau = sigma z with
    z the (1 - k_mean / E) normal quantile."""
    from statistics import NormalDist
    sigma = math.sqrt(cfg.d) * cfg.sigma_in
    return -sigma * NormalDist().inv_cdf(1.0 - k_mean / cfg.E)
