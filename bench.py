#!/usr/bin/env python3
"""MoE-layer forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward pass of the whole layer (route, permute, routed expert
GEMMs, shared experts, combine, balance statistics) over one batch of
synthetic inputs already resident in HBM.  Prints one JSON line with
tokens/s, the roofline of the dominant kernel (the fused gate/up grouped GEMM,
timed with HIP events on the stream it runs on) and the CPU oracle's
throughput on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/sec (1 GPU) + grouped-GEMM MFMA util % / HBM GB/s"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_bf16")
    ap.add_argument("--gather", default="fused", choices=["fused", "copy"])
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0: chosen per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(inp, cfg, n_tok):
    """The oracle as it stands, on the first n_tok tokens taken as a batch of
    their own (same shapes, weights, biases and capacity factor)."""
    import numpy as np

    import oracle
    from moe_inputs import as_f32
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    x = as_f32(inp["x"])[:n_tok]
    shared = ()
    if inp["shared_gate"] is not None:
        shared = [(inp["shared_gate"][s], inp["shared_up"][s], inp["shared_down"][s])
                  for s in range(cfg.n_shared)]
    cap = oracle.capacity(cfg.cf, n_tok, cfg.k, cfg.E)
    t0 = time.perf_counter()
    oracle.forward(x, as_f32(inp["w_router"]), inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k,
                   shared=shared, logit_bias=inp["logit_bias"], select_bias=inp["select_bias"],
                   cap=cap, alpha=cfg.alpha)
    dt = time.perf_counter() - t0
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tok} of {cfg.T} tokens of {cfg.name} as one batch "
                      f"(float64 NumPy, {dt:.1f} s)",
            "seconds": dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_inputs import WORKLOADS, generate
    from sparse_mixture_experts_moe_amd.workload import layer_from_inputs, to_device

    cfg = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = generate(cfg)
    print(f"# inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    layer = layer_from_inputs(inp, args.gather)
    x = to_device(inp["x"])
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        layer(x)
    torch.cuda.synchronize()

    marks = []

    def mark(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks[-1].append((name, ev))

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    t_host = time.perf_counter()
    for _ in range(args.steps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        marks.append([("start", ev0)])
        res = layer(x, mark=mark)
    end.record(stream)
    host_ms = (time.perf_counter() - t_host) * 1e3 / args.steps  # enqueue cost per step
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps

    phases = {}
    for step in marks:
        for (_, a), (name, b) in zip(step[:-1], step[1:]):
            phases.setdefault(name, []).append(a.elapsed_time(b))
    phase_ms = {k: float(np.mean(v)) for k, v in phases.items()}

    counts = res["expert_count"].cpu().numpy()
    offs = res["expert_offset"].cpu().numpy()
    kept = offs[1:] - offs[:-1]
    R_kept = int(offs[-1])
    touched = int(np.sum(kept > 0))
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    esz = 2 if cfg.dtype == "bf16" else 4

    # dominant kernel: the fused gate/up grouped GEMM (one moe_expert_gate_up call)
    gu_ms = phase_ms["gate_up"]
    gu_flops = 4.0 * R_kept * d * h
    gu_bytes = touched * 2 * h * d * esz + R_kept * (d + h) * esz
    if cfg.name.startswith("decode"):
        achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["kernel"] = "moe_expert_gate_up (fused gate/up grouped GEMM + SiLU*mul)"
    roof["per_launch"] = {"flops": gu_flops, "bytes": gu_bytes, "avg_ms": gu_ms}

    # whole-layer algorithmic work
    hs = cfg.n_shared * cfg.h_shared
    flops = 2.0 * T * d * E + 6.0 * d * h * R_kept + 6.0 * d * hs * T
    bytes_ = (T * d * esz * 2 + E * d * esz + touched * 3 * h * d * esz + 3 * hs * d * esz +
              T * E * 4 + T * k * 8)
    expert_ms = phase_ms["gate_up"] + phase_ms["down"] + phase_ms.get("shared", 0.0)
    expert_flops = 6.0 * d * h * R_kept + 6.0 * d * hs * T

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded normal inputs and random-init weights of the workload's shape)",
        "config": {"workload": cfg.name, "T": T, "d": d, "E": E, "k": k, "h": h,
                   "n_shared": cfg.n_shared, "h_shared": cfg.h_shared, "cf": cfg.cf,
                   "gather": args.gather, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "expert_gemm_mfma_util": expert_flops / (expert_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "layer_tflops": flops / (ms * 1e-3) / 1e12,
        "layer_hbm_gbs": bytes_ / (ms * 1e-3) / 1e9,
        "phase_ms": phase_ms,
        "host_enqueue_ms_per_step": host_ms,
        "routing": {"kept_pairs": R_kept, "dropped_pairs": T * k - R_kept,
                    "touched_experts": touched, "max_rows": int(kept.max()),
                    "min_rows": int(kept.min()), "max_demand": int(counts.max())},
    }
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or {"tiny_f32": 64, "mixtral_bf16": 256,
                                    "finegrained_shared_bf16": 512,
                                    "capacity_balance_bf16": 512, "decode_bf16": 64}[cfg.name]
        cb = cpu_baseline(inp, cfg, n_tok)
        cb.pop("seconds")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
