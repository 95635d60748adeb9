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
import gc
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
BYPASS_COUNTS = (1, 1, 2)   # zero, copy and constant experts of --variant bypass
RELU_K_MUL = 2              # --variant relu: at most RELU_K_MUL * k experts per token


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
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="time only --workload (by default the Mixtral-shaped headline run "
                         "also times the fine-grained, capacity and decode workloads and "
                         "reports them under \"workloads\")")
    ap.add_argument("--serial-shared", action="store_true",
                    help="run the shared experts in line on the layer's stream instead of "
                         "overlapping them on a second stream")
    ap.add_argument("--balance", action="store_true",
                    help="apply the per-step load-balancing updates after every step "
                         "(selection-bias step 1e-3, rolling-load decay 0.9, adaptive per-expert "
                         "budgets with C_base = the workload's capacity factor or 1 and gamma = E)")
    ap.add_argument("--variant", choices=["relu", "bypass"], default=None,
                    help="routing variant: ReLU routing (at most 2k experts per token, a logit "
                         "offset that makes k positive on average) or zero-computation experts "
                         "(1 zero, 1 copy, 2 constant after the FFN experts)")
    ap.add_argument("--backward", action="store_true",
                    help="time training steps instead: forward (keeping the pre-activations) "
                         "plus the backward pass of <dy, y> + loss + 1e-3 zloss")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the warmup, copy a buffer of this many MiB three times with a "
                         "plain device-to-device copy, so that a counter run can scale its byte "
                         "counters by a copy of known size (0: off)")
    return ap.parse_args()


def gate_up_sources():
    """The files the gate/up kernel is built from, hashed (comments and blank
    lines dropped) to tell whether a recorded traffic measurement still
    describes the kernel that runs."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("grouped_gemm.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "sparse_mixture_experts_moe_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from the counter summary in
    profiles/, or None when there is none or the kernel changed since."""
    import re
    path = os.path.join(ROOT, "profiles", f"gate_up_gemm_{workload}_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != gate_up_sources():
        return None
    return float(val.group(1))


def timing_events(torch, stream, n):
    """n timing events, each recorded once on ``stream`` (which creates the
    HIP event) and completed, ready to be recorded again in a timed region."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for ev in evs:
        ev.record(stream)
    torch.cuda.synchronize()
    return evs


def _median_ms(torch, fn, warmup=3, reps=7):
    """Median duration of fn() over reps launches (HIP events on the current
    stream, one pair per launch), after warmup launches.  All launches are
    enqueued back to back and synchronized once at the end, so that the
    device never idles between them (an idle device lowers its clock)."""
    import statistics
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for _ in range(warmup):
        fn()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in evs])


def measured_ceilings(torch, gemm_shape):
    """What this device sustains, measured right after the timed steps:
    bf16 MFMAs on register-resident random operands (no memory traffic), a
    streaming read of a 4 GiB buffer, and the vendor library's dense bf16 GEMM
    (hipBLASLt through torch.matmul) of the given shape [M, K, N]."""
    from sparse_mixture_experts_moe_amd import _lib as L
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4096
    src = torch.randn(ncu * 256 * 64, device="cuda").to(torch.bfloat16)
    out = torch.empty(ncu * 256, dtype=torch.float32, device="cuda")
    ms = _median_ms(torch, lambda: L.moe_probe_mfma_bf16(src, ncu, iters, out=out))
    mfma = ncu * 4 * iters * 16 * 32768 / (ms * 1e-3) / 1e12
    del src, out
    nbytes = 4 << 30
    buf = torch.full((nbytes // 4,), 0x01010101, dtype=torch.int32, device="cuda")
    rout = torch.empty(8192 * 256, dtype=torch.int32, device="cuda")
    ms = _median_ms(torch, lambda: L.moe_probe_read(buf, 8192, out=rout))
    hbm = nbytes / (ms * 1e-3) / 1e9
    del buf, rout
    res = {"mfma_bf16_tflops": mfma, "hbm_read_gbs": hbm,
           "how": f"MFMA: {ncu} workgroups x 4 waves x {iters} x 16 v_mfma_f32_32x32x16_bf16 on "
                  "random-normal register operands; read: 4 GiB streamed once in 16-byte non-temporal loads, "
                  "16 in flight per lane; "
                  "median of 7 launches after 3"}
    if gemm_shape is not None:
        res["library_gemm"] = library_gemm(torch, gemm_shape)
    torch.cuda.synchronize()
    return res


def library_gemm(torch, shape):
    """The vendor library's dense bf16 GEMM (hipBLASLt through torch.matmul)
    of shape [M, K, N]: median of 7 launches after 3."""
    M, K, N = shape
    a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    b = (torch.randn(K, N, device="cuda") * K ** -0.5).to(torch.bfloat16)
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ms = _median_ms(torch, lambda: torch.matmul(a, b, out=c))
    del a, b, c
    torch.cuda.synchronize()
    return {"shape_mkn": [M, K, N], "tflops": 2.0 * M * K * N / (ms * 1e-3) / 1e12, "ms": ms}


def cpu_threads():
    """Host threads of the oracle's timing: ``cores`` is the number of BLAS
    threads its matrix products ran on (the threads it actually used);
    ``host_cpus`` the CPUs this process may run on, len(os.sched_getaffinity(0));
    ``blas`` the BLAS library (threadpoolctl's report)."""
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:
        host = os.cpu_count() or 1
    threads, vendor = 1, "unknown"
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            threads = max(int(p.get("num_threads", 1)) for p in blas)
            vendor = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}"
                                       for p in blas}))
    except Exception:  # noqa: BLE001
        pass
    return {"cores": threads, "host_cpus": host, "blas": vendor, "blas_threads": threads}


def cpu_baseline(inp, cfg, n_tok, min_seconds=10.0, max_passes=5, variant=None):
    """The oracle as it stands, on the first n_tok tokens taken as a batch of
    their own (same shapes, weights, biases and capacity factor), repeated
    until at least min_seconds of CPU work (at most max_passes passes).
    ``variant`` = (kind, extras) runs the oracle of that routing variant."""
    import numpy as np

    import oracle
    from moe_inputs import as_f32
    cpu = cpu_threads()
    x = as_f32(inp["x"])[:n_tok]
    wr = as_f32(inp["w_router"])
    shared = ()
    if inp["shared_gate"] is not None:
        shared = [(inp["shared_gate"][s], inp["shared_up"][s], inp["shared_down"][s])
                  for s in range(cfg.n_shared)]
    cap = oracle.capacity(cfg.cf, n_tok, cfg.k, cfg.E)
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        if variant is None:
            oracle.forward(x, wr, inp["w_gate"], inp["w_up"], inp["w_down"], cfg.k,
                           shared=shared, logit_bias=inp["logit_bias"],
                           select_bias=inp["select_bias"], cap=cap, alpha=cfg.alpha)
        elif variant[0] == "relu":
            oracle.forward_relu(x, wr, inp["w_gate"], inp["w_up"], inp["w_down"],
                                variant[1]["k_max"], shared=shared,
                                logit_bias=variant[1]["logit_bias"], cap=cap, alpha=cfg.alpha)
        else:
            ex = variant[1]
            oracle.forward_bypass(x, np.concatenate([wr, as_f32(ex["rows"])], 0), inp["w_gate"],
                                  inp["w_up"], inp["w_down"], cfg.k, ex["n_zero"], ex["n_copy"],
                                  as_f32(ex["const"]), shared=shared, cap=cap, alpha=cfg.alpha)
        dt += time.perf_counter() - t0
        passes += 1
    return {"value": n_tok * passes / dt, "unit": "tokens/s", **cpu,
            "kind": "oracle",
            "sample": f"first {n_tok} of {cfg.T} tokens of {cfg.name}"
                      f"{'' if variant is None else ' (' + variant[0] + ' variant)'} as one "
                      f"batch, {passes} passes (float64 NumPy, {dt:.1f} s)"}


def cpu_baseline_backward(inp, dy, cfg, n_tok, c_bal, c_z, min_seconds=10.0, max_passes=5,
                          relu=None, bypass=None):
    """The backward oracle as it stands (its forward included) on the first
    n_tok tokens as a batch of their own, repeated until min_seconds.
    ``relu`` = (k_max, logit_bias) runs the ReLU-routed layer's oracle,
    ``bypass`` (the variant's dict) the one with zero-computation experts."""
    import numpy as np

    import oracle
    from moe_inputs import as_f32
    cpu = cpu_threads()
    x = as_f32(inp["x"])[:n_tok]
    dyf = as_f32(dy)[:n_tok]
    wr = as_f32(inp["w_router"])
    shared = ()
    if inp["shared_gate"] is not None:
        shared = [(inp["shared_gate"][s], inp["shared_up"][s], inp["shared_down"][s])
                  for s in range(cfg.n_shared)]
    wg, wu, wd = as_f32(inp["w_gate"]), as_f32(inp["w_up"]), as_f32(inp["w_down"])
    cap = oracle.capacity(cfg.cf, n_tok, cfg.k, cfg.E)
    passes, dt = 0, 0.0
    while passes < max_passes and (passes == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        if bypass is not None:
            oracle.backward_bypass(x, np.concatenate([wr, as_f32(bypass["rows"])], 0), wg, wu,
                                   wd, cfg.k, bypass["n_zero"], bypass["n_copy"],
                                   as_f32(bypass["const"]), dyf, shared=shared, cap=cap,
                                   alpha=cfg.alpha, c_bal=c_bal, c_z=c_z)
        elif relu is None:
            oracle.backward(x, wr, wg, wu, wd, cfg.k, dyf, shared=shared,
                            logit_bias=inp["logit_bias"], select_bias=inp["select_bias"], cap=cap,
                            alpha=cfg.alpha, c_bal=c_bal, c_z=c_z)
        else:
            oracle.backward_relu(x, wr, wg, wu, wd, relu[0], dyf, shared=shared,
                                 logit_bias=relu[1], cap=cap, alpha=cfg.alpha, c_bal=c_bal,
                                 c_z=c_z)
        dt += time.perf_counter() - t0
        passes += 1
    return {"value": n_tok * passes / dt, "unit": "tokens/s", **cpu,
            "kind": "oracle",
            "sample": f"first {n_tok} of {cfg.T} tokens of {cfg.name}"
                      f"{' (relu variant)' if relu else (' (bypass variant)' if bypass else '')}"
                      f" as one batch, forward and "
                      f"backward, {passes} passes (float64 NumPy, {dt:.1f} s)"}


def main_backward(args):
    """Training steps: forward(train=True) + backward, K timed steps."""
    import numpy as np
    import torch

    from moe_inputs import WORKLOADS, generate, generate_dy
    from sparse_mixture_experts_moe_amd.workload import layer_from_inputs, to_device

    cfg = WORKLOADS[args.workload]
    if cfg.dtype != "bf16":
        print(json.dumps({"error": "the backward pass runs in bf16 only"}), flush=True)
        sys.exit(2)
    c_bal, c_z = 1.0, 1e-3
    inp = generate(cfg)
    dy_h = generate_dy(cfg)
    layer = layer_from_inputs(inp, args.gather)
    relu = bypass = None
    if args.variant == "bypass":
        from moe_inputs import generate_bypass
        from sparse_mixture_experts_moe_amd.workload import bypass_layer_from_inputs
        rows, const = generate_bypass(cfg, *BYPASS_COUNTS)
        layer = bypass_layer_from_inputs(inp, rows, const, BYPASS_COUNTS[0], BYPASS_COUNTS[1],
                                         args.gather)
        bypass = {"n_zero": BYPASS_COUNTS[0], "n_copy": BYPASS_COUNTS[1],
                  "n_const": BYPASS_COUNTS[2], "rows": rows, "const": const}
    if args.variant == "relu":
        from moe_inputs import relu_logit_offset
        from sparse_mixture_experts_moe_amd.workload import relu_layer_from_inputs, relu_logit_bias
        off = relu_logit_offset(cfg, cfg.k)
        k_max = min(cfg.E, RELU_K_MUL * cfg.k)
        layer = relu_layer_from_inputs(inp, k_max, off, args.gather)
        relu = (k_max, relu_logit_bias(inp, off))
    layer.overlap_shared = not args.serial_shared
    x = to_device(inp["x"])
    dy = to_device(dy_h)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib > 0:  # a copy of known size for counter runs, before the warmup
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # timed region: events only around the expert backward call (the roofline);
    # events, collection and warmup ordered as in the forward measurement
    events = timing_events(torch, stream, 2 * args.steps + 2)
    ex_marks = []

    def mark_experts(name):
        if name in ("route_bwd", "experts_bwd"):  # enqueued right before / after the call
            ev = events.pop()
            ev.record(stream)
            ex_marks[-1].append(ev)

    start, end = events.pop(), events.pop()
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        layer.forward(x, train=True)
        layer.backward(dy, c_bal, c_z)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        ex_marks.append([])
        layer.forward(x, train=True)
        res = layer.backward(dy, c_bal, c_z, mark=mark_experts)
    end.record(stream)
    gc.enable()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    ex_ms = float(np.mean([a.elapsed_time(b) for a, b in ex_marks]))

    # phase breakdown in a separate pass (shared experts in line)
    marks = []

    def mark(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks[-1].append((name, ev))

    overlap = layer.overlap_shared
    layer.overlap_shared = False
    for _ in range(args.steps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        marks.append([("start", ev0)])
        layer.forward(x, mark=mark, train=True)
        layer.backward(dy, c_bal, c_z, mark=mark)
    torch.cuda.synchronize()
    layer.overlap_shared = overlap
    phases = {}
    for step in marks:
        for (_, a), (name, b) in zip(step[:-1], step[1:]):
            phases.setdefault(name, []).append(a.elapsed_time(b))
    phase_ms = {k: float(np.mean(v)) for k, v in phases.items()}

    offs = res["expert_offset"].cpu().numpy()[:layer.E + 1]  # the FFN experts
    kept = offs[1:] - offs[:-1]
    R_kept = int(offs[-1])
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    hs = cfg.n_shared * cfg.h_shared
    # the routed experts' backward call: five GEMMs, 12 d h flops per kept row
    ex_flops = 12.0 * R_kept * d * h
    achieved = ex_flops / (ex_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
            "kernel": "moe_expert_swiglu_backward (dgrad with SiLU-backward epilogue, dgrad of "
                      "the gate/up input, three weight-gradient GEMMs over each expert's rows, "
                      "the row gather of x)",
            "per_launch": {"flops": ex_flops, "avg_ms": ex_ms}}
    ceil = measured_ceilings(torch, None)
    roof["measured_peak"] = ceil["mfma_bf16_tflops"]
    roof["frac_of_measured"] = achieved / ceil["mfma_bf16_tflops"]
    step_flops = (2.0 * T * d * E) * 3 + 18.0 * d * h * R_kept + 18.0 * d * hs * T
    out = {
        "metric": "MoE-layer training tokens/sec (forward + backward, 1 GPU)",
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
        "data": "synthetic (seeded normal inputs, upstream gradient and random-init weights of "
                "the workload's shape)",
        "config": {"workload": cfg.name, "T": T, "d": d, "E": E, "k": k, "h": h,
                   "n_shared": cfg.n_shared, "h_shared": cfg.h_shared, "cf": cfg.cf,
                   "coef_balance": c_bal, "coef_z": c_z, "parallelism": "none (1 GPU)",
                   **({"variant": {"kind": "relu", "k_max": relu[0]}} if relu else {}),
                   **({"variant": {"kind": "bypass", "n_zero": bypass["n_zero"],
                                   "n_copy": bypass["n_copy"], "n_const": bypass["n_const"]}}
                      if bypass else {})},
        "roofline": roof,
        "measured_ceilings": ceil,
        "step_tflops": step_flops / (ms * 1e-3) / 1e12,
        "phase_ms": phase_ms,
        "phase_ms_source": "a separate pass of the same steps with a HIP event after every library "
                           "call (outside the timed region)",
        "routing": {"kept_pairs": R_kept, "max_rows": int(kept.max()), "min_rows": int(kept.min())},
    }
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or {"mixtral_bf16": 1024, "finegrained_shared_bf16": 2048,
                                    "capacity_balance_bf16": 2048, "decode_bf16": 64}[cfg.name]
        out["cpu_baseline"] = cpu_baseline_backward(inp, dy_h, cfg, n_tok, c_bal, c_z, relu=relu,
                                                    bypass=bypass)
    print(json.dumps(out), flush=True)


EXTRA_WORKLOADS = ("finegrained_shared_bf16", "capacity_balance_bf16", "decode_bf16")


def measure_forward(args, cfg, ceil=None, extra=False):
    """Forward steps of workload ``cfg``: ``args.warmup`` untimed steps, then
    ``args.steps`` timed ones, then the per-phase pass.  Returns (out, inp):
    the bench fields of this workload and its host inputs.  ``ceil`` reuses
    measured ceilings (else they are measured here); ``extra`` leaves out the
    variant, balance and copy-calibration options."""
    import numpy as np
    import torch

    from moe_inputs import generate
    from sparse_mixture_experts_moe_amd.workload import layer_from_inputs, to_device

    t_gen = time.perf_counter()
    inp = generate(cfg)
    print(f"# {cfg.name}: inputs generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)
    layer = layer_from_inputs(inp, args.gather)
    variant = None
    if args.variant == "relu" and not extra:
        from moe_inputs import relu_logit_offset
        from sparse_mixture_experts_moe_amd.workload import relu_layer_from_inputs, relu_logit_bias
        off = relu_logit_offset(cfg, cfg.k)
        k_max = min(cfg.E, RELU_K_MUL * cfg.k)
        layer = relu_layer_from_inputs(inp, k_max, off, args.gather)
        variant = ("relu", {"k_max": k_max, "logit_offset": off,
                            "logit_bias": relu_logit_bias(inp, off)})
    elif args.variant == "bypass" and not extra:
        from moe_inputs import generate_bypass
        from sparse_mixture_experts_moe_amd.workload import bypass_layer_from_inputs
        rows, const = generate_bypass(cfg, *BYPASS_COUNTS)
        layer = bypass_layer_from_inputs(inp, rows, const, BYPASS_COUNTS[0], BYPASS_COUNTS[1],
                                         args.gather)
        variant = ("bypass", {"n_zero": BYPASS_COUNTS[0], "n_copy": BYPASS_COUNTS[1],
                              "n_const": BYPASS_COUNTS[2], "rows": rows, "const": const})
    layer.overlap_shared = not args.serial_shared
    balance = None
    if args.balance and variant:
        raise SystemExit("--balance does not combine with --variant")
    if args.balance and not extra:
        balance = dict(bias_step=1e-3, ema_decay=0.9, cf_base=cfg.cf if cfg.cf > 0 else 1.0,
                       gamma=float(cfg.E))
        layer = type(layer)(layer.w_router, layer.w_gate, layer.w_up, layer.w_down, cfg.k,
                            shared=None if layer.shared is None else
                            tuple(w[0] for w in layer.shared),
                            logit_bias=layer.logit_bias, select_bias=layer.select_bias,
                            alpha=cfg.alpha, gather=args.gather,
                            overlap_shared=not args.serial_shared, balance=balance)
    x = to_device(inp["x"])
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(mark=None):
        res_ = layer(x, mark=mark)
        if balance:
            layer.update_balance()
            if mark:
                mark("balance_update")
        return res_
    if args.copy_calibration_mib > 0 and not extra:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Timed region: K steps with only the two events the roofline needs, around
    # the gate/up call (each event recorded on the stream delays the next
    # kernel by a few microseconds, so the per-phase events are kept out of
    # it).  Consecutive gate/up start events give the per-step durations.
    # The events are created (recorded once) and Python's garbage collector
    # runs before the warmup steps, and the collector stays paused until the
    # timed steps end: the timed steps then follow the warmup with nothing
    # but the synchronization between them (a GPU left idle for some 20 ms
    # lowers its clock, and the first steps after such a gap run up to 35%
    # slower), and no collection stalls the host while it enqueues them.
    events = timing_events(torch, stream, 2 * args.steps + 2)
    gu_marks = []

    def mark_gate_up(name):
        if name in ("permute", "gate_up"):  # enqueued right before / after the gate/up call
            ev = events.pop()
            ev.record(stream)
            gu_marks[-1].append(ev)

    start, end = events.pop(), events.pop()
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start.record(stream)
    t_host = time.perf_counter()
    for _ in range(args.steps):
        gu_marks.append([])
        res = step(mark_gate_up)
    end.record(stream)
    host_ms = (time.perf_counter() - t_host) * 1e3 / args.steps  # enqueue cost per step
    gc.enable()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    gu_step_ms = [a.elapsed_time(b) for a, b in gu_marks]
    step_ms = np.array([gu_marks[i][0].elapsed_time(gu_marks[i + 1][0])
                        for i in range(len(gu_marks) - 1)] or [ms])

    # Phase breakdown: a separate pass of the same K steps with an event after
    # every library call (outside the timed region; each phase includes the
    # few microseconds its opening event costs)
    # (the shared experts, which the timed steps overlap with the routed path
    # on a second stream, run in line here so that they get a phase of their own)
    marks = []

    def mark(name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream)
        marks[-1].append((name, ev))

    overlap = layer.overlap_shared
    layer.overlap_shared = False
    for _ in range(args.steps):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        marks.append([("start", ev0)])
        step(mark)
    torch.cuda.synchronize()
    layer.overlap_shared = overlap
    phases = {}
    for st in marks:
        for (_, a), (name, b) in zip(st[:-1], st[1:]):
            phases.setdefault(name, []).append(a.elapsed_time(b))
    phase_ms = {k: float(np.mean(v)) for k, v in phases.items()}

    # routing structure over the FFN experts (the zero-computation experts of
    # the bypass variant take no rows; ReLU routing leaves slots empty)
    E_ffn = layer.E
    counts = res["expert_count"].cpu().numpy()
    offs = res["expert_offset"].cpu().numpy()[:E_ffn + 1]
    kept = offs[1:] - offs[:-1]
    R_kept = int(offs[-1])
    touched = int(np.sum(kept > 0))
    used_slots = int((res["topk_idx"].cpu().numpy() >= 0).sum())
    bypass_pairs = int(counts[E_ffn:].sum())
    T, d, h, E, k = cfg.T, cfg.d, cfg.h, cfg.E, cfg.k
    esz = 2 if cfg.dtype == "bf16" else 4

    # dominant kernel: the fused gate/up grouped GEMM (one moe_expert_gate_up
    # call), its mean duration over the timed steps
    gu_ms = float(np.mean(gu_step_ms))
    gu_flops = 4.0 * R_kept * d * h
    gu_bytes = touched * 2 * h * d * esz + R_kept * (d + h) * esz
    if cfg.name.startswith("decode"):
        achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = gu_flops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    # HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counter runs
    # recorded in profiles/ (scaled by a plain copy of known size), or null
    roof["traffic"] = None if variant else recorded_traffic(cfg.name)
    # the vendor library's dense GEMM of the same FLOPs (one group of R_kept
    # rows, no gather, no SiLU), timed right after the steps as the layer was,
    # before the ceiling probes
    lib = None
    if roof["bound"] == "mfma" and cfg.dtype == "bf16" and R_kept > 0:
        lib = library_gemm(torch, (R_kept, d, 2 * h))
        roof["library_dense_gemm"] = lib
        roof["vs_library_dense"] = achieved / lib["tflops"]
    if ceil is None:
        ceil = measured_ceilings(torch, None)
        if lib is not None:
            ceil["library_gemm"] = lib
    if roof["bound"] == "hbm":
        roof["measured_peak"] = ceil["hbm_read_gbs"]
    elif cfg.dtype == "bf16":
        roof["measured_peak"] = ceil["mfma_bf16_tflops"]
    if "measured_peak" in roof:
        roof["frac_of_measured"] = roof["achieved"] / roof["measured_peak"]
    roof["kernel"] = "moe_expert_gate_up (fused gate/up grouped GEMM + SiLU*mul)"
    roof["per_launch"] = {"flops": gu_flops, "bytes": gu_bytes, "avg_ms": gu_ms}
    if "gate_up" in phase_ms:
        # the same call in the per-phase pass, where every call runs alone in
        # line (in the timed steps a layer with shared experts runs them on a
        # second stream, partly beside this call, whose duration then includes
        # the compute units they hold); its opening event's few microseconds
        # included
        in_ms = phase_ms["gate_up"]
        in_ach = (gu_bytes / (in_ms * 1e-3) / 1e9 if roof["bound"] == "hbm"
                  else gu_flops / (in_ms * 1e-3) / 1e12)
        roof["in_line"] = {"avg_ms": in_ms, "achieved": in_ach, "frac": in_ach / roof["peak"]}
    if cfg.n_shared and layer.overlap_shared:
        roof["timed_beside"] = ("the shared experts' launches on a second stream (from the start "
                                "of the call; tiled ones on part of the compute units), so the "
                                "timed duration includes the compute units they hold; in_line "
                                "is the call alone")

    # algorithmic HBM bytes of the memory-bound phases (per call) and the rate
    # the phase achieved, against the 8 TB/s peak
    rows_moved = R_kept if args.gather == "copy" else 0  # x_perm written and read back
    phase_bytes = {
        "route": T * d * esz + E * d * esz + T * E * 4 + T * k * 8,
        "permute": T * k * 4 + (E + 1) * 4 + 2 * T * k * 4 + 2 * rows_moved * d * esz,
        "combine": (R_kept + T + (T if cfg.n_shared else 0)) * d * esz + T * k * 8,
        "stats": T * E * 4,
    }
    phase_gbs = {name: phase_bytes[name] / (phase_ms[name] * 1e-3) / 1e9
                 for name in phase_bytes if phase_ms.get(name, 0) > 0}

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
        "step_ms": {"median": float(np.median(step_ms)), "p10": float(np.percentile(step_ms, 10)),
                    "p90": float(np.percentile(step_ms, 90))},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded normal inputs and random-init weights of the workload's shape)",
        "config": {"workload": cfg.name, "T": T, "d": d, "E": E, "k": k, "h": h,
                   "n_shared": cfg.n_shared, "h_shared": cfg.h_shared, "cf": cfg.cf,
                   "gather": args.gather, "parallelism": "none (1 GPU)",
                   "shared_overlap": bool(cfg.n_shared and layer.overlap_shared),
                   **({"balance": balance} if balance else {}),
                   **({"variant": {k_: v_ for k_, v_ in variant[1].items()
                                   if k_ in ("k_max", "logit_offset", "n_zero", "n_copy",
                                             "n_const")} | {"kind": variant[0]}}
                      if variant else {})},
        "roofline": roof,
        "measured_ceilings": ceil,
        "expert_gemm_mfma_util": expert_flops / (expert_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "layer_tflops": flops / (ms * 1e-3) / 1e12,
        "layer_hbm_gbs": bytes_ / (ms * 1e-3) / 1e9,
        "phase_ms": phase_ms,
        "phase_ms_source": "a separate pass of the same steps with a HIP event after every library "
                           "call (outside the timed region)",
        "phase_hbm_gbs": phase_gbs,
        "host_enqueue_ms_per_step": host_ms,
        "routing": {"kept_pairs": R_kept, "dropped_pairs": used_slots - bypass_pairs - R_kept,
                    "touched_experts": touched, "max_rows": int(kept.max()),
                    "min_rows": int(kept.min()), "max_demand": int(counts[:E_ffn].max()),
                    **({"experts_per_token": used_slots / T,
                        "empty_slots": T * layer.k - used_slots} if args.variant == "relu"
                       else {}),
                    **({"bypass_pairs": bypass_pairs} if args.variant == "bypass" else {})},
    }
    return out, inp, variant


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.backward:
        return main_backward(args)

    import torch

    from moe_inputs import WORKLOADS

    cfg = WORKLOADS[args.workload]
    out, inp, variant = measure_forward(args, cfg)
    torch.cuda.empty_cache()
    # The other large workloads, each timed the same way (same K and W, inputs
    # resident in HBM before its timed region), one after the other in this
    # process; the headline value above stays that of --workload.  The CPU
    # baseline runs after them, so that no workload's warmup follows the
    # seconds the device would idle during it.
    extra = [] if (args.no_extra_workloads or args.variant or args.balance or
                   args.workload != "mixtral_bf16") else list(EXTRA_WORKLOADS)
    if extra:
        out["workloads"] = {}
        keep = ("value", "unit", "ms_per_step", "step_ms", "dtype", "config", "roofline",
                "expert_gemm_mfma_util", "layer_tflops", "layer_hbm_gbs", "phase_ms",
                "phase_hbm_gbs", "routing")
        for name in extra:
            o, i_, _ = measure_forward(args, WORKLOADS[name], ceil=out["measured_ceilings"],
                                       extra=True)
            del i_
            torch.cuda.empty_cache()
            out["workloads"][name] = {key: o[key] for key in keep}
            print(f"# {name}: {o['value']:.4g} tokens/s, {o['ms_per_step']:.3f} ms per step, "
                  f"roofline frac {o['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        n_tok = args.cpu_tokens or {"tiny_f32": 64, "mixtral_bf16": 4096,
                                    "finegrained_shared_bf16": 8192,
                                    "capacity_balance_bf16": 8192, "decode_bf16": 64}[cfg.name]
        out["cpu_baseline"] = cpu_baseline(inp, cfg, n_tok, variant=variant)
    del inp
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
