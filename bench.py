#!/usr/bin/env python3
"""Benchmark of the fused MoE multi-LoRA layer on one MI355X.

A step is one pass of the whole layer over one batch of synthetic input:
moelora_align (routing + bucketed permutation) followed by moelora_forward
(base grouped GEMMs, LoRA shrink/expand, SiLU-mul, top-k combination), with
every input already resident in HBM.  Prints one JSON line on stdout; details
go to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: prefill_h4096 (4096 tokens as 8 requests of 512, h 4096,
I 11008, 16 experts top-2 with a per-expert logit bias, 8 adapters rank 32,
bf16), the largest configuration, where the base grouped GEMMs are bound by the
matrix cores.  Kernel durations come from HIP events that the
library records on the launch stream around its kernels
(moelora_forward_profiled): an untimed pass records every stage boundary for
the per-stage breakdown; the timed K steps record only the two events around
the dominant kernel, whose mean duration gives the roofline figure.  Also
untimed: the per-step latency (p10/p50/p90 of event-bracketed align + forward),
warm and cold (a 1 GiB read before each step evicts the MALL and the L2s).
The CPU baseline times the plain C oracle on the host's cores over a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer tokens/s; shrink/expand HBM GB/s and GEMM MFMA % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA bf16; fp32 (vector/MFMA)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it (model name, with the family /
    model / stepping numbers, which identify the core generation when a
    virtualised host reports a generic name), or "unknown"."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break  # first processor only
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if ids else name


def stage_work(cfg, offsets, fusion):
    """Algorithmic bytes and flops per stage of one forward launch, from the active
    experts and (expert, adapter) buckets of this batch.  A LoRA expand fused into
    its GEMM's epilogue moves into that GEMM's figures (no G round trip) and its
    own stage is empty."""
    import numpy as np
    T, h, I, E, k, L, r = (cfg.tokens, cfg.hidden, cfg.intermediate, cfg.experts, cfg.top_k,
                           cfg.adapters, cfg.rank)
    S = T * k
    b = 2 if cfg.dtype == "bf16" else 4
    counts = np.diff(offsets)
    P = int(np.count_nonzero(counts))                            # active buckets
    Eact = int(np.count_nonzero(counts.reshape(E, -1).sum(axis=1)))  # active experts
    w = {
        "prep": (S * 4 * 3 + (E * L + 1) * 4, 0),
        "zero": (2 * S * r * 4, 0),
        "gemm_gate_up": (Eact * 2 * I * h * b + S * h * b + S * 2 * I * 4, 2 * S * h * 2 * I),
        "shrink_gate_up": (P * h * r * b + S * h * b + S * r * 4, 2 * S * h * r),
        "expand_gate_up": (P * r * 2 * I * b + S * r * 4 + S * 2 * I * 4 + S * I * b, 2 * S * r * 2 * I),
        "gemm_down": (Eact * h * I * b + S * I * b + S * h * 4, 2 * S * I * h),
        "shrink_down": (P * I * r * b + S * I * b + S * r * 4, 2 * S * I * r),
        "expand_down": (P * r * h * b + S * r * 4 + 2 * S * h * 4, 2 * S * r * h),
        "combine": (S * h * 4 + T * h * b + S * 8, 2 * S * h),
    }
    if fusion["gate_up"]:
        w["gemm_gate_up"] = (Eact * 2 * I * h * b + S * h * b + P * r * 2 * I * b + S * r * 4 + S * I * b,
                             2 * S * h * 2 * I + 2 * S * r * 2 * I)
        w["expand_gate_up"] = (0, 0)
    if fusion.get("down_shrink"):
        # the down shrink runs in the gate_up epilogue: its A_dn reads and Z2
        # writes move there; ACT is not read again
        gb, gf = w["gemm_gate_up"]
        w["gemm_gate_up"] = (gb + P * I * r * b + S * r * 4, gf + 2 * S * I * r)
        w["shrink_down"] = (0, 0)
    if fusion["down"]:
        w["gemm_down"] = (Eact * h * I * b + S * I * b + P * r * h * b + S * r * 4 + S * h * 4,
                          2 * S * I * h + 2 * S * r * h)
        w["expand_down"] = (0, 0)
    return w, Eact, P


def run_dense(args, cfg) -> int:
    """The dense multi-LoRA projection (moelora_dense_forward): a step is one
    call over the batch.  It has no per-stage events, so its roofline line is
    the whole call against the bytes it must move (the weight, the active
    adapters, x and out, plus the fp32 partial output round trip of this
    decomposition)."""
    import numpy as np
    import torch
    from moe_lora_layer_amd import ops, synth

    dev = torch.device("cuda:0")
    inp = synth.make_dense_inputs(cfg)
    t = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                   else torch.from_numpy(a)).to(dev)
    if args.in_out:
        x, w = t(inp["x"]), t(np.ascontiguousarray(inp["w"].T))
        a, b = (t(np.ascontiguousarray(np.swapaxes(inp[n], 1, 2))) for n in ("a", "b"))
    else:
        x, w, a, b = t(inp["x"]), t(inp["w"]), t(inp["a"]), t(inp["b"])
    ad = torch.from_numpy(inp["adapter_ids"]).to(dev)
    from moe_lora_layer_amd import tune
    d = ops.make_dense_dims(cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters, cfg.rank,
                            cfg.dtype, deterministic=args.deterministic, in_out=args.in_out)
    plan_source = "automatic"
    if args.plan == "tuned":
        d, plan_source = tune.with_packaged_plan(d)
    plan = ops.dense_forward_plan(d)
    log(f"[bench] {cfg.name}: plan {plan} ({plan_source})")
    ws = ops.workspace(ops.dense_workspace_size(d), dev)
    out = torch.empty((cfg.tokens, cfg.out_features), dtype=x.dtype, device=dev)
    st = torch.zeros((4,), dtype=torch.int32, device=dev)
    step = lambda: ops.dense_forward(d, x, w, a, b, ad, out=out, workspace_buf=ws, status=st)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    call_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    T, K, N, r = cfg.tokens, cfg.in_features, cfg.out_features, cfg.rank
    bsz = 2 if cfg.dtype == "bf16" else 4
    P = int(np.unique(inp["adapter_ids"]).size)
    by = N * K * bsz + P * r * (K + N) * bsz + T * K * bsz + T * N * bsz + 2 * T * N * 4
    roof = {"bound": "hbm", "achieved": round(by / (call_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s"}
    roof.update(frac=round(roof["achieved"] / roof["peak"], 4), traffic=None, algorithmic_bytes=by,
                kernel="whole dense call", kernel_us=round(call_ms * 1e3, 2))
    value = T * args.steps / elapsed
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(T, args.cpu_tokens)
        sel = np.linspace(0, T - 1, n).round().astype(np.int64)
        reps, tc = 0, time.perf_counter()
        while reps < 200 and (reps == 0 or time.perf_counter() - tc < args.cpu_seconds):
            oracle.dense(inp["x"], inp["w"], inp["a"], inp["b"], inp["adapter_ids"], cfg.dtype,
                         tokens=sel, threads=oracle.max_threads())
            reps += 1
        tcpu = time.perf_counter() - tc
        cpu = {"value": round(reps * n / tcpu, 3), "unit": "tokens/s", "cores": oracle.max_threads(),
               "kind": "oracle", "cpu": cpu_model(), "host_cpus": os.cpu_count(),
               "sample": f"{reps} passes over {n} of {T} tokens, fp64 C oracle, {tcpu:.1f} s wall"}
    log(f"[bench] {cfg.name}: {value:.1f} tokens/s, call {call_ms * 1e3:.1f} us, "
        f"{roof['achieved']:.0f} GB/s")
    rec = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
           "data": "synthetic (seeded normal inputs, random-init weights)",
           "config": {"workload": cfg.name, "tokens": T, "in_features": K, "out_features": N,
                      "adapters": cfg.adapters, "rank": r, "parallelism": "single GPU"},
           "roofline": roof, "cpu_baseline": cpu, "deterministic": args.deterministic,
           "plan": plan, "plan_source": plan_source}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    from moe_lora_layer_amd import synth

    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_h4096",
                    choices=synth.WORKLOAD_ORDER + list(synth.DENSE_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--deterministic", action="store_true",
                    help="MOELORA_FLAG_DETERMINISTIC: ordered split-K partial sums, no atomics")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens in the oracle's timed sample (default 64)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="repeat the oracle's sample for about this long (default 12 s)")
    ap.add_argument("--in-out", action="store_true",
                    help="MOELORA_FLAG_IN_OUT: pass every weight h_in x h_out as the page writes "
                         "it (default: K-contiguous, i.e. transposed)")
    ap.add_argument("--plan", choices=["tuned", "auto"], default="tuned",
                    help="tile plan: the packaged tuned table's entry for the workload when it has "
                         "one (default), or the library's automatic plan")
    args = ap.parse_args()

    if args.gpus != 1:
        log(f"bench.py: --gpus {args.gpus} is not supported: this layer is built and measured on "
            "one GPU only (no collectives); run with --gpus 1")
        return 2
    if args.steps < 1 or args.warmup < 0:
        log("bench.py: --steps must be >= 1 and --warmup >= 0")
        return 2

    import numpy as np
    import torch
    from moe_lora_layer_amd import ops

    if args.workload in synth.DENSE_WORKLOADS:
        return run_dense(args, synth.DENSE_WORKLOADS[args.workload])
    cfg = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = synth.make_inputs(cfg)
    log(f"[bench] {cfg.name}: inputs generated in {time.time() - t0:.1f}s")

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    names = ["w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down"]
    # h_in x h_out weights: the K-contiguous arrays transposed in their last two axes
    W = {n: dev_t(np.ascontiguousarray(np.swapaxes(inp[n], -1, -2)) if args.in_out else inp[n])
         for n in names}
    x = dev_t(inp["x"])
    logits = torch.from_numpy(inp["logits"]).to(dev)
    adapter_ids = torch.from_numpy(inp["adapter_ids"]).to(dev)
    from moe_lora_layer_amd import tune
    d = ops.dims_for(cfg, deterministic=args.deterministic, in_out=args.in_out)
    plan_source = "automatic"
    if args.plan == "tuned":
        d, plan_source = tune.with_packaged_plan(d)
    plan = ops.forward_plan(d)
    log(f"[bench] {cfg.name}: plan {plan} ({plan_source})")
    layer = ops.MoELoRALayer(d, W, dev)
    nst = len(ops.STAGES)

    def new_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
        for e in evs:
            e.record()          # creates the underlying HIP event
        return evs

    def step(evs=None):
        ids, w, ss, off, _ = ops.align(d, logits, adapter_ids, out=layer.routing,
                                       workspace_buf=layer.ws_align, status=layer.status)
        return ops.forward(d, x, *[W[n] for n in names], w, ss, off, topk_ids=ids, out=layer.out,
                           workspace_buf=layer.ws_fwd, stage_events=evs)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(layer.status[0].item()) != 0:
        log("[bench] align reported a bad adapter id")
        return 1

    # per-stage breakdown (untimed pass; every stage boundary recorded)
    events = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = np.array([[events[i][s].elapsed_time(events[i][s + 1]) for s in range(nst)]
                         for i in range(args.steps)])
    mean_ms = stage_ms.mean(axis=0)
    dom_i = int(np.argmax(mean_ms))
    dom = ops.STAGES[dom_i]

    # per-step latency (untimed): warm, and cold with a 1 GiB read before each
    # step (outside its events) that evicts the MALL and the L2s; a read, not a
    # write, so that no dirty line is written back inside the timed step
    def latency(flush):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in evs:
            if flush is not None:
                flush.sum()
            e0.record()
            step()
            e1.record()
        torch.cuda.synchronize()
        us = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
        return {q: round(float(np.percentile(us, p)), 2) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}
    lat_warm = latency(None)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    lat_cold = latency(flush_buf)
    del flush_buf

    # timed region: exactly K steps; events only around the dominant kernel
    dom_events = []
    for _ in range(args.steps):
        evs = [None] * (nst + 1)
        evs[dom_i], evs[dom_i + 1] = new_events()[:2]
        dom_events.append(evs)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(dom_events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # --------------------------------------------------------------------------
    dom_ms = float(np.mean([ev[dom_i].elapsed_time(ev[dom_i + 1]) for ev in dom_events]))

    # the same K steps replayed from a HIP graph of the step (align + forward
    # captured once; no host launch cost per kernel), for context
    try:
        cs = ops.CapturedStep(ops.MoELoRALayer(d, W, dev), x, logits, adapter_ids)
        for _ in range(args.warmup):
            cs.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            cs.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter() - tg
        graph = {"value": round(cfg.tokens * args.steps / tg, 2),
                 "ms_per_step": round(tg * 1e3 / args.steps, 4)}
        del cs
    except Exception as exc:  # reported, not fatal: the eager line above is the measurement
        graph = {"error": str(exc)[:200]}
    log(f"[bench] HIP graph replay: {graph}")

    offsets = layer.routing[3].cpu().numpy()
    fusion = ops.forward_fusion(d)
    work, Eact, P = stage_work(cfg, offsets, fusion)
    ms_per_step = elapsed * 1e3 / args.steps
    value = cfg.tokens * args.steps / elapsed

    stages = {}
    for sname, ms in zip(ops.STAGES, mean_ms):
        by, fl = work[sname]
        if by == 0:  # fused into a GEMM epilogue: only the event gap (or an ordered sum) remains
            stages[sname] = {"us": round(ms * 1e3, 2), "fused": True}
            log(f"[bench] {sname:15s} {ms * 1e3:9.2f} us  (fused into a GEMM epilogue)")
            continue
        stages[sname] = {"us": round(ms * 1e3, 2), "GB/s": round(by / (ms * 1e-3) / 1e9, 1),
                         "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 2)}
        log(f"[bench] {sname:15s} {ms * 1e3:9.2f} us  {stages[sname]['GB/s']:8.1f} GB/s "
            f"({100 * stages[sname]['GB/s'] / HBM_PEAK_GBS:5.1f}% HBM)  "
            f"{stages[sname]['TFLOP/s']:8.2f} TFLOP/s")
    by, fl = work[dom]
    dom_s = dom_ms * 1e-3   # measured in the timed region
    peak_f = MFMA_PEAK_TFLOPS[cfg.dtype]
    if fl / (peak_f * 1e12) > by / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(fl / dom_s / 1e12, 2), "peak": peak_f,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(by / dom_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled by a
    # device-copy calibration), kept under profiles/; None once the kernels changed
    from moe_lora_layer_amd import profiling
    roof["traffic"] = profiling.load_traffic(cfg.name, dom)
    roof["algorithmic_bytes"] = by
    roof["kernel"] = dom
    roof["kernel_us"] = round(dom_s * 1e6, 2)
    # the two base grouped GEMMs together (gate_up and down, each with its fused
    # LoRA expand when fused) against the bf16 matrix-core peak
    gemm_us = (mean_ms[ops.STAGES.index("gemm_gate_up")] + mean_ms[ops.STAGES.index("gemm_down")]) * 1e3
    gemm_fl = work["gemm_gate_up"][1] + work["gemm_down"][1]
    base_fl = 2 * cfg.tokens * cfg.top_k * cfg.hidden * cfg.intermediate * 3
    gemms = {"us": round(gemm_us, 2), "flops": gemm_fl, "TFLOP/s": round(gemm_fl / gemm_us / 1e6, 2),
             "frac": round(gemm_fl / gemm_us / 1e6 / peak_f, 4),
             "us_at_half_peak": round(base_fl / (0.5 * peak_f * 1e12) * 1e6, 2)}
    log(f"[bench] base GEMMs (gate_up + down): {gemms}")
    log(f"[bench] latency per step (us): warm {lat_warm}, cold {lat_cold}")
    log(f"[bench] {cfg.name}: {value:.1f} tokens/s, {ms_per_step:.3f} ms/step, "
        f"sum of stages {mean_ms.sum():.3f} ms, active experts {Eact}, active buckets {P}")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(cfg.tokens, args.cpu_tokens)
        sel = np.linspace(0, cfg.tokens - 1, n).round().astype(np.int64)
        threads = oracle.max_threads()
        # repeat the sample until about args.cpu_seconds of CPU work (at most 200 passes)
        reps, tc = 0, time.perf_counter()
        while reps < 200 and (reps == 0 or time.perf_counter() - tc < args.cpu_seconds):
            ids, wts = oracle.route(inp["logits"], cfg.top_k)
            oracle.align(ids, inp["adapter_ids"], cfg.experts, cfg.adapters)
            oracle.forward(inp, oracle.dims_of(cfg), ids, wts, tokens=sel, threads=threads)
            reps += 1
        tcpu = time.perf_counter() - tc
        cpu = {"value": round(reps * n / tcpu, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "cpu": cpu_model(), "host_cpus": os.cpu_count(),
               "sample": f"{reps} passes over {n} of {cfg.tokens} tokens (routing and permutation of "
                         f"all {cfg.tokens} each pass), fp64 C oracle, {tcpu:.1f} s wall"}
        log(f"[bench] cpu oracle: {reps} x {n} tokens in {tcpu:.1f}s on {threads} threads")

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded normal inputs, random-init weights)",
        "config": {"workload": cfg.name, "tokens": cfg.tokens, "hidden": cfg.hidden,
                   "intermediate": cfg.intermediate, "experts": cfg.experts, "top_k": cfg.top_k,
                   "adapters": cfg.adapters, "rank": cfg.rank, "requests": cfg.requests,
                   "adapter_dist": cfg.adapter_dist, "parallelism": "single GPU"},
        "roofline": roof,
        "value_cold_p50": round(cfg.tokens / (lat_cold["p50"] * 1e-6), 2),
        "graph_replay": graph,
        "latency_us": {"warm": lat_warm, "cold_1GiB_read_flush": lat_cold},
        "gemms": gemms,
        "fusion": fusion,
        "plan": plan,
        "plan_source": plan_source,
        "deterministic": args.deterministic,
        "weights": "h_in x h_out" if args.in_out else "K-contiguous",
        "cpu_baseline": cpu,
        "stages": stages,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
