"""Offline tuner of the tile plan, and the table of tuned plans.

The vLLM blog page "Multi-LoRA" (section "Kernel configuration tuning for
Amazon SageMaker AI and Amazon Bedrock") tunes the MoE-LoRA kernels' block
sizes and split-K per shape offline and lets users load their own tuned
configurations.  Here the tunable choices are the fields of `moelora_plan`
(include/moelora.h): M-tile rows and form of the base GEMMs, LoRA tile rows,
the two split-K counts and whether the expand runs in the GEMM epilogue.

`tune_layer` / `tune_dense` run the layer (or the dense projection) on the GPU
through the C ABI for one set of dimensions and search the plan one field at a
time from the library's automatic plan, keeping a change only when it is
faster; every candidate's output must match the automatic plan's output within
the layer's tolerance, otherwise the candidate is reported and skipped.  A
table is a JSON file of entries {"kind", "dims", "plan", "us", "auto_us"};
`plan_for` returns the tuned plan of matching dims, or None.

    python -m moe_lora_layer_amd.tune --workload decode_h4096 --out plans.json

The packaged table `plans/mi355x.json` (if present) is what `packaged_plan`
reads.
"""
import argparse
import ctypes
import json
import os
import statistics
import sys

import numpy as np
import torch

from . import ops, synth

TABLE_VERSION = 1
PACKAGED_TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "plans", "mi355x.json")
TOL = {ops.MOELORA_BF16: 1e-2, ops.MOELORA_F32: 1e-4}

LAYER_KEYS = ["tokens", "hidden", "intermediate", "experts", "top_k", "adapters", "rank", "dtype",
              "flags"]
DENSE_KEYS = ["tokens", "in_features", "out_features", "adapters", "rank", "dtype", "flags"]

# values tried per field (gemm_rows and gemm_form move together)
GEMM_SHAPES = [(32, 1), (64, 1), (128, 1), (128, 2), (128, 3), (256, 2)]
SPLITS = [1, 2, 3, 4, 5, 6, 8, 12, 16]


def _key(d) -> tuple:
    if isinstance(d, ops.DenseDims):
        return ("dense",) + tuple(int(getattr(d, k)) for k in DENSE_KEYS)
    return ("layer",) + tuple(int(getattr(d, k)) for k in LAYER_KEYS)


def _entry_key(e: dict) -> tuple:
    keys = DENSE_KEYS if e["kind"] == "dense" else LAYER_KEYS
    return (e["kind"],) + tuple(int(e["dims"][k]) for k in keys)


def load_table(path: str) -> list:
    with open(path) as f:
        t = json.load(f)
    if t.get("version") != TABLE_VERSION:
        raise ValueError(f"{path}: plan table version {t.get('version')}, expected {TABLE_VERSION}")
    return t["entries"]


def save_table(path: str, entries: list):
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump({"version": TABLE_VERSION, "device": "gfx950", "entries": entries}, f, indent=1)
        f.write("\n")


def merge(entries: list, new: list) -> list:
    """entries with every entry of new replacing the one of the same dims."""
    keys = {_entry_key(e) for e in new}
    return [e for e in entries if _entry_key(e) not in keys] + list(new)


def plan_for(d, entries) -> dict | None:
    """The tuned plan of dims d (the plan field of d is ignored), or None."""
    k = _key(d)
    for e in entries:
        if _entry_key(e) == k:
            return dict(e["plan"])
    return None


def packaged_plan(d) -> dict | None:
    """The plan the packaged table holds for d, or None (no table or no entry)."""
    if not os.path.exists(PACKAGED_TABLE):
        return None
    return plan_for(d, load_table(PACKAGED_TABLE))


def with_packaged_plan(d):
    """(dims, source): d with the packaged table's plan for its dims, or d
    unchanged (the library's automatic plan) when the table has none."""
    plan = packaged_plan(d)
    if plan is None:
        return d, "automatic"
    return _with_plan(d, plan), "tuned table"


def _with_plan(d, plan: dict):
    c = type(d).from_buffer_copy(d)
    c.plan = ops.make_plan(plan)
    return c


def _valid(d, plan: dict) -> bool:
    c = _with_plan(d, plan)
    n = ctypes.c_size_t()
    lib = ops.library()
    f = lib.moelora_dense_workspace_size if isinstance(d, ops.DenseDims) else \
        lib.moelora_forward_workspace_size
    return f(ctypes.byref(c), ctypes.byref(n)) == 0


def _to_dev(a: np.ndarray, dev) -> torch.Tensor:
    """A host array on dev (bf16 arrays are stored as their uint16 bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _time_us(fn, steps: int, repeats: int = 3) -> float:
    fn()
    torch.cuda.synchronize()
    runs = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) * 1e3 / steps)
    return statistics.median(runs)


def _warm(fn, seconds: float):
    """Run fn for about `seconds` first, so that the clocks have settled."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    while True:
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        if e0.elapsed_time(e1) > seconds * 1e3:
            return


def _search(d, run, fields: list, steps: int, rounds: int, log):
    """Coordinate search from the automatic plan.  run(dims) -> output tensor.
    The winner is re-timed against the automatic plan in alternation and kept
    only if it is still faster by more than 3% (run-to-run noise of a step is
    about 1-2%)."""
    auto = (ops.dense_forward_plan if isinstance(d, ops.DenseDims) else ops.forward_plan)(d)
    auto_dims = _with_plan(d, auto)
    ref = run(auto_dims).float()
    _warm(lambda: run(auto_dims), 1.0)
    scale = max(float(ref.abs().max()), 1e-30)
    tol = TOL[d.dtype]
    cache = {}

    def cost(plan: dict) -> float | None:
        k = tuple(sorted(plan.items()))
        if k in cache:
            return cache[k]
        c = _with_plan(d, plan)
        # the library may resolve a requested plan to the same effective one
        eff = (ops.dense_forward_plan if isinstance(d, ops.DenseDims) else ops.forward_plan)(c)
        ek = ("eff",) + tuple(sorted(eff.items()))
        if ek in cache:
            cache[k] = cache[ek]
            return cache[k]
        try:
            got = run(c)
        except RuntimeError as ex:  # e.g. a grid past the launch limits
            log(f"  plan {plan}: {ex} (skipped)")
            cache[k] = cache[ek] = None
            return None
        err = float((got.float() - ref).abs().max()) / scale
        if not err <= tol:
            log(f"  plan {plan}: output differs from the automatic plan by {err:.3e} (skipped)")
            cache[k] = cache[ek] = None
            return None
        us = _time_us(lambda: run(c), steps)
        log(f"  plan {eff}: {us:.1f} us")
        cache[k] = cache[ek] = us
        return us

    best = dict(auto)
    auto_us = best_us = cost(best)
    for _ in range(rounds):
        improved = False
        for field in fields:
            if field == "gemm":
                options = [{"gemm_rows": r, "gemm_form": f} for r, f in GEMM_SHAPES]
            elif field == "lora_rows":
                options = [{"lora_rows": v} for v in (16, 64)]
            elif field == "fuse":
                options = [{"fuse": v} for v in (1, 2, 3)]
            elif field == "order":
                options = [{"order": v} for v in (1, 2, 3, 4, 5)]
            else:
                options = [{field: v} for v in SPLITS]
            for opt in options:
                cand = dict(best, **opt)
                if cand == best or not _valid(d, cand):
                    continue
                us = cost(cand)
                if us is not None and us < best_us * 0.99:
                    best, best_us, improved = cand, us, True
        if not improved:
            break
    final = (ops.dense_forward_plan if isinstance(d, ops.DenseDims) else ops.forward_plan)(
        _with_plan(d, best))
    if final != auto:
        best_dims = _with_plan(d, final)
        ta, tb = [], []
        for _ in range(5):
            ta.append(_time_us(lambda: run(auto_dims), steps, 1))
            tb.append(_time_us(lambda: run(best_dims), steps, 1))
        auto_us, best_us = statistics.median(ta), statistics.median(tb)
        log(f"  alternating re-time: automatic {auto_us:.1f} us, tuned {best_us:.1f} us")
        if not best_us < auto_us * 0.97:
            final, best_us = auto, auto_us
    return final, best_us, auto_us


def tune_layer(cfg, steps: int = 10, rounds: int = 2, log=print) -> dict:
    """Tune the plan of one layer workload (synth.LayerConfig) on cuda:0."""
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(cfg)
    names = ["x", "w_gate_up", "w_down", "a_gate_up", "b_gate_up", "a_down", "b_down"]
    t = {n: _to_dev(inp[n], dev) for n in names}
    logits = _to_dev(inp["logits"], dev)
    aids = _to_dev(inp["adapter_ids"], dev)
    d = ops.dims_for(cfg)
    _, w, ss, off, _ = ops.align(d, logits, aids)
    ws = {}

    def run(c):
        n = ops.forward_workspace_size(c)
        if n not in ws:
            ws.clear()
            ws[n] = ops.workspace(n, dev)
        return ops.forward(c, t["x"], t["w_gate_up"], t["w_down"], t["a_gate_up"],
                           t["b_gate_up"], t["a_down"], t["b_down"], w, ss, off,
                           workspace_buf=ws[n])

    log(f"tuning {cfg.name}")
    plan, us, auto_us = _search(d, run, ["gemm", "lora_rows", "ksplit_gate_up", "ksplit_down",
                                         "fuse", "order"], steps, rounds, log)
    return {"kind": "layer", "name": cfg.name, "dims": {k: int(getattr(d, k)) for k in LAYER_KEYS},
            "plan": plan, "us": round(us, 2), "auto_us": round(auto_us, 2)}


def tune_dense(cfg, steps: int = 10, rounds: int = 2, log=print) -> dict:
    """Tune the plan of one dense projection workload (synth.DenseConfig) on cuda:0."""
    dev = torch.device("cuda:0")
    inp = synth.make_dense_inputs(cfg)
    t = {n: _to_dev(inp[n], dev) for n in ["x", "w", "a", "b", "adapter_ids"]}
    d = ops.make_dense_dims(cfg.tokens, cfg.in_features, cfg.out_features, cfg.adapters, cfg.rank,
                            cfg.dtype)
    ws = {}

    def run(c):
        n = ops.dense_workspace_size(c)
        if n not in ws:
            ws.clear()
            ws[n] = ops.workspace(n, dev)
        out, _ = ops.dense_forward(c, t["x"], t["w"], t["a"], t["b"], t["adapter_ids"],
                                   workspace_buf=ws[n])
        return out

    log(f"tuning {cfg.name}")
    plan, us, auto_us = _search(d, run, ["gemm", "lora_rows", "ksplit_down", "fuse", "order"], steps,
                                rounds, log)
    return {"kind": "dense", "name": cfg.name, "dims": {k: int(getattr(d, k)) for k in DENSE_KEYS},
            "plan": plan, "us": round(us, 2), "auto_us": round(auto_us, 2)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", action="append", required=True,
                    help="a layer workload (synth.WORKLOADS) or a dense one (synth.DENSE_WORKLOADS)")
    ap.add_argument("--out", required=True, help="plan table to write (entries merged into it)")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--rounds", type=int, default=2)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("tune: no GPU", file=sys.stderr)
        return 2
    log = lambda s: print(s, file=sys.stderr, flush=True)  # noqa: E731
    new = []
    for w in args.workload:
        if w in synth.WORKLOADS:
            new.append(tune_layer(synth.WORKLOADS[w], args.steps, args.rounds, log))
        elif w in synth.DENSE_WORKLOADS:
            new.append(tune_dense(synth.DENSE_WORKLOADS[w], args.steps, args.rounds, log))
        else:
            raise SystemExit(f"unknown workload {w}")
        log(f"{w}: {new[-1]['plan']} {new[-1]['us']} us (automatic {new[-1]['auto_us']} us)")
    old = load_table(args.out) if os.path.exists(args.out) else []
    save_table(args.out, merge(old, new))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
