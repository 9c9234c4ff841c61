"""Turn rocprofv3 output into the short summaries kept under profiles/.

  python -m moe_lora_layer_amd.profiling trace  <csv_dir> <out.md> <title> <command...>
  python -m moe_lora_layer_amd.profiling traffic <out.json> <out.md> <kernel-substring>
        <fetch_dir> <write_dir> <copy_fetch_dir> <copy_write_dir> <copy_bytes> <algo_bytes>
  python -m moe_lora_layer_amd.profiling kernels <out.md> <title> <trace_dir> <fetch_dir>
        <write_dir> <copy_fetch_dir> <copy_write_dir> <copy_bytes> <command...>
  python -m moe_lora_layer_amd.profiling counters <out.md> <title> <kernel-substring>
        <pmc_dir>... -- <command...>

`trace` reads <csv_dir>/run_kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv).  `kernels` tabulates, for every kernel of the library,
the scaled FETCH_SIZE + WRITE_SIZE bytes per dispatch over its average
duration in the kernel trace of the same workload (achieved HBM GB/s).
`counters` averages raw SQ/GRBM counters per dispatch of one kernel and
derives the engine clock and the MFMA-busy fraction from them.  `traffic` reads per-dispatch FETCH_SIZE and WRITE_SIZE
(KiB) of the named kernel from two --pmc runs, and the same counters for a
device copy of known size; the counters are scaled by known/counted of the
copy.  The traffic record carries a digest of the kernel sources: bench.py
reports the traffic only while the sources are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
PROFILES = os.path.join(ROOT, "profiles")


def source_digest() -> str:
    """sha256 over the HIP sources and the public header (kernel identity)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(_HERE, "csrc", "*"))) + [os.path.join(ROOT, "include", "moelora.h")]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def load_traffic(workload: str, kernel: str):
    """Bytes per launch of `kernel` at `workload` from profiles/, or None when the
    record is missing or was taken on different kernel sources."""
    path = os.path.join(PROFILES, f"{workload}_{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("traffic_bytes")


def _pmc(dirname: str):
    rows = list(csv.DictReader(open(os.path.join(dirname, "run_counter_collection.csv"))))
    out = {}
    for r in rows:
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(d: dict, sub: str):
    keys = [k for k in d if sub in k]
    if len(keys) != 1:
        raise SystemExit(f"kernel '{sub}' matches {len(keys)} names: {keys}")
    return keys[0], d[keys[0]]


def trace(csv_dir: str, out_md: str, title: str, command: str) -> None:
    rows = list(csv.DictReader(open(os.path.join(csv_dir, "run_kernel_stats.csv"))))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:120]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic(out_json: str, out_md: str, kernel: str, fetch_dir: str, write_dir: str,
            copy_fetch_dir: str, copy_write_dir: str, copy_bytes: float, algo_bytes: float,
            commands: list[str]) -> None:
    name, fetch = _pick(_pmc(fetch_dir), kernel)
    _, write = _pick(_pmc(write_dir), kernel)
    _, cf = _pick(_pmc(copy_fetch_dir), "copyBuffer")
    _, cw = _pick(_pmc(copy_write_dir), "copyBuffer")
    fscale = copy_bytes / (statistics.mean(cf) * 1024.0)
    wscale = copy_bytes / (statistics.mean(cw) * 1024.0)
    fb = statistics.mean(fetch) * 1024.0 * fscale
    wb = statistics.mean(write) * 1024.0 * wscale
    rec = {"kernel": name, "dispatches": len(fetch), "fetch_kib_per_dispatch": statistics.mean(fetch),
           "write_kib_per_dispatch": statistics.mean(write), "copy_bytes": copy_bytes,
           "copy_fetch_kib": statistics.mean(cf), "copy_write_kib": statistics.mean(cw),
           "fetch_scale": fscale, "write_scale": wscale, "traffic_bytes": fb + wb,
           "algorithmic_bytes": algo_bytes, "traffic_over_algorithmic": (fb + wb) / algo_bytes,
           "source_sha256": source_digest(), "commands": commands}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic of `{name[:100]}`", "",
             "Commands (from the repository root on one MI355X):", "", "```", *commands, "```", "",
             f"- dispatches averaged: {len(fetch)}",
             f"- FETCH_SIZE per dispatch: {statistics.mean(fetch):.6g} KiB; WRITE_SIZE: {statistics.mean(write):.6g} KiB",
             f"- copy calibration ({copy_bytes / 2**30:.3g} GiB device copy): FETCH_SIZE "
             f"{statistics.mean(cf):.6g} KiB -> scale {fscale:.4g}; WRITE_SIZE {statistics.mean(cw):.6g} KiB "
             f"-> scale {wscale:.4g}",
             f"- scaled traffic per launch: {fb / 1e9:.4g} GB read + {wb / 1e9:.4g} GB written = {(fb + wb) / 1e9:.4g} GB",
             f"- algorithmic bytes per launch: {algo_bytes / 1e9:.4g} GB (ratio {(fb + wb) / algo_bytes:.3f})",
             f"- kernel sources sha256: {rec['source_sha256']}"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _calibration(copy_fetch_dir: str, copy_write_dir: str, copy_bytes: float):
    _, cf = _pick(_pmc(copy_fetch_dir), "copyBuffer")
    _, cw = _pick(_pmc(copy_write_dir), "copyBuffer")
    return (copy_bytes / (statistics.mean(cf) * 1024.0), copy_bytes / (statistics.mean(cw) * 1024.0),
            statistics.mean(cf), statistics.mean(cw))


def kernels(out_md: str, title: str, trace_dir: str, fetch_dir: str, write_dir: str,
            copy_fetch_dir: str, copy_write_dir: str, copy_bytes: float, command: str) -> None:
    stats = {r["Name"]: r for r in csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv")))}
    fetch, write = _pmc(fetch_dir), _pmc(write_dir)
    fscale, wscale, cf, cw = _calibration(copy_fetch_dir, copy_write_dir, copy_bytes)
    lines = [f"# {title}", "", "Commands (from the repository root on one MI355X; the kernel trace "
             "of the same workload gives the durations):", "", "```", command, "```", "",
             f"Counter scale from a {copy_bytes / 2**30:.3g} GiB device copy: FETCH_SIZE x{fscale:.4g}, "
             f"WRITE_SIZE x{wscale:.4g} (the copy reads {cf:.6g} KiB and writes {cw:.6g} KiB as counted).",
             "", "| kernel | dispatches | average us | read MB | written MB | achieved GB/s | of 8 TB/s |",
             "|---|---|---|---|---|---|---|"]
    for name in sorted(fetch, key=lambda n: -float(stats[n]["TotalDurationNs"]) if n in stats else 0):
        if "moelora::" not in name or name not in write or name not in stats:
            continue
        rb = statistics.mean(fetch[name]) * 1024.0 * fscale
        wb = statistics.mean(write[name]) * 1024.0 * wscale
        us = float(stats[name]["AverageNs"]) / 1e3
        gbs = (rb + wb) / (us * 1e-6) / 1e9
        lines.append(f"| `{name[:90]}` | {len(fetch[name])} | {us:.2f} | {rb / 1e6:.1f} | "
                     f"{wb / 1e6:.1f} | {gbs:.0f} | {gbs / 8000.0:.2f} |")
    lines += ["", f"- kernel sources sha256: {source_digest()}"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters(out_md: str, title: str, kernel: str, pmc_dirs: list[str], command: str) -> None:
    vals, dur = {}, []
    for d in pmc_dirs:
        rows = [r for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv")))
                if kernel in r["Kernel_Name"]]
        names = {r["Kernel_Name"] for r in rows}
        if len(names) != 1:
            raise SystemExit(f"kernel '{kernel}' matches {len(names)} names in {d}")
        name = names.pop()
        for r in rows:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    avg = {k: statistics.mean(v) for k, v in vals.items()}
    us = statistics.mean(dur) / 1e3
    lines = [f"# {title}", "", f"Kernel `{name[:100]}`; commands (from the repository root on one "
             "MI355X, one counter group per run):", "", "```", command, "```", "",
             "| counter | mean per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:.6g} |" for k, v in sorted(avg.items())]
    lines += ["", f"- mean dispatch duration under counter collection: {us:.1f} us"]
    if "GRBM_GUI_ACTIVE" in avg:
        clk = avg["GRBM_GUI_ACTIVE"] / 8 / (us * 1e-6)  # GRBM_GUI_ACTIVE sums the 8 XCDs
        lines.append(f"- engine clock: GRBM_GUI_ACTIVE / 8 XCDs / duration = {clk / 1e9:.2f} GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            simd_cycles = avg["GRBM_GUI_ACTIVE"] / 8 * 1024  # 256 CUs x 4 SIMDs
            lines.append(f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles) = "
                         f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}")
    if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in avg and "GRBM_GUI_ACTIVE" in avg:
        # the counter counts 64-byte units of LDS reads, summed over the CUs
        per_cu_clk = avg["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64 / 256 / (avg["GRBM_GUI_ACTIVE"] / 8)
        lines.append(f"- LDS reads: 64 x SQ_INSTS_LDS_LOAD_BANDWIDTH = "
                     f"{avg['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / 1e9:.1f} GB per dispatch, "
                     f"{per_cu_clk:.0f} bytes per clock per CU")
    if "SQ_WAVE_CYCLES" in avg:
        for k, what in (("SQ_WAIT_ANY", "at s_waitcnt"), ("SQ_WAIT_INST_ANY", "for an instruction to issue")):
            if k in avg:
                lines.append(f"- waves waiting {what}: {k} / SQ_WAVE_CYCLES = "
                             f"{avg[k] / avg['SQ_WAVE_CYCLES']:.2f}")
    if "TCC_EA0_RDREQ_LEVEL_sum" in avg and avg.get("TCC_EA0_RDREQ_sum", 0) > 0:
        # reads in flight summed over cycles, over reads: the mean L2-miss read latency
        lines.append(f"- L2-miss read latency: TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum = "
                     f"{avg['TCC_EA0_RDREQ_LEVEL_sum'] / avg['TCC_EA0_RDREQ_sum']:.0f} cycles")
    if "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum" in avg and "GRBM_GUI_ACTIVE" in avg:
        lines.append(f"- DRAM credit stalls: TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum / cycles = "
                     f"{avg['TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum'] / (avg['GRBM_GUI_ACTIVE'] / 8):.3f} "
                     f"(summed over the L2 channels)")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
        fl = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        lines.append(f"- bf16 MFMA work issued: 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 = {fl / 1e12:.3f} TFLOP "
                     f"per dispatch (padding rows included)")
    lines.append(f"- kernel sources sha256: {source_digest()}")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "kernels":
        a = sys.argv
        kernels(a[2], a[3], a[4], a[5], a[6], a[7], a[8], float(a[9]), " ".join(a[10:]))
    elif sys.argv[1] == "counters":
        a = sys.argv
        sep = a.index("--")
        counters(a[2], a[3], a[4], a[5:sep], " ".join(a[sep + 1:]))
    elif sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]))
    elif sys.argv[1] == "traffic":
        a = sys.argv
        traffic(a[2], a[3], a[4], a[5], a[6], a[7], a[8], float(a[9]), float(a[10]), a[11:])
    else:
        raise SystemExit(__doc__)
