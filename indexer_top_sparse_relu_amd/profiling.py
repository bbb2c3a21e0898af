"""Summaries of rocprofv3 output for the kernels of the sparse attention path.

Two jobs, both run on the output directories of rocprofv3 runs of bench.py:

  stats   — `rocprofv3 --kernel-trace --stats` kernel table -> markdown summary
            (calls, average, min, max per kernel of the path).
  traffic — two `rocprofv3 --pmc` runs (FETCH_SIZE, then WRITE_SIZE) of
            `bench.py --calibrate-copy` -> HBM bytes per launch of each path
            kernel, calibrated against the copy kernel bench.py runs first
            (it reads and writes a known number of bytes), written as JSON
            (keyed by workload and stage, with the hash of the kernel source
            the counters were taken on) and as a markdown summary.

Usage (from the repository root):
  python -m indexer_top_sparse_relu_amd.profiling stats <dir> --workload W --command "..." --out F.md
  python -m indexer_top_sparse_relu_amd.profiling traffic <fetch_dir> <write_dir> --workload W \
         --copy-bytes N --command-fetch "..." --command-write "..." --json F.json --out F.md
  python -m indexer_top_sparse_relu_amd.profiling counters <dir> [<dir> ...] --workload W \
         --command "..." [--command "..."] --out F.md

  counters — `rocprofv3 --pmc` runs with any counters -> per path kernel the
            median value per dispatch of each counter, plus derived figures
            when their counters are present: the shader clock (GRBM_GUI_ACTIVE
            is counted on each of the 8 XCDs), MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES
            over the SIMD-cycles of the dispatch: it counts on each of a CU's 4 SIMDs), and LDS bank-conflict cycles
            per LDS-active cycle.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = {
    "indexer": "indexer_top_sparse_relu_amd/csrc/indexer.hip",
    "topk": "indexer_top_sparse_relu_amd/csrc/topk.hip",
    "attn": "indexer_top_sparse_relu_amd/csrc/attn.hip",
}
STAGE_OF_KERNEL = (("sa::indexer_", "indexer"), ("sa::topk_", "topk"), ("sa::attn_", "attn"))
COPY_KERNEL_MARK = "neg_kernel"


def source_hash(stage: str) -> str:
    """Hash of the sources that define a stage's kernels (used to invalidate stale counters)."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES[stage], "indexer_top_sparse_relu_amd/csrc/sa_device.h"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stage_of(kernel: str):
    for mark, st in STAGE_OF_KERNEL:
        if mark in kernel:
            return st
    return None


def short_name(kernel: str) -> str:
    k = kernel.replace("void ", "")
    cut = k.find("(")
    return k[:cut] if cut > 0 else k


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(dirpath: str):
    """Per path kernel: calls, average, min and max from the stats table, plus the median
    duration from the kernel trace (the average includes the cold first launches)."""
    rows = list(csv.DictReader(open(_one(os.path.join(dirpath, "**", "*kernel_stats.csv")))))
    durs = {}
    trace = glob.glob(os.path.join(dirpath, "**", "*kernel_trace.csv"), recursive=True)
    if trace:
        for r in csv.DictReader(open(sorted(trace)[0])):
            if stage_of(r["Kernel_Name"]) is not None:
                durs.setdefault(r["Kernel_Name"], []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    out = []
    for r in rows:
        name = r["Name"]
        if stage_of(name) is None:
            continue
        d = durs.get(name)
        out.append({"kernel": short_name(name), "calls": int(r["Calls"]),
                    "avg_ms": float(r["AverageNs"]) / 1e6, "median_ms": statistics.median(d) if d else None,
                    "min_ms": float(r["MinNs"]) / 1e6, "max_ms": float(r["MaxNs"]) / 1e6})
    return out


def counter_per_dispatch(dirpath: str, counter: str):
    """{kernel name: [value per dispatch]} of one counter (summed over its instances)."""
    rows = list(csv.DictReader(open(_one(os.path.join(dirpath, "**", "*counter_collection.csv")))))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int):
    """HBM bytes per launch of each path kernel, each counter scaled so that the copy kernel
    reads and writes exactly copy_bytes."""
    f = counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    w = counter_per_dispatch(write_dir, "WRITE_SIZE")

    def copy_value(d):
        vals = [v for k, vs in d.items() if COPY_KERNEL_MARK in k for v in vs
                if v * 1024 > 0.25 * copy_bytes]
        if not vals:
            raise RuntimeError("copy kernel not found in the counter output")
        return statistics.median(vals) * 1024.0

    kf = copy_bytes / copy_value(f)
    kw = copy_bytes / copy_value(w)
    res = {"calibration": {"copy_bytes": copy_bytes, "fetch_factor": kf, "write_factor": kw}, "kernels": {}}
    for name in sorted(set(f) | set(w)):
        st = stage_of(name)
        if st is None:
            continue
        fb = statistics.median(f.get(name, [0.0])) * 1024.0 * kf
        wb = statistics.median(w.get(name, [0.0])) * 1024.0 * kw
        res["kernels"][short_name(name)] = {"stage": st, "fetch_bytes": fb, "write_bytes": wb,
                                            "bytes_per_launch": fb + wb, "dispatches": len(f.get(name, []))}
    return res


N_XCD = 8
N_CU = 256


def counters(dirs):
    """{kernel: {counter: median per dispatch}} over the counter output of several runs, plus
    the median kernel duration of the dispatches (ns) where the output carries timestamps."""
    out = {}
    for d in dirs:
        rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
        per, dur = {}, {}
        for r in rows:
            name = r["Kernel_Name"]
            if stage_of(name) is None:
                continue
            disp = r.get("Dispatch_Id", r.get("Correlation_Id", ""))
            key = (name, r["Counter_Name"], disp)
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                dur[(name, disp)] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        agg = {}
        for (name, cn, disp), v in per.items():
            agg.setdefault((name, cn), []).append(v)
            if cn == "GRBM_GUI_ACTIVE" and dur.get((name, disp), 0) >= 50000:     # 50 us or longer
                agg.setdefault((name, "clock_GHz"), []).append(v / N_XCD / dur[(name, disp)])
        for (name, cn), vs in agg.items():
            out.setdefault(short_name(name), {})[cn] = statistics.median(vs)
    for k, c in out.items():
        g = c.get("GRBM_GUI_ACTIVE")
        if g:
            cyc = g / N_XCD                      # cycles of the dispatch (per XCD)
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                c["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_CU * 4)
            if "SQ_BUSY_CU_CYCLES" in c:
                c["cu_busy_frac"] = c["SQ_BUSY_CU_CYCLES"] / (cyc * N_CU)
        if c.get("SQ_LDS_IDX_ACTIVE"):
            c["lds_bank_conflict_per_active"] = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"]
    return out


def _counters_md(workload, commands, res, stats=None):
    lines = [f"# Counters per dispatch — {workload}", "", "Counter runs (repository root, one MI355X):", "", "```",
             "export TMPDIR=/tmp", *commands, "```", "",
             "Median over the dispatches of each kernel.  Derived: `cycles` = GRBM_GUI_ACTIVE / 8 (it counts on each "
             "of the 8 XCDs); `mfma_busy_frac` = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 256 CUs x 4 SIMDs); `cu_busy_frac` = "
             "SQ_BUSY_CU_CYCLES / (cycles x 256); `lds_bank_conflict_per_active` = SQ_LDS_BANK_CONFLICT / "
             "SQ_LDS_IDX_ACTIVE; `clock_GHz` = cycles over the dispatch's own duration (its timestamps in the counter run).", ""]
    for k, c in res.items():
        lines.append(f"## `{k}`")
        lines.append("")
        lines.append("| counter | value |")
        lines.append("|---|---|")
        for cn in sorted(c):
            v = c[cn]
            lines.append(f"| {cn} | {v:.4g} |" if isinstance(v, float) else f"| {cn} | {v} |")
        lines.append("")
    return "\n".join(lines) + "\n"


def _stats_md(workload, command, stats):
    lines = [f"# Kernel stats — {workload}", "", "Command (repository root, one MI355X):", "", "```",
             "export TMPDIR=/tmp", command, "```", "",
             "| kernel | calls | avg ms | median ms | min ms | max ms |", "|---|---|---|---|---|---|"]
    for s in sorted(stats, key=lambda s: -s["avg_ms"]):
        med = "—" if s["median_ms"] is None else f"{s['median_ms']:.3f}"
        lines.append(f"| `{s['kernel']}` | {s['calls']} | {s['avg_ms']:.3f} | {med} | {s['min_ms']:.3f} | "
                     f"{s['max_ms']:.3f} |")
    return "\n".join(lines) + "\n"


def _traffic_md(workload, cmd_f, cmd_w, res):
    c = res["calibration"]
    lines = [f"# HBM traffic per launch — {workload}", "",
             "Two counter runs (repository root, one MI355X):", "", "```", "export TMPDIR=/tmp", cmd_f, cmd_w, "```", "",
             f"Calibration: bench.py first runs a copy kernel that reads and writes {c['copy_bytes']} bytes; "
             f"FETCH_SIZE is scaled by {c['fetch_factor']:.4f} and WRITE_SIZE by {c['write_factor']:.4f} "
             "so that the copy kernel reads as exactly that many bytes.", "",
             "| kernel | stage | fetch GB | write GB | total GB / launch |", "|---|---|---|---|---|"]
    for k, v in res["kernels"].items():
        lines.append(f"| `{k}` | {v['stage']} | {v['fetch_bytes'] / 1e9:.3f} | {v['write_bytes'] / 1e9:.3f} | "
                     f"{v['bytes_per_launch'] / 1e9:.3f} |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--workload", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--out", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--workload", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    b.add_argument("--json", required=True)
    b.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--workload", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--stats-dir", default=None, help="a --kernel-trace --stats run of the same command (kernel times)")
    c.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "counters":
        res = counters(args.dirs)
        times = None
        if args.stats_dir:
            times = {s["kernel"]: (s["median_ms"] or s["avg_ms"]) for s in kernel_stats(args.stats_dir)}
        with open(args.out, "w") as f:
            f.write(_counters_md(args.workload, args.command, res, times))
        json.dump(res, sys.stdout)
        print()
        return 0
    if args.cmd == "stats":
        st = kernel_stats(args.dir)
        with open(args.out, "w") as f:
            f.write(_stats_md(args.workload, args.command, st))
        json.dump(st, sys.stdout)
        print()
        return 0
    res = traffic(args.fetch_dir, args.write_dir, args.copy_bytes)
    # one entry per stage: the path's kernel of that stage with the most traffic
    by_stage = {}
    for k, v in res["kernels"].items():
        if v["stage"] not in by_stage or v["bytes_per_launch"] > by_stage[v["stage"]]["bytes_per_launch"]:
            by_stage[v["stage"]] = dict(v, kernel=k, source_hash=source_hash(v["stage"]))
    data = {}
    if os.path.exists(args.json):
        with open(args.json) as f:
            data = json.load(f)
    data[args.workload] = {"calibration": res["calibration"], **by_stage}
    with open(args.json, "w") as f:
        json.dump(data, f, indent=1)
    with open(args.out, "w") as f:
        f.write(_traffic_md(args.workload, args.command_fetch, args.command_write, res))
    json.dump(by_stage, sys.stdout)
    print()
    return 0


if __name__ == "__main__":
    sys.exit(main())
