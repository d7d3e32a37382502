"""Summaries of rocprofv3 output for the profiles/ folder.

Two commands, each reading the CSV files a rocprofv3 run writes with
``--output-format csv``:

  python -m exact_attention_state_amd.profsum trace --csv RUN_kernel_trace.csv \\
      --title "..." --command "..." [--only SUBSTR ...] [--min-grid N] [--max-grid N] > profiles/X.md

    Per-kernel table of a ``--kernel-trace`` run: calls, average / minimum /
    maximum duration in microseconds and share of the summed time.  ``--only``
    keeps kernels whose name contains one of the substrings; the grid bounds
    keep launches whose grid size (threads) lies in the range, which tells
    apart launches of one kernel that differ in shape.

  python -m exact_attention_state_amd.profsum traffic --fetch RUN_F_counter_collection.csv \\
      --write RUN_W_counter_collection.csv --copy-fetch COPY_F.csv --copy-write COPY_W.csv \\
      --copy-bytes N [--only SUBSTR ...] [--min-grid N] [--max-grid N] [--command CMD ...] > profiles/traffic_X.json

    HBM bytes per dispatch from ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``
    runs (KiB per dispatch), each scaled by the factor that makes the same
    counter read N bytes for a plain copy kernel of N bytes (the ``copyBuffer``
    dispatches of the copy runs, median).

  python -m exact_attention_state_amd.profsum step-traffic --workload W --fetch ... --write ... \\
      --copy-fetch ... --copy-write ... --copy-bytes N [--command CMD ...] > profiles/traffic_W_step.json

    The same, per kernel class of the block step as bench.py names them
    (qkv, qkv_prep, qkv_gemm, attn, merge, block_rows, invariant_rows), over
    the dispatches of each class's step grid size (the grid launched about as
    often as the attention, which runs in steps only; the refresh's launches
    differ in shape), with the sha256 of the class's sources and its
    algorithmic bytes from bench.py, which reads this record for its
    roofline's traffic while the sources are unchanged.
"""

from __future__ import annotations

import argparse
import csv
import json
import re
import statistics
import sys


def short_name(name: str) -> str:
    """Kernel name without its argument list (library GEMM names cut to 60 characters)."""
    name = name.strip('"')
    if name.startswith("Cijk_"):
        return name[:60] + "..."
    m = re.match(r"(.*?)\(", name)
    base = m.group(1) if m else name
    return base[:90]


def _keep(name: str, only, grid: int, lo, hi) -> bool:
    if only and not any(s in name for s in only):
        return False
    if lo is not None and grid < lo:
        return False
    if hi is not None and grid > hi:
        return False
    return True


def trace_table(path: str, only=None, min_grid=None, max_grid=None):
    """Rows (name, calls, avg_us, min_us, max_us, share) of a kernel-trace CSV, by total time."""
    per = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        if not _keep(name, only, grid, min_grid, max_grid):
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(short_name(name), []).append(us)
    total = sum(sum(v) for v in per.values()) or 1.0
    rows = [(k, len(v), sum(v) / len(v), min(v), max(v), sum(v) / total) for k, v in per.items()]
    return sorted(rows, key=lambda x: -x[1] * x[2])


def trace_markdown(path, title, command, only=None, min_grid=None, max_grid=None) -> str:
    out = [f"# {title}", "", "Command (repo root on the GPU box as $REPO):", "", "```", command, "```", "",
           f"Summarised with `python -m exact_attention_state_amd.profsum trace` from `{path.split('/')[-1]}`"
           + (f", kernels matching {', '.join(only)}" if only else "")
           + (f", grid {min_grid or 0}..{max_grid or 'any'} threads" if (min_grid or max_grid) else "") + ".", "",
           "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for k, n, avg, mn, mx, sh in trace_table(path, only, min_grid, max_grid):
        out.append(f"| `{k}` | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {100 * sh:.1f}% |")
    return "\n".join(out) + "\n"


def _counter(path, only=None, min_grid=None, max_grid=None):
    per = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        if not _keep(name, only, grid, min_grid, max_grid):
            continue
        per.setdefault(short_name(name), []).append(float(r["Counter_Value"]))
    return per


def copy_factor(path: str, n_bytes: int) -> float:
    """n_bytes / (the counter's median KiB for copyBuffer dispatches x 1024)."""
    v = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if "copyBuffer" in r["Kernel_Name"]]
    if not v:
        raise SystemExit(f"{path}: no copyBuffer dispatch")
    return n_bytes / (statistics.median(v) * 1024)


def traffic(fetch, write, copy_fetch, copy_write, copy_bytes, only=None, min_grid=None, max_grid=None) -> dict:
    ff, wf = copy_factor(copy_fetch, copy_bytes), copy_factor(copy_write, copy_bytes)
    f, w = _counter(fetch, only, min_grid, max_grid), _counter(write, only, min_grid, max_grid)
    res = {"calibration": {"copy_bytes": copy_bytes, "fetch_factor": ff, "write_factor": wf}, "kernels": {}}
    for k in sorted(set(f) | set(w)):
        e = {}
        if k in f:
            e["fetch_bytes_median"] = statistics.median(f[k]) * 1024 * ff
            e["dispatches"] = len(f[k])
        if k in w:
            e["write_bytes_median"] = statistics.median(w[k]) * 1024 * wf
        res["kernels"][k] = e
    return res


# Kernel classes of the block step (bench.py's names), by substring of the
# kernel name; the first match wins.
STEP_CLASSES = (("qkv_prep", ("qkv_prep_kernel",)), ("qkv_gemm", ("qkv_gemm", "qkv_skinny")),
                ("qkv", ("qkv_fused_kernel",)), ("attn", ("attn_ab_kernel",)), ("merge", ("merge_kernel",)),
                ("block_rows", ("block_rows_stream_kernel", "block_rows_kernel")),
                ("invariant_rows", ("invariant_stream_kernel", "invariant_rows_kernel")))


def step_class(name: str):
    for cls, subs in STEP_CLASSES:
        if any(x in name for x in subs):
            return cls
    return None


def step_traffic(workload, fetch, write, copy_fetch, copy_write, copy_bytes) -> dict:
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    from exact_attention_state_amd import synth
    ff, wf = copy_factor(copy_fetch, copy_bytes), copy_factor(copy_write, copy_bytes)
    acc = bench.step_accounting(synth.WORKLOADS[workload])["kernels"]

    def per_class(path):
        out = {}
        for r in csv.DictReader(open(path)):
            cls = step_class(r["Kernel_Name"])
            if cls:
                grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
                out.setdefault(cls, {}).setdefault(grid, []).append(float(r["Counter_Value"]))
        return out

    f, w = per_class(fetch), per_class(write)
    # Step launches: the attention classes run in steps only; a projection
    # class's step grid is the one launched about as often (the refresh's
    # launches differ in shape and count; a class launched far less often
    # than the steps belongs to the refresh alone and is left out).
    n_step = max((max(len(v) for v in f[c].values()) for c in ("attn", "block_rows", "invariant_rows") if c in f),
                 default=0)

    def step_grid(cls):
        cands = [(abs(len(v) - n_step), g) for g, v in f[cls].items() if len(v) >= 0.9 * n_step]
        return min(cands)[1] if cands else None

    res = {"workload": workload,
           "what": f"HBM traffic per launch of the block-step kernels ({workload} workload, cold-cache protocol with "
                   "rotating sets); per kernel class the dispatches of its step grid size (launched about as often "
                   "as the step's attention); median over those dispatches",
           "calibration": {"copy_kernel": f"__amd_rocclr_copyBuffer, {copy_bytes} bytes read and written "
                                          "(bench.py --copy-calibration)",
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                           "note": "bytes = counter (KiB) x 1024 x factor; the factor is what the same counter "
                                   "reads for the copy"},
           "kernels": {}}
    for cls in sorted(set(f) & set(w)):
        grid = step_grid(cls)
        if grid is None:
            continue
        fk, wk = statistics.median(f[cls][grid]), statistics.median(w[cls].get(grid, [0.0]))
        e = {"source_sha256": bench.kernel_source_hash(cls), "launches": len(f[cls][grid]), "grid_size": grid,
             "fetch_size_kib": round(fk, 1), "write_size_kib": round(wk, 1),
             "hbm_fetch_bytes": round(fk * 1024 * ff), "hbm_write_bytes": round(wk * 1024 * wf)}
        e["hbm_bytes_per_launch"] = e["hbm_fetch_bytes"] + e["hbm_write_bytes"]
        if cls in acc:
            e["algorithmic_bytes"] = acc[cls]["bytes"]
        res["kernels"][cls] = e
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--csv", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--only", nargs="*")
    t.add_argument("--min-grid", type=int)
    t.add_argument("--max-grid", type=int)
    c = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        c.add_argument(a, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--only", nargs="*")
    c.add_argument("--min-grid", type=int)
    c.add_argument("--max-grid", type=int)
    c.add_argument("--command", action="append", default=[], help="a command of the runs (recorded)")
    st = sub.add_parser("step-traffic")
    st.add_argument("--workload", required=True)
    for a_ in ("--fetch", "--write", "--copy-fetch", "--copy-write"):
        st.add_argument(a_, required=True)
    st.add_argument("--copy-bytes", type=int, required=True)
    st.add_argument("--command", action="append", default=[], help="a command of the runs (recorded)")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_markdown(a.csv, a.title, a.command, a.only, a.min_grid, a.max_grid))
    elif a.cmd == "step-traffic":
        res = step_traffic(a.workload, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes)
        res["commands"] = a.command
        json.dump(res, sys.stdout, indent=1)
        sys.stdout.write("\n")
    else:
        res = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.only, a.min_grid, a.max_grid)
        res["commands"] = a.command
        json.dump(res, sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
