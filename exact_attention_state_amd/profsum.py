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
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_markdown(a.csv, a.title, a.command, a.only, a.min_grid, a.max_grid))
    else:
        res = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.only, a.min_grid, a.max_grid)
        res["commands"] = a.command
        json.dump(res, sys.stdout, indent=1)
        sys.stdout.write("\n")


if __name__ == "__main__":
    main()
