"""Kernel-trace summary of one bench run (measurement support).

    rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o run \\
        -- python -u bench.py --steps 20 --warmup 5 --no-cpu-baseline
    python -m long_context_sparse_lightning_amd.prof_trace DIR/run_kernel_stats.csv OUT.md \\
        --title "..." --command "rocprofv3 ..." [--bench bench_line.json]

Writes a table of calls and average / min / max duration per kernel (template arguments kept,
parameter lists dropped) and, with ``--bench``, the bench line of the same build: its step time,
throughput and the dominant call's roofline figures.
"""
from __future__ import annotations

import argparse
import csv
import json
import re


# torch kernels the bench runs around the steps
NOTES = {"gen_fill_kernel": "input setup, not a step",
         "reduce_kernel<…>": "torch sum: the cold-cache pass's 1 GiB flush read, outside the steps",
         "vectorized_elementwise_kernel<…>": "torch fill, setup"}


def short(name: str) -> str:
    """``void ns::(anonymous namespace)::kernel<1, 2>(Params)`` -> ``kernel<1, 2>``; long or
    lambda-bearing template argument lists become ``<…>``."""
    s = name[5:] if name.startswith("void ") else name
    s = s.replace("(anonymous namespace)::", "")
    cut = [k for k in (s.find("<"), s.find("(")) if k >= 0]
    i = min(cut) if cut else len(s)
    base = s[:i].split("::")[-1]
    if i < len(s) and s[i] == "<":
        depth, j = 0, i
        for j in range(i, len(s)):
            depth += (s[j] == "<") - (s[j] == ">")
            if depth == 0:
                break
        args = s[i:j + 1]
        return base + (args if "(" not in args and len(args) <= 40 else "<…>")
    return base


def summarize(stats_csv: str, title: str, command: str, bench: dict | None = None) -> str:
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "",
             f"    {command}", "", "| kernel | calls | avg us | min us | max us |",
             "|---|---|---|---|---|"]
    with open(stats_csv, newline="") as f:
        for r in csv.DictReader(f):
            n = short(r["Name"])
            if n in NOTES:
                n += f" ({NOTES[n]})"
            lines.append(f"| {n} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    if bench:
        rf = bench["roofline"]
        lines += ["", f"bench.py's line from this traced run (HIP events, {bench['steps']} timed steps; the "
                  f"profiler adds per-launch overhead, so unprofiled runs are faster): "
                  f"{bench['ms_per_step']} ms/step, {bench['value']} {bench['unit']}; {rf['kernel']} "
                  f"average launch {rf['avg_launch_ms'] * 1e3:.1f} us -> {rf['achieved']} {rf['unit']} "
                  f"algorithmic ({rf['frac'] * 100:.1f}% of {rf['peak']} {rf['unit']})."]
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("stats_csv")
    ap.add_argument("out")
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--bench", default=None, help="file holding the bench's JSON line")
    a = ap.parse_args()
    bench = None
    if a.bench:
        with open(a.bench) as f:
            bench = json.loads([l for l in f if l.startswith("{")][-1])
    text = summarize(a.stats_csv, a.title, a.command, bench)
    with open(a.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
