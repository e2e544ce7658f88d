"""Matrix-core utilisation of the matrix-core-bound kernels from one rocprofv3 counter run
(measurement support).

    rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 --output-format csv -d DIR -o run \\
        -- python -u bench.py --workload prefill_128k --steps 1 --warmup 1 --no-cpu-baseline
    python -m long_context_sparse_lightning_amd.pmc_mfma DIR/run_counter_collection.csv \\
        --workload prefill_128k --command "rocprofv3 ..."

``MfmaUtil`` is rocprofv3's derived metric: MFMA-busy cycles summed over the SIMDs over
(GPU-active cycles x SIMD count), in percent.  ``SQ_INSTS_VALU_MFMA_MOPS_BF16`` counts bf16
matrix operations in units of 512 flops.  Counter runs serialise and slow kernels, so the
durations here are the profiled ones; the rate worth quoting is the utilisation.  Writes
``profiles/index_qb_and_attention_<workload>_mfma.md``.
"""
from __future__ import annotations

import argparse
import csv
import os
import statistics

from long_context_sparse_lightning_amd.prof_trace import short

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNELS = ("index_scores_qb_kernel", "sparse_mla_kernel", "frontend_proj_lds_kernel")


def per_dispatch(path: str):
    """{dispatch id: {"kernel": name, "ns": duration, counter: value, ...}}."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            d = out.setdefault(int(r["Dispatch_Id"]), {
                "kernel": r["Kernel_Name"],
                "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize(csv_path: str, workload: str, command: str) -> str:
    disp = per_dispatch(csv_path)
    lines = [f"# Matrix-core utilisation: {workload}", "",
             "Command (repository root, one MI355X):", "", f"    {command}", "",
             "| kernel | dispatches | MfmaUtil % (mean) | bf16 matrix flops per dispatch | "
             "profiled duration (us, mean) |", "|---|---|---|---|---|"]
    by_name = {}
    for d in disp.values():
        if "MfmaUtil" in d and any(k in d["kernel"] for k in KERNELS):
            by_name.setdefault(short(d["kernel"]), []).append(d)
    for name in sorted(by_name, key=lambda n: [k in n for k in KERNELS].index(True)):
        ds = by_name[name]
        util = statistics.mean(d["MfmaUtil"] for d in ds)
        flops = statistics.mean(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 for d in ds)
        dur = statistics.mean(d["ns"] for d in ds) / 1e3
        lines.append(f"| {name} | {len(ds)} | {util:.1f} | {flops:.4g} | {dur:.1f} |")
    lines += ["", "MfmaUtil = MFMA-busy cycles summed over SIMDs / (GPU-active cycles x SIMDs); "
              "bf16 matrix flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (includes the padded "
              "and clamped steps the kernels run past the causal edge)."]
    out = os.path.join(ROOT, "profiles", f"index_qb_and_attention_{workload}_mfma.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("csv")
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--command", required=True)
    a = ap.parse_args()
    path = summarize(a.csv, a.workload, a.command)
    with open(path) as f:
        print(f.read())


if __name__ == "__main__":
    main()
