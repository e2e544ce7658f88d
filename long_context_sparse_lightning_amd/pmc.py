"""HBM traffic of the indexer kernel from rocprofv3 counter runs (measurement support).

Two counter runs of ``bench.py --path P --calib-copy-mib M`` are needed, one with ``--pmc FETCH_SIZE`` and
one with ``--pmc WRITE_SIZE`` (rocprofv3 cannot hold both in one pass).  Each run also contains
one device-to-device copy of M MiB, which reads and writes exactly M MiB; the ratio of its
counter value to those bytes calibrates the counter, and the indexer's per-dispatch values are
scaled by it.

    python -m long_context_sparse_lightning_amd.pmc FETCH_CSV WRITE_CSV --calib-mib M \\
        --workload decode_128k --path fused --command-fetch "..." --command-write "..."

writes ``profiles/<stage>_<workload>_traffic.json`` (read by bench.py) and a short ``.md``.
The JSON records a hash of the indexer sources; bench.py reports the traffic only while the
sources still hash to it.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# per bench path: the kernels of the measured call (one dispatch each per call), their sources
PATHS = {
    "split": {"name": "index_scores", "kernels": ("index_scores_kernel",),
              "sources": ("csrc/lsa_indexer.hip", "csrc/lsa_select.h", "csrc/lsa_internal.h")},
    "fused": {"name": "index_topk", "kernels": ("index_scores_kernel", "topk_merge_kernel"),
              "sources": ("csrc/lsa_indexer.hip", "csrc/lsa_select.h", "csrc/lsa_topk.hip",
                          "csrc/lsa_internal.h")},
    # one decode attention call (lsa_sparse_mla_decode): the split kernel and the combine
    "attention": {"name": "attention", "kernels": ("sparse_mla_kernel", "mla_combine_kernel"),
                  "sources": ("csrc/lsa_mla.hip", "csrc/lsa_internal.h")},
}
COPY_MATCH = "copyBuffer"


def sources_sha256(path: str) -> str:
    h = hashlib.sha256()
    for rel in PATHS[path]["sources"]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(workload: str, path: str) -> str:
    return os.path.join(ROOT, "profiles", f"{PATHS[path]['name']}_{workload}_traffic.json")


def load_traffic(workload: str, path: str):
    """Measured HBM bytes per call of the path's indexer stage, or None if absent or stale."""
    try:
        with open(traffic_path(workload, path)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sources_sha256(path):
        return None
    return rec.get("traffic_bytes_per_launch")


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value in KiB)} for one counter."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            prev = out.get(d)
            out[d] = (name, val + (prev[1] if prev else 0.0))
    return out


def summarize(fetch_csv, write_csv, calib_mib, workload, path, alg_bytes, cmd_fetch, cmd_write):
    calib = calib_mib * (1 << 20)
    kernels = PATHS[path]["kernels"]
    res = {}
    for counter, csv_path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(csv_path, counter)
        c = [v * 1024.0 for n, v in disp.values() if COPY_MATCH in n]
        if not c:
            raise SystemExit(f"{csv_path}: no {COPY_MATCH} dispatch")
        factor = max(c) / calib  # the largest copy is the calibration copy
        # The first kernel runs once per call; the others may run more than once (a two-level
        # merge): per call, every matching dispatch summed over the number of calls.
        raw, calls = 0.0, None
        per_kernel = {}
        for kname in kernels:
            k = [v * 1024.0 for n, v in disp.values() if kname in n]
            if not k:
                raise SystemExit(f"{csv_path}: no {kname} dispatches")
            if calls is None:
                calls = len(k)
            raw += sum(k) / calls
            per_kernel[kname] = sum(k) / calls / factor
        res[counter] = {"kernel_raw_bytes_mean": raw, "dispatches": calls,
                        "copy_raw_bytes": max(c), "factor": factor,
                        "kernel_bytes_per_launch": raw / factor,
                        "bytes_per_kernel": {k: round(v) for k, v in per_kernel.items()}}
    traffic = res["FETCH_SIZE"]["kernel_bytes_per_launch"] + res["WRITE_SIZE"]["kernel_bytes_per_launch"]
    rec = {"kernels": list(kernels), "path": path, "workload": workload,
           "traffic_bytes_per_launch": round(traffic),
           "alg_bytes_per_launch": alg_bytes,
           "traffic_over_alg": round(traffic / alg_bytes, 4) if alg_bytes else None,
           "counters": res, "calibration_copy_bytes": calib,
           "source_sha256": sources_sha256(path),
           "commands": [cmd_fetch, cmd_write]}
    out = traffic_path(workload, path)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    with open(out[:-5] + ".md", "w") as f:
        f.write(f"# HBM traffic of {' + '.join(kernels)} ({path} path): {workload}\n\n")
        f.write("Commands (repository root, one MI355X):\n\n")
        f.write(f"    {cmd_fetch}\n    {cmd_write}\n\n")
        f.write("| counter | kernels raw (per call) | copy raw | factor (raw / true copy bytes) | bytes per call |\n")
        f.write("|---|---|---|---|---|\n")
        for cn, r in res.items():
            f.write(f"| {cn} | {r['kernel_raw_bytes_mean'] / 1e6:.1f} MB ({r['dispatches']} dispatches) | "
                    f"{r['copy_raw_bytes'] / 1e6:.1f} MB | {r['factor']:.4f} | {r['kernel_bytes_per_launch'] / 1e6:.1f} MB |\n")
        f.write("\n| kernel | FETCH_SIZE bytes per call | WRITE_SIZE bytes per call |\n|---|---|---|\n")
        for kname in kernels:
            f.write(f"| {kname} | {res['FETCH_SIZE']['bytes_per_kernel'][kname] / 1e6:.1f} MB | "
                    f"{res['WRITE_SIZE']['bytes_per_kernel'][kname] / 1e6:.1f} MB |\n")
        f.write(f"\nTraffic per call: {traffic / 1e6:.1f} MB; algorithmic bytes per call: "
                f"{alg_bytes / 1e6:.1f} MB (ratio {traffic / alg_bytes:.4f}).  Calibration: one "
                f"device copy of {calib_mib} MiB in the same process.\n")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--path", choices=tuple(PATHS), default="fused")
    ap.add_argument("--command-fetch", required=True)
    ap.add_argument("--command-write", required=True)
    a = ap.parse_args()
    import sys
    sys.path.insert(0, ROOT)
    from bench import attention_call_bytes, fused_call_bytes, indexer_bytes
    from long_context_sparse_lightning_amd.workloads import WORKLOADS
    wl = WORKLOADS[a.workload]
    alg = {"fused": fused_call_bytes, "split": indexer_bytes,
           "attention": attention_call_bytes}[a.path](wl)
    rec = summarize(a.fetch_csv, a.write_csv, a.calib_mib, a.workload, a.path, alg,
                    a.command_fetch, a.command_write)
    print(json.dumps({k: rec[k] for k in ("traffic_bytes_per_launch", "alg_bytes_per_launch",
                                           "traffic_over_alg")}))


if __name__ == "__main__":
    main()
