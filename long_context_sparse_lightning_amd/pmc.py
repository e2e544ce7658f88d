"""HBM traffic of the indexer kernel from rocprofv3 counter runs (measurement support).

Two counter runs of ``bench.py --calib-copy-mib M`` are needed, one with ``--pmc FETCH_SIZE`` and
one with ``--pmc WRITE_SIZE`` (rocprofv3 cannot hold both in one pass).  Each run also contains
one device-to-device copy of M MiB, which reads and writes exactly M MiB; the ratio of its
counter value to those bytes calibrates the counter, and the indexer's per-dispatch values are
scaled by it.

    python -m long_context_sparse_lightning_amd.pmc FETCH_CSV WRITE_CSV --calib-mib M \\
        --workload decode_128k --command-fetch "..." --command-write "..."

writes ``profiles/index_scores_<workload>_traffic.json`` (read by bench.py) and a short ``.md``.
The JSON records a hash of the indexer sources; bench.py reports the traffic only while the
sources still hash to it.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KERNEL_SOURCES = ("csrc/lsa_indexer.hip", "csrc/lsa_internal.h")
KERNEL_MATCH = "index_scores_kernel"
COPY_MATCH = "copyBuffer"


def sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"index_scores_{workload}_traffic.json")


def load_traffic(workload: str):
    """Measured HBM bytes per indexer launch, or None if absent or stale."""
    try:
        with open(traffic_path(workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sources_sha256():
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


def summarize(fetch_csv, write_csv, calib_mib, workload, alg_bytes, cmd_fetch, cmd_write):
    calib = calib_mib * (1 << 20)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        disp = _per_dispatch(path, counter)
        k = [v * 1024.0 for n, v in disp.values() if KERNEL_MATCH in n]
        c = [v * 1024.0 for n, v in disp.values() if COPY_MATCH in n]
        if not k or not c:
            raise SystemExit(f"{path}: no {KERNEL_MATCH} or {COPY_MATCH} dispatches")
        factor = max(c) / calib  # the largest copy is the calibration copy
        res[counter] = {"kernel_raw_bytes_mean": statistics.mean(k), "dispatches": len(k),
                        "copy_raw_bytes": max(c), "factor": factor,
                        "kernel_bytes_per_launch": statistics.mean(k) / factor}
    traffic = res["FETCH_SIZE"]["kernel_bytes_per_launch"] + res["WRITE_SIZE"]["kernel_bytes_per_launch"]
    rec = {"kernel": "index_scores_kernel", "workload": workload,
           "traffic_bytes_per_launch": round(traffic),
           "alg_bytes_per_launch": alg_bytes,
           "traffic_over_alg": round(traffic / alg_bytes, 4) if alg_bytes else None,
           "counters": res, "calibration_copy_bytes": calib,
           "source_sha256": sources_sha256(),
           "commands": [cmd_fetch, cmd_write]}
    os.makedirs(os.path.dirname(traffic_path(workload)), exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        json.dump(rec, f, indent=1)
    md = traffic_path(workload)[:-5] + ".md"
    with open(md, "w") as f:
        f.write(f"# HBM traffic of index_scores_kernel: {workload}\n\n")
        f.write("Commands (repository root, one MI355X):\n\n")
        f.write(f"    {cmd_fetch}\n    {cmd_write}\n\n")
        f.write("| counter | kernel raw (mean per dispatch) | copy raw | factor (raw / true copy bytes) | kernel bytes per launch |\n")
        f.write("|---|---|---|---|---|\n")
        for cn, r in res.items():
            f.write(f"| {cn} | {r['kernel_raw_bytes_mean'] / 1e6:.1f} MB ({r['dispatches']} dispatches) | "
                    f"{r['copy_raw_bytes'] / 1e6:.1f} MB | {r['factor']:.4f} | {r['kernel_bytes_per_launch'] / 1e6:.1f} MB |\n")
        f.write(f"\nTraffic per launch: {traffic / 1e6:.1f} MB; algorithmic bytes per launch: "
                f"{alg_bytes / 1e6:.1f} MB (ratio {traffic / alg_bytes:.4f}).  Calibration: one "
                f"device copy of {calib_mib} MiB in the same process.\n")
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--command-fetch", required=True)
    ap.add_argument("--command-write", required=True)
    a = ap.parse_args()
    import sys
    sys.path.insert(0, ROOT)
    from bench import indexer_bytes
    from long_context_sparse_lightning_amd.workloads import WORKLOADS
    rec = summarize(a.fetch_csv, a.write_csv, a.calib_mib, a.workload,
                    indexer_bytes(WORKLOADS[a.workload]), a.command_fetch, a.command_write)
    print(json.dumps({k: rec[k] for k in ("traffic_bytes_per_launch", "alg_bytes_per_launch",
                                           "traffic_over_alg")}))


if __name__ == "__main__":
    main()
