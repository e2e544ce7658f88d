"""Host logic of the counter summaries (no GPU): the copy-calibrated HBM traffic that bench.py
reports as roofline.traffic, its staleness rule, and the matrix-core utilisation table."""
import csv
import json

import pytest

from long_context_sparse_lightning_amd import pmc, pmc_mfma, prof_trace

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (name, counter, value, t0, t1) in enumerate(rows, 1):
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1})


K1 = "void lsa::(anonymous namespace)::index_scores_kernel<128, true>(lsa::(anonymous namespace)::IndexParams)"
MERGE = "lsa::(anonymous namespace)::topk_merge_kernel(lsa::(anonymous namespace)::TopkParams)"
COPY = "__amd_rocclr_copyBuffer"


def test_traffic_is_calibrated_by_the_copy_and_goes_stale_with_the_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(pmc, "ROOT", str(tmp_path))
    # counters in KiB; FETCH_SIZE reads half the true bytes of the 64 MiB copy, WRITE_SIZE all
    fetch = [(K1, "FETCH_SIZE", 1000.0, 0, 1), (MERGE, "FETCH_SIZE", 40.0, 1, 2),
             (K1, "FETCH_SIZE", 1200.0, 2, 3), (MERGE, "FETCH_SIZE", 60.0, 3, 4),
             (COPY, "FETCH_SIZE", 32 * 1024.0, 4, 5)]
    write = [(K1, "WRITE_SIZE", 10.0, 0, 1), (MERGE, "WRITE_SIZE", 2.0, 1, 2),
             (K1, "WRITE_SIZE", 14.0, 2, 3), (MERGE, "WRITE_SIZE", 4.0, 3, 4),
             (COPY, "WRITE_SIZE", 64 * 1024.0, 4, 5)]
    _write_csv(tmp_path / "f.csv", fetch)
    _write_csv(tmp_path / "w.csv", write)
    rec = pmc.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 64, "unit_wl", "fused",
                        4_000_000, "cmd f", "cmd w")
    # per call: mean K1 + mean merge, scaled by the copy's raw/true ratio
    fetch_bytes = (1100.0 + 50.0) * 1024 / 0.5
    write_bytes = (12.0 + 3.0) * 1024 / 1.0
    assert rec["counters"]["FETCH_SIZE"]["factor"] == pytest.approx(0.5)
    assert rec["counters"]["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == round(fetch_bytes + write_bytes)
    assert rec["counters"]["FETCH_SIZE"]["dispatches"] == 2
    # bench.py reads it back while the kernel sources hash the same ...
    assert pmc.load_traffic("unit_wl", "fused") == round(fetch_bytes + write_bytes)
    on_disk = json.load(open(pmc.traffic_path("unit_wl", "fused")))
    assert on_disk["commands"] == ["cmd f", "cmd w"]
    assert (tmp_path / "profiles" / "index_topk_unit_wl_traffic.md").exists()
    # ... and not once they differ from the recorded hash
    monkeypatch.setattr(pmc, "sources_sha256", lambda path: "0" * 64)
    assert pmc.load_traffic("unit_wl", "fused") is None


def test_traffic_counts_every_dispatch_of_a_multi_launch_call(tmp_path, monkeypatch):
    """A call whose merge runs in two launches (two merge dispatches per indexer dispatch): both
    count, per call."""
    monkeypatch.setattr(pmc, "ROOT", str(tmp_path))
    fetch = [(K1, "FETCH_SIZE", 1000.0, 0, 1), (MERGE, "FETCH_SIZE", 40.0, 1, 2),
             (MERGE, "FETCH_SIZE", 20.0, 2, 3), (K1, "FETCH_SIZE", 1200.0, 3, 4),
             (MERGE, "FETCH_SIZE", 60.0, 4, 5), (MERGE, "FETCH_SIZE", 30.0, 5, 6),
             (COPY, "FETCH_SIZE", 64 * 1024.0, 6, 7)]
    write = [(K1, "WRITE_SIZE", 10.0, 0, 1), (MERGE, "WRITE_SIZE", 2.0, 1, 2),
             (MERGE, "WRITE_SIZE", 1.0, 2, 3), (K1, "WRITE_SIZE", 14.0, 3, 4),
             (MERGE, "WRITE_SIZE", 4.0, 4, 5), (MERGE, "WRITE_SIZE", 3.0, 5, 6),
             (COPY, "WRITE_SIZE", 64 * 1024.0, 6, 7)]
    _write_csv(tmp_path / "f.csv", fetch)
    _write_csv(tmp_path / "w.csv", write)
    rec = pmc.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 64, "unit_wl", "fused",
                        1_000_000, "cmd f", "cmd w")
    fetch_bytes = (1100.0 + (40.0 + 20.0 + 60.0 + 30.0) / 2) * 1024
    write_bytes = (12.0 + (2.0 + 1.0 + 4.0 + 3.0) / 2) * 1024
    assert rec["counters"]["FETCH_SIZE"]["dispatches"] == 2
    assert rec["traffic_bytes_per_launch"] == round(fetch_bytes + write_bytes)


def test_traffic_without_a_calibration_copy_is_refused(tmp_path, monkeypatch):
    monkeypatch.setattr(pmc, "ROOT", str(tmp_path))
    _write_csv(tmp_path / "f.csv", [(K1, "FETCH_SIZE", 1.0, 0, 1), (MERGE, "FETCH_SIZE", 1.0, 1, 2)])
    _write_csv(tmp_path / "w.csv", [(K1, "WRITE_SIZE", 1.0, 0, 1), (MERGE, "WRITE_SIZE", 1.0, 1, 2)])
    with pytest.raises(SystemExit):
        pmc.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 64, "unit_wl", "fused", 1,
                      "f", "w")


def test_mfma_table(tmp_path, monkeypatch):
    monkeypatch.setattr(pmc_mfma, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    qb = "void lsa::(anonymous namespace)::index_scores_qb_kernel<8, 2>(lsa::(anonymous namespace)::QbParams)"
    mla = "void lsa::(anonymous namespace)::sparse_mla_kernel<576, 512, true>(lsa::(anonymous namespace)::MlaParams)"
    rows = []
    # two dispatches of each kernel, each with both counters (one row per counter)
    for d, (name, util, mops, t0, t1) in enumerate([(qb, 60.0, 1000.0, 0, 3000), (qb, 64.0, 1000.0, 5000, 9000),
                                                    (mla, 20.0, 10.0, 9000, 10000), (mla, 22.0, 30.0, 10000, 12000)], 1):
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "MfmaUtil",
                     "Counter_Value": util, "Start_Timestamp": t0, "End_Timestamp": t1})
        rows.append({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                     "Counter_Value": mops, "Start_Timestamp": t0, "End_Timestamp": t1})
    with open(tmp_path / "m.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)
    out = pmc_mfma.summarize(str(tmp_path / "m.csv"), "unit_wl", "the command")
    text = open(out).read()
    assert "    the command" in text
    assert "| index_scores_qb_kernel<8, 2> | 2 | 62.0 | 5.12e+05 | 3.5 |" in text
    assert "| sparse_mla_kernel<576, 512, true> | 2 | 21.0 | 1.024e+04 | 1.5 |" in text


def test_trace_summary(tmp_path):
    stats = tmp_path / "run_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": K1, "Calls": 45, "AverageNs": 183800.0, "MinNs": 178800, "MaxNs": 239900})
        w.writerow({"Name": "(anonymous namespace)::gen_fill_kernel(void*, int, unsigned int)",
                    "Calls": 7, "AverageNs": 2000.0, "MinNs": 1000, "MaxNs": 3000})
    bench = {"steps": 20, "ms_per_step": 0.25, "value": 128000.0, "unit": "queries/s",
             "roofline": {"kernel": "lsa_index_topk", "avg_launch_ms": 0.2041, "achieved": 5262.9,
                          "unit": "GB/s", "frac": 0.6579, "peak": 8000.0}}
    text = prof_trace.summarize(str(stats), "t", "rocprofv3 cmd", bench)
    assert "    rocprofv3 cmd" in text
    assert "| index_scores_kernel<128, true> | 45 | 183.8 | 178.8 | 239.9 |" in text
    assert "| gen_fill_kernel (input setup, not a step) | 7 | 2.0 | 1.0 | 3.0 |" in text
    assert "average launch 204.1 us -> 5262.9 GB/s algorithmic (65.8% of 8000.0 GB/s)" in text
    assert "profiler adds per-launch overhead" in text
