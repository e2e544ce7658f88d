"""bench.py's accounting (CPU): the algorithmic bytes and flops it divides by, against the figures
worked out by hand for the headline and prefill workloads, and its one-GPU contract."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_sparse_lightning_amd.workloads import WORKLOADS  # noqa: E402


def test_decode_128k_bytes():
    wl = WORKLOADS["decode_128k"]
    # per row: keys 131072 * 128 * 2, query 32 * 128 * 2 + weights 32 * 4, indices 2048 * 4 + n_sel 4
    assert bench.fused_call_bytes(wl) == 32 * (131072 * 256 + 8192 + 128 + 8192 + 4) == 1_074_270_336
    # the plain indexer writes one fp32 score per key instead of the indices
    assert bench.indexer_bytes(wl) == 32 * (131072 * 260 + 8192 + 128) == 1_090_785_280
    alg, score_rt = bench.algorithmic_bytes(wl)
    # + two attention calls per row: 2048 rows * 1152 B, q 32 * 1152, out 32 * 1024, indices 2048 * 4
    per_mla = 2048 * 1152 + 32 * 1152 + 32 * 1024 + 2048 * 4
    assert alg == 32 * (131072 * 256 + 8192 + 128 + 2048 * 4 + 2 * per_mla) == 1_230_245_888
    assert score_rt == 32 * 2 * 131072 * 4


def test_mtp_decode_128k_bytes():
    wl = WORKLOADS["mtp_decode_128k"]
    assert wl.attn_calls == 3 and [wl.attn_inputs(c) for c in range(3)] == [
        ("q0", "kv0", 0), ("q1", "kv0", 1), ("q2", "kv0", 2)]
    # one index pass over 131070 keys, then draft step c gathers 2048 + c latent rows
    n = 131070
    per_draft = lambda c: (2048 + c) * 1152 + 32 * 1152 + 32 * 1024 + 2048 * 4
    alg, _ = bench.algorithmic_bytes(wl)
    assert alg == 32 * (n * 256 + 8192 + 128 + 2048 * 4 + sum(per_draft(c) for c in range(3)))


def test_hier_decode_128k_bytes():
    wl = WORKLOADS["hier_decode_128k"]
    # window from 131072 - 1024 = 130048: 2032 complete blocks of 64 scored, 32 kept (2048
    # tokens scored), no partial block; the sink and window are forced
    assert bench.index_keys_read(wl, 131072) == 2032 + 32 * 64
    assert bench.index_keys_read(wl, 2000) == 0  # dense fallback: nothing scored
    per_row = 4080 * 256 + 8192 + 128 + 2048 * 4
    assert bench.hier_call_bytes(wl) == 32 * (per_row + 4)
    per_mla = 2048 * 1152 + 32 * 1152 + 32 * 1024 + 2048 * 4
    assert bench.algorithmic_bytes(wl)[0] == 32 * (per_row + 2 * per_mla)


def test_prefill_128k_flops():
    wl = WORKLOADS["prefill_128k"]
    # query i of 4096 sees 126976 + i + 1 keys
    pairs = 4096 * 126976 + 4096 * 4097 // 2
    assert bench.indexer_flops(wl) == 2 * 32 * 128 * pairs == 4_329_343_811_584
    assert bench.query_blocked(wl) and not bench.query_blocked(WORKLOADS["decode_128k"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
