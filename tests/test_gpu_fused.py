"""The fused indexer + top-k entry point (lsa_index_topk) against the two-call path and the
oracle: identical indices and n_sel, bit for bit, on every workload and on edge geometries
(ragged rows, the dense fallback, no free slot, small chunks, prefill rows, odd head counts)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import lsa
from long_context_sparse_lightning_amd.workloads import WORKLOADS, Workload, device_inputs, host_slice
from lsa_check import check_invariants

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

EDGE = [
    Workload("f_ragged", B=6, S_max=3000, Lq=1, seqlens=(1, 17, 256, 257, 3000, 2048), Hi=4, Di=32,
             topk=256, init=4, local=64, H=4, Dqk=80, Dv=64, seed=91),
    Workload("f_odd_heads_di64", B=3, S_max=5000, Lq=1, seqlens=(5000, 4097, 999), Hi=17, Di=64,
             topk=512, init=16, local=100, H=4, Dqk=80, Dv=64, seed=92),
    Workload("f_prefill", B=2, S_max=9000, Lq=40, seqlens=(9000, 3000), Hi=32, Di=128, topk=1024,
             init=16, local=256, H=4, Dqk=80, Dv=64, seed=93),
    Workload("f_no_free_slot", B=2, S_max=2000, Lq=1, seqlens=(2000, 1500), Hi=8, Di=32, topk=96,
             init=32, local=64, H=4, Dqk=80, Dv=64, seed=94),
    Workload("f_multi_chunk", B=3, S_max=70001, Lq=1, seqlens=(70001, 40000, 2049), Hi=8, Di=128,
             topk=2048, init=16, local=1024, H=4, Dqk=80, Dv=64, seed=95),
    # topk = 1 with no forced column: the arg-max, lowest position among ties
    Workload("f_topk1", B=3, S_max=5000, Lq=1, seqlens=(1, 2, 5000), Hi=4, Di=32, topk=1, init=0,
             local=0, H=4, Dqk=80, Dv=64, seed=96),
    # the longest supported row (S_max = 2^20)
    Workload("f_max_len", B=1, S_max=1 << 20, Lq=1, seqlens=(1 << 20,), Hi=4, Di=32, topk=2048,
             init=16, local=1024, H=4, Dqk=80, Dv=64, seed=97),
]


def _both(wl):
    X = device_inputs(wl)
    sc = lsa.lsa_index_scores(X["qidx"], X["w"], X["kidx"], X["seqlens"])
    idx_u, ns_u = lsa.lsa_topk_select(sc, X["seqlens"], wl.topk, wl.init, wl.local)
    idx_f, ns_f = lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init,
                                     wl.local)
    torch.cuda.synchronize()
    return X, sc, idx_u, ns_u, idx_f, ns_f


@pytest.mark.parametrize("name", ["tiny_decode", "decode_32k", "decode_128k", "prefill_128k",
                                  "decode_1m"])
def test_fused_equals_two_call_path(name):
    wl = WORKLOADS[name]
    print(f"case {name}", flush=True)
    X, sc, idx_u, ns_u, idx_f, ns_f = _both(wl)
    assert torch.equal(ns_f, ns_u)
    assert torch.equal(idx_f, idx_u)
    check_invariants(wl, idx_f, ns_f, wl.seqlens)


@pytest.mark.parametrize("wl", EDGE, ids=lambda w: w.name)
def test_fused_edges_against_oracle(wl):
    print(f"case {wl.name}", flush=True)
    X, sc, idx_u, ns_u, idx_f, ns_f = _both(wl)
    assert torch.equal(ns_f, ns_u)
    assert torch.equal(idx_f, idx_u)
    check_invariants(wl, idx_f, ns_f, wl.seqlens)
    # a few rows straight against the oracle's selection over the oracle's scores
    for b in range(wl.B):
        qidx = host_slice(wl, "qidx", b)
        w = host_slice(wl, "w", b)
        keys = host_slice(wl, "kidx", b)
        for i in sorted({0, wl.Lq - 1}):
            n = wl.seqlens[b] - wl.Lq + i + 1
            ref_sc = oracle.index_scores(qidx[None, i:i + 1], w[None, i:i + 1], keys[None, :n],
                                         np.array([n], np.int32), 1)[0, 0]
            ref_idx, ref_n = oracle.topk_select(ref_sc[None, None, :], np.array([n], np.int32),
                                                wl.topk, wl.init, wl.local)
            assert int(ns_f[b, i]) == int(ref_n[0, 0])
            assert np.array_equal(idx_f[b, i].cpu().numpy(), ref_idx[0, 0]), f"row (b={b}, i={i})"


def test_fused_is_deterministic_and_ignores_workspace_contents():
    wl = WORKLOADS["decode_32k"]
    X = device_inputs(wl)
    need = lsa.lsa_index_topk_workspace_bytes(wl.B, wl.Lq, wl.S_max, wl.topk, wl.init, wl.local)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    a = lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init, wl.local,
                           workspace=ws)
    ws.fill_(0x5A)
    b = lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init, wl.local,
                           workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("B,S,seqlens", [
    # chunks of 8192 keys (25 lists per row): every chunk cuts its tied list to its exact top R,
    # then two merge levels
    (8, 200000, (200000, 150001, 99999, 2049, 2048, 60000, 131072, 7000)),
    # 37 lists per row, two merge levels, rows of very different lengths
    (2, 300000, (300000, 5000)),
    # chunks of 6272 keys (16 lists per row): the cut lists, one merge
    (2, 100000, (100000, 33333)),
])
def test_fused_all_equal_scores_many_lists(B, S, seqlens):
    """Zero index queries make every score 0: the selection is then decided by positions alone
    (the lowest middle positions), through the chunks' exact cut and the two-level merge."""
    print(f"case all-equal B={B} S={S}", flush=True)
    wl = Workload("f_tied", B=B, S_max=S, Lq=1, seqlens=seqlens, Hi=8, Di=128, topk=2048, init=16,
                  local=1024, H=4, Dqk=80, Dv=64, seed=96)
    X = device_inputs(wl)
    q0 = torch.zeros_like(X["qidx"])
    idx_f, ns_f = lsa.lsa_index_topk(q0, X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init, wl.local)
    sc = lsa.lsa_index_scores(q0, X["w"], X["kidx"], X["seqlens"])
    idx_u, ns_u = lsa.lsa_topk_select(sc, X["seqlens"], wl.topk, wl.init, wl.local)
    torch.cuda.synchronize()
    zeros = np.zeros((B, 1, S), np.float32)
    ref_idx, ref_n = oracle.topk_select(zeros, np.array(seqlens, np.int32), wl.topk, wl.init,
                                        wl.local)
    assert np.array_equal(ns_f.cpu().numpy(), ref_n) and np.array_equal(ns_u.cpu().numpy(), ref_n)
    assert np.array_equal(idx_f.cpu().numpy(), ref_idx)
    assert np.array_equal(idx_u.cpu().numpy(), ref_idx)
