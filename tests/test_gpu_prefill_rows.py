"""Prefill attention on calls of at least 256 (query row, head group) units (one workgroup per
unit, no split of the selection), against the oracle: on lists from the top-k (ragged rows and
dense [0, n) rows, odd row counts, a second head group with padding, small windows, the small
80/64 head dims) and on arbitrary lists a caller may pass (shuffled, repeated positions,
overlapping runs, random, empty), which are also compared with the same rows computed by a call
of fewer rows (split selections and the combine)."""
import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import lsa
from long_context_sparse_lightning_amd.workloads import Workload, device_inputs, host_slice
from lsa_check import (LSE_ABS, assert_attention_close, bf16_to_f64, check_invariants,
                       check_rows_against_oracle, run_path)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

MLA = dict(Dqk=576, Dv=512)
CASES = [
    # one sequence, 520 rows: every list is sink + middle + window
    (Workload("pb_plain", B=1, S_max=6000, Lq=520, seqlens=(6000,), Hi=8, Di=64, topk=512,
              init=16, local=128, H=32, seed=301, **MLA),
     [(0, 0), (0, 1), (0, 2), (0, 3), (0, 260), (0, 518), (0, 519)]),
    # two sequences, 301 rows each (the last block has one row): the short sequence's rows see
    # 400..700 positions, so many lists are the dense [0, n) (one leading run)
    (Workload("pb_ragged_dense", B=2, S_max=3000, Lq=301, seqlens=(3000, 700), Hi=8, Di=64,
              topk=512, init=16, local=128, H=32, seed=302, **MLA),
     [(0, 0), (0, 300), (1, 0), (1, 110), (1, 111), (1, 112), (1, 299), (1, 300)]),
    # 40 heads: a second head group with 8 heads and 24 padding lanes; 513 rows
    (Workload("pb_heads40", B=1, S_max=4000, Lq=513, seqlens=(4000,), Hi=8, Di=64, topk=256,
              init=4, local=64, H=40, seed=303, **MLA),
     [(0, 0), (0, 255), (0, 512)]),
    # small sink and window, big middle
    (Workload("pb_small_window", B=1, S_max=5000, Lq=512, seqlens=(5000,), Hi=8, Di=64,
              topk=384, init=2, local=8, H=32, seed=304, **MLA),
     [(0, 0), (0, 1), (0, 511)]),
    # the small head dims (80 / 64: a tile is not a whole number of DMA instructions)
    (Workload("pb_small_dims", B=1, S_max=3000, Lq=300, seqlens=(3000,), Hi=4, Di=32, topk=256,
              init=4, local=64, H=4, Dqk=80, Dv=64, scale=1.0 / 80 ** 0.5, seed=306),
     [(0, 0), (0, 1), (0, 150), (0, 299)]),
]


@pytest.mark.parametrize("wl,rows", CASES, ids=[c[0].name for c in CASES])
def test_prefill_rows_against_oracle(wl, rows):
    print(f"case {wl.name}", flush=True)
    assert wl.B * wl.Lq * ((wl.H + 31) // 32) >= 256  # one workgroup per unit
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, rows)


def _lists(rng, Lq, S, topk):
    """Index lists of every kind a caller may pass, row i at position p = S - Lq + i."""
    idx = np.full((1, Lq, topk), 0x3fffffff, dtype=np.int32)  # entries past n_sel: never read
    nsel = np.zeros((1, Lq), dtype=np.int32)
    for i in range(Lq):
        p = S - Lq + i
        kind = i % 6
        sink, win = list(range(16)), list(range(p - 63, p + 1))
        mid = sorted(rng.choice(np.arange(16, p - 63), size=topk - 80, replace=False).tolist())
        if kind == 0:    # what the top-k produces
            lst = sink + mid + win
        elif kind == 1:  # the same set in random order
            lst = rng.permutation(sink + mid + win).tolist()
        elif kind == 2:  # repeated positions inside the sink run, the middle and the window
            lst = sink + [3, 3, 15] + mid[: topk - 83 - 3] + [p, p] + win
            lst = lst[:topk]
        elif kind == 3:  # a trailing run that reaches back into the leading run
            lst = list(range(40)) + list(range(20, 60))
        elif kind == 4:  # random positions with repeats, random length
            lst = rng.integers(0, p + 1, size=int(rng.integers(1, topk + 1))).tolist()
        else:            # empty for every sixth row, else a single position
            lst = [] if (i // 6) % 2 == 0 else [int(rng.integers(0, p + 1))]
        nsel[0, i] = len(lst)
        idx[0, i, : len(lst)] = lst
    return idx, nsel


def test_prefill_rows_arbitrary_lists():
    wl = Workload("pb_lists", B=1, S_max=2500, Lq=600, seqlens=(2500,), Hi=8, Di=64, topk=256,
                  init=16, local=64, H=32, seed=305, **MLA)
    print(f"case {wl.name}", flush=True)
    rng = np.random.default_rng(305)
    idx_h, nsel_h = _lists(rng, wl.Lq, wl.S_max, wl.topk)
    X = device_inputs(wl)
    idx = torch.from_numpy(idx_h).cuda()
    nsel = torch.from_numpy(nsel_h).cuda()
    lse = torch.empty(1, wl.Lq, wl.H, dtype=torch.float32, device="cuda")
    out = lsa.lsa_sparse_mla_prefill(X["q0"], X["kv0"], idx, nsel, X["seqlens"], wl.Dv, wl.scale,
                                     lse=lse)
    # the last 200 rows again in a call of 200 rows (each row's selection split over workgroups)
    tail = 200
    lse_s = torch.empty(1, tail, wl.H, dtype=torch.float32, device="cuda")
    out_s = lsa.lsa_sparse_mla_prefill(X["q0"][:, -tail:].contiguous(), X["kv0"],
                                       idx[:, -tail:].contiguous(), nsel[:, -tail:].contiguous(),
                                       X["seqlens"], wl.Dv, wl.scale, lse=lse_s)
    torch.cuda.synchronize()
    for i in range(wl.Lq - tail, wl.Lq):
        assert_attention_close(bf16_to_f64(out[0, i]), bf16_to_f64(out_s[0, i - (wl.Lq - tail)]),
                               f"row {i} vs the 200-row call")
    q_h = host_slice(wl, "q0", 0)
    kv_h = host_slice(wl, "kv0", 0)
    for i in sorted(set(range(0, 24)) | {299, 300, 301, 302, 303, 304, 596, 597, 598, 599}):
        p = wl.S_max - wl.Lq + i
        ref_out, ref_lse = oracle.sparse_mla(q_h[i][None, None], kv_h[None], idx_h[:, i:i + 1],
                                             nsel_h[:, i:i + 1], np.array([p + 1], np.int32),
                                             wl.Dv, wl.scale)
        if nsel_h[0, i] == 0:
            assert torch.count_nonzero(out[0, i]) == 0, f"row {i}: empty list, nonzero output"
            assert torch.all(torch.isneginf(lse[0, i])), f"row {i}: empty list, finite lse"
            continue
        assert_attention_close(bf16_to_f64(out[0, i]), ref_out[0, 0], f"row {i} (kind {i % 6})")
        got_lse = lse[0, i].cpu().numpy().astype(np.float64)
        assert np.abs(got_lse - ref_lse[0, 0]).max() <= LSE_ABS, f"lse row {i}"
