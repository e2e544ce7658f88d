"""lsa_index_topk_noalloc (static per-device workspace, no allocation) through the C ABI against
lsa_index_topk with a caller workspace: identical indices and n_sel, bit for bit, on two calls
in a row -- decode_32k's shapes, then a smaller, ragged call (the static array keeps the first
call's contents, which must not matter) -- and once more at the first shape."""
import ctypes

import numpy as np
import pytest
import torch

from conftest import gpu_available
from long_context_sparse_lightning_amd import lsa
from long_context_sparse_lightning_amd.workloads import WORKLOADS, Workload, device_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SMALL = Workload("noalloc_small", B=3, S_max=5000, Lq=2, seqlens=(5000, 2100, 1500), Hi=17, Di=64,
                 topk=512, init=16, local=100, H=4, Dqk=80, Dv=64, seed=97)


def _noalloc(wl, X):
    idx = torch.full((wl.B, wl.Lq, wl.topk), -7, dtype=torch.int32, device="cuda")
    ns = torch.full((wl.B, wl.Lq), -7, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lsa.lib().lsa_index_topk_noalloc(
        p(X["qidx"]), p(X["w"]), p(X["kidx"]), p(X["seqlens"]), wl.B, wl.Lq, wl.Hi, wl.Di,
        wl.S_max, wl.topk, wl.init, wl.local, p(idx), p(ns),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lsa.lib().lsa_last_error().decode()
    return idx, ns


def _reference(wl, X):
    return lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init, wl.local)


def test_noalloc_equals_workspace_call_on_two_calls():
    big = WORKLOADS["decode_32k"]
    for wl in (big, SMALL, big):
        print(f"case noalloc {wl.name}", flush=True)
        X = device_inputs(wl)
        idx_n, ns_n = _noalloc(wl, X)
        idx_r, ns_r = _reference(wl, X)
        torch.cuda.synchronize()
        assert torch.equal(ns_n, ns_r), wl.name
        assert torch.equal(idx_n, idx_r), wl.name
        assert np.all(ns_n.cpu().numpy() > 0)
