"""GPU parity of the whole hot path at every workload size, through the C ABI, against the CPU
oracle on the same seeded inputs: indexer scores and index sets bit for bit (dyadic index
inputs make the fp32 scores exact), attention within the stated tolerance."""
import dataclasses
import gc

import pytest
import torch

from conftest import gpu_available
from long_context_sparse_lightning_amd.workloads import WORKLOADS, device_inputs
from lsa_check import check_invariants, check_rows_against_oracle, run_path

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _say(msg):
    print(msg, flush=True)


def test_tiny_decode_all_rows():
    wl = WORKLOADS["tiny_decode"]
    _say(f"case {wl.name}")
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, [(b, 0) for b in range(wl.B)])


def test_tiny_decode_four_queries_on_one_cache():
    """Four decode steps at positions 4092..4095 of one 4096-token cache (sequence 0's),
    plus the whole attention step for each, against the oracle."""
    wl = WORKLOADS["tiny_decode"]
    X = device_inputs(wl)
    one = {k: v[:1].contiguous() for k, v in X.items() if k != "seqlens"}
    for n in (4093, 4094, 4095, 4096):
        w1 = dataclasses.replace(wl, B=1, seqlens=(n,))
        X1 = dict(one, seqlens=torch.tensor([n], dtype=torch.int32, device="cuda"))
        sc, idx, nsel, outs, lses = run_path(w1, X1)
        torch.cuda.synchronize()
        check_invariants(w1, idx, nsel, [n])
        check_rows_against_oracle(w1, sc, idx, nsel, outs, lses, [(0, 0)])


def test_decode_32k_all_rows():
    wl = WORKLOADS["decode_32k"]
    _say(f"case {wl.name}")
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, [(b, 0) for b in range(wl.B)])
    del X, sc, idx, nsel, outs, lses
    _free()


def test_decode_128k_two_subblocks_share_indices():
    wl = WORKLOADS["decode_128k"]
    _say(f"case {wl.name}")
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, [(0, 0), (17, 0), (31, 0)])
    del X, sc, idx, nsel, outs, lses
    _free()


def test_prefill_128k_sampled_rows():
    wl = WORKLOADS["prefill_128k"]
    _say(f"case {wl.name}")
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, [(0, 0), (0, 1), (0, 2047), (0, 4095)])
    del X, sc, idx, nsel, outs, lses
    _free()


def test_decode_1m_sampled_rows():
    wl = WORKLOADS["decode_1m"]
    _say(f"case {wl.name}")
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, [(0, 0), (3, 0)])
    del X, sc, idx, nsel, outs, lses
    _free()
