"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare sampled
rows against the CPU oracle on the same seeded inputs (regenerated on the host)."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
from long_context_sparse_lightning_amd import lsa
from long_context_sparse_lightning_amd.workloads import Workload, host_kv_rows, host_slice

# Attention tolerance (per output tensor): max|err| <= 1e-2 * max|ref| and
# ||err||_2 <= 5e-3 * ||ref||_2.  The GPU rounds probabilities and outputs to bf16 (relative
# half-ulp 2^-9), which bounds the expected error near 2e-3 in relative L2.
ATT_MAX_REL = 1e-2
ATT_L2_REL = 5e-3
# log-sum-exp: fp32 logits and bf16-rounded probabilities in the normaliser
LSE_ABS = 5e-3


def assert_attention_close(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    err = got.astype(np.float64) - ref
    maxref = float(np.abs(ref).max())
    maxerr = float(np.abs(err).max())
    l2 = float(np.linalg.norm(err)) / max(float(np.linalg.norm(ref)), 1e-300)
    if os.environ.get("LSA_ERR_LOG"):  # margin report: one line per compared tensor
        with open(os.environ["LSA_ERR_LOG"], "a") as f:
            f.write(f"{what}\tmax_rel {maxerr / max(maxref, 1e-300):.3e}\tl2 {l2:.3e}\n")
    assert maxerr <= ATT_MAX_REL * maxref, f"{what}: max|err| {maxerr:.3e} > 1e-2*{maxref:.3e}"
    assert l2 <= ATT_L2_REL, f"{what}: relative L2 {l2:.3e} > 5e-3"


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_path(wl: Workload, X: dict):
    """One pass of the whole hot path: scores -> top-k -> one MLA call per attention sub-block
    (all sub-blocks share the index pass)."""
    sc = lsa.lsa_index_scores(X["qidx"], X["w"], X["kidx"], X["seqlens"])
    idx, nsel = lsa.lsa_topk_select(sc, X["seqlens"], wl.topk, wl.init, wl.local)
    outs, lses = [], []
    for c in range(wl.mla_calls):
        q, kv = X[f"q{c}"], X[f"kv{c}"]
        lse = torch.empty(wl.B, wl.Lq, wl.H, dtype=torch.float32, device=q.device)
        if wl.decode:
            out = lsa.lsa_sparse_mla_decode(q[:, 0], kv, idx[:, 0], nsel[:, 0], X["seqlens"], wl.Dv,
                                            wl.scale, lse=lse[:, 0])
            out = out[:, None]
        else:
            out = lsa.lsa_sparse_mla_prefill(q, kv, idx, nsel, X["seqlens"], wl.Dv, wl.scale, lse=lse)
        outs.append(out)
        lses.append(lse)
    return sc, idx, nsel, outs, lses


def check_invariants(wl: Workload, idx: torch.Tensor, nsel: torch.Tensor, seqlens) -> None:
    """Properties every row must have (checked on all rows, on the device)."""
    sl = torch.as_tensor(seqlens, dtype=torch.int64, device=idx.device)
    pos = sl[:, None] - wl.Lq + torch.arange(wl.Lq, device=idx.device)[None, :]  # [B, Lq]
    n = pos + 1
    want_n = torch.clamp(n, max=wl.topk)
    assert torch.equal(nsel.long(), want_n), "n_sel != min(n, topk)"
    K = wl.topk
    j = torch.arange(K, device=idx.device)[None, None, :]
    valid = j < want_n[..., None]
    assert bool(((idx >= 0) == valid).all()), "padding must be exactly the slots past n_sel"
    i64 = idx.long()
    assert bool((torch.where(valid, i64, 0) <= pos[..., None]).all()), "index past the query"
    d = i64[..., 1:] - i64[..., :-1]
    assert bool(torch.where(valid[..., 1:], d > 0, True).all()), "indices must be ascending"
    long_rows = n > K
    if bool(long_rows.any()) and wl.topk > wl.init + wl.local:
        first = i64[..., : wl.init]
        assert bool(torch.where(long_rows[..., None], first == torch.arange(wl.init, device=idx.device),
                                True).all()), "sink columns missing"
        last = i64[..., K - wl.local:]
        want_last = pos[..., None] - wl.local + 1 + torch.arange(wl.local, device=idx.device)
        assert bool(torch.where(long_rows[..., None], last == want_last, True).all()), \
            "window columns missing"


def check_rows_against_oracle(wl: Workload, sc, idx, nsel, outs, lses, rows) -> None:
    """Bit-exact scores and index sets, and attention within tolerance, for rows (b, i)."""
    by_b = {}
    for b, i in rows:
        by_b.setdefault(b, []).append(i)
    for b, qs in by_b.items():
        qidx = host_slice(wl, "qidx", b)
        w = host_slice(wl, "w", b)
        keys = host_slice(wl, "kidx", b)
        for i in qs:
            p = wl.seqlens[b] - wl.Lq + i
            n = p + 1
            ref_sc = oracle.index_scores(qidx[None, i:i + 1], w[None, i:i + 1], keys[None, :n],
                                         np.array([n], np.int32), 1)[0, 0]
            got_sc = sc[b, i, :n].cpu().numpy()
            mism = np.nonzero(got_sc.view(np.uint32) != ref_sc.view(np.uint32))[0]
            assert mism.size == 0, (f"scores row (b={b}, i={i}): {mism.size} mismatches, first at "
                                    f"{mism[:5]}: got {got_sc[mism[:5]]} want {ref_sc[mism[:5]]}")
            ref_idx, ref_n = oracle.topk_select(ref_sc[None, None, :], np.array([n], np.int32),
                                                wl.topk, wl.init, wl.local)
            got_idx = idx[b, i].cpu().numpy()
            assert int(nsel[b, i]) == int(ref_n[0, 0])
            assert np.array_equal(got_idx, ref_idx[0, 0]), (
                f"indices row (b={b}, i={i}) differ at {np.nonzero(got_idx != ref_idx[0, 0])[0][:8]}")
            sel = ref_idx[0, 0, : ref_n[0, 0]]
            m = sel.size
            for c in range(wl.mla_calls):
                kv_rows = host_kv_rows(wl, f"kv{c}", b, sel)
                q_row = host_slice(wl, f"q{c}", b)[i]
                ref_out, ref_lse = oracle.sparse_mla(
                    q_row[None, None], kv_rows[None], np.arange(m, dtype=np.int32)[None, None],
                    np.array([[m]], np.int32), np.array([m], np.int32), wl.Dv, wl.scale)
                assert_attention_close(bf16_to_f64(outs[c][b, i]), ref_out[0, 0],
                                       f"{wl.name} call {c} row (b={b}, i={i})")
                got_lse = lses[c][b, i].cpu().numpy().astype(np.float64)
                assert np.abs(got_lse - ref_lse[0, 0]).max() <= LSE_ABS, f"lse row (b={b}, i={i})"
