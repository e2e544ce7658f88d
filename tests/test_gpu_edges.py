"""GPU edge cases against the oracle: ragged and tiny sequences, n around topk, odd head
counts, several head groups, prefill chunks, deep top-k trees, heavy ties and signed zeros,
R = 0, dense attention, determinism and input immutability."""
import dataclasses
import hashlib

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import inputs as gen
from long_context_sparse_lightning_amd import lsa
from long_context_sparse_lightning_amd.workloads import Workload, device_inputs, host_slice
from lsa_check import (assert_attention_close, bf16_to_f64, check_invariants,
                       check_rows_against_oracle, run_path)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SMALL = [
    # ragged decode; 40 heads -> two head groups; full-size latent rows
    Workload("ragged_decode", B=6, S_max=3000, Lq=1, seqlens=(1, 17, 256, 257, 3000, 2048), Hi=4,
             Di=32, topk=256, init=4, local=64, H=40, seed=77),
    # odd index-head count, Di = 128, the tiny latent shape
    Workload("odd_heads", B=3, S_max=5000, Lq=1, seqlens=(5000, 4097, 999), Hi=17, Di=128,
             topk=512, init=16, local=100, H=4, Dqk=80, Dv=64, scale=0.11, seed=79),
    # Di = 64, prefill chunk of 50 queries on two ragged sequences, 2 calls sharing indices
    Workload("prefill_small", B=2, S_max=700, Lq=50, seqlens=(700, 300), Hi=32, Di=64, topk=128,
             init=2, local=8, H=4, Dqk=80, Dv=64, scale=0.125, mla_calls=2, seed=78),
    # topk == init + local: no free slot
    Workload("no_free_slot", B=2, S_max=2000, Lq=1, seqlens=(2000, 1500), Hi=8, Di=32, topk=96,
             init=32, local=64, H=4, Dqk=80, Dv=64, seed=80),
    # query-blocked prefill scan (Di = 128, Lq >= 16): ragged sequences, a partial query block,
    # a sequence as short as its chunk, odd index-head count
    Workload("prefill_qblock", B=3, S_max=5000, Lq=21, seqlens=(5000, 2100, 21), Hi=17, Di=128,
             topk=256, init=4, local=32, H=4, Dqk=80, Dv=64, scale=0.125, seed=83),
    # several top-k chunks (S_max > 16384) with a single merge level
    Workload("multi_chunk", B=2, S_max=40000, Lq=1, seqlens=(40000, 20000), Hi=8, Di=32, topk=256,
             init=4, local=16, H=32, seed=81),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_small_workloads_all_rows(wl):
    print(f"case {wl.name}", flush=True)
    X = device_inputs(wl)
    sc, idx, nsel, outs, lses = run_path(wl, X)
    torch.cuda.synchronize()
    check_invariants(wl, idx, nsel, wl.seqlens)
    rows = [(b, i) for b in range(wl.B) for i in range(wl.Lq)]
    check_rows_against_oracle(wl, sc, idx, nsel, outs, lses, rows)


def _topk_both(scores_np, seqlens, topk, init, local):
    sc = torch.from_numpy(scores_np).cuda()
    sl = torch.tensor(seqlens, dtype=torch.int32, device="cuda")
    idx, nsel = lsa.lsa_topk_select(sc, sl, topk, init, local)
    torch.cuda.synchronize()
    ref_idx, ref_n = oracle.topk_select(scores_np, np.array(seqlens, np.int32), topk, init, local)
    return idx.cpu().numpy(), nsel.cpu().numpy(), ref_idx, ref_n


@pytest.mark.parametrize("S,topk,init,local,seqlens", [
    (300000, 8192, 16, 1024, (300000, 123457)),   # R = 7152: merge groups of 2 -> deep tree
    (200000, 2048, 16, 1024, (200000, 16385)),
    (40000, 64, 0, 0, (40000, 33000)),
    (16384, 2048, 16, 1024, (16384, 2049)),
    # degenerate selections: the arg-max (lowest position among ties), the sink alone, the
    # current position alone, one of each; rows of one and two positions take the dense path
    (5000, 1, 0, 0, (5000, 2, 1)),
    (5000, 1, 1, 0, (5000, 2, 1)),
    (5000, 1, 0, 1, (5000, 2, 1)),
    (70000, 2, 1, 1, (70000, 3)),
])
def test_topk_on_tied_fp32_scores(S, topk, init, local, seqlens):
    """Scores built from bf16 values (8-bit mantissa -> heavy ties), negatives and signed
    zeros; both sides rank the same fp32 values."""
    print(f"case topk S={S} topk={topk}", flush=True)
    B = len(seqlens)
    h = gen.hashes(4242, gen.TAGS["scores"], np.arange(B * S, dtype=np.uint64))
    vals = gen.bf16_bits_to_f32(gen.values_from_hashes(h, gen.NORMAL)).reshape(B, 1, S).copy()
    vals[:, :, 100:400] = 0.0
    vals[:, :, 200:300] = -0.0
    idx, nsel, ref_idx, ref_n = _topk_both(vals, seqlens, topk, init, local)
    assert np.array_equal(nsel, ref_n)
    assert np.array_equal(idx, ref_idx)


def test_topk_extreme_finite_scores():
    """Rows reaching -FLT_MAX and +FLT_MAX, subnormals and signed zeros, over several chunks
    whose first and last ones are partial: the selection marks positions outside a chunk's
    competing range with the key 0, which must stay below every finite score's key (the
    smallest is that of -FLT_MAX) and out of every histogram and list."""
    print("case topk extreme finite scores", flush=True)
    S, B = 70000, 3
    big = np.float32(np.finfo(np.float32).max)
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    h = gen.hashes(4343, gen.TAGS["scores"], np.arange(B * S, dtype=np.uint64))
    vals = gen.bf16_bits_to_f32(gen.values_from_hashes(h, gen.NORMAL)).reshape(B, 1, S).copy()
    vals[0, 0, ::7] = -big                   # the lowest key in every chunk
    vals[0, 0, 5::11] = big                  # and the highest
    vals[0, 0, 3::13] = tiny
    vals[0, 0, 4::13] = -tiny
    vals[1, 0, :] = -big                     # one key value everywhere but a few positions
    vals[1, 0, 9000:9300] = -0.0
    vals[1, 0, 30000:30010] = big
    vals[2, 0, :] = 0.0                      # signed zeros and extremes only
    vals[2, 0, 1::2] = -0.0
    vals[2, 0, 17::1000] = -big
    vals[2, 0, 18::1000] = big
    idx, nsel, ref_idx, ref_n = _topk_both(vals, (70000, 40001, 16385), 2048, 16, 1024)
    assert np.array_equal(nsel, ref_n)
    assert np.array_equal(idx, ref_idx)


def test_topk_many_rows_half_size_merges():
    """1024 query rows select through 512-thread merges (two per CU): heavily tied bf16-valued
    scores, signed zeros, and rows where more keys than one such merge ranks share the
    threshold value, against the oracle."""
    print("case topk 1024 rows", flush=True)
    S, Lq = 20000, 1024
    h = gen.hashes(4444, gen.TAGS["scores"], np.arange(Lq * S, dtype=np.uint64))
    vals = gen.bf16_bits_to_f32(gen.values_from_hashes(h, gen.DYADIC)).reshape(1, Lq, S).copy()
    vals[0, ::3, 2000:9000] = 0.0          # thousands of keys tied at the threshold
    vals[0, 1::3, 5000:5600] = -0.0
    idx, nsel, ref_idx, ref_n = _topk_both(vals, (S,), 2048, 16, 1024)
    assert np.array_equal(nsel, ref_n)
    assert np.array_equal(idx, ref_idx)


def test_topk_all_equal_scores():
    S = 50000
    vals = np.zeros((2, 1, S), np.float32)
    idx, nsel, ref_idx, ref_n = _topk_both(vals, (S, 30000), 2048, 16, 1024)
    assert np.array_equal(idx, ref_idx) and np.array_equal(nsel, ref_n)


def test_topk_prefill_rows_boundaries():
    """Lq rows crossing n = topk: rows below use the dense fallback, rows above select."""
    S, Lq, topk = 600, 40, 580
    h = gen.hashes(99, gen.TAGS["scores"], np.arange(S * Lq, dtype=np.uint64))
    vals = gen.bf16_bits_to_f32(gen.values_from_hashes(h, gen.DYADIC)).reshape(1, Lq, S).copy()
    idx, nsel, ref_idx, ref_n = _topk_both(vals, (S,), topk, 3, 5)
    assert np.array_equal(idx, ref_idx) and np.array_equal(nsel, ref_n)


def _dense_case(Lq):
    wl = Workload("dense", B=2, S_max=900, Lq=Lq, seqlens=(900, 333), Hi=4, Di=32, topk=64, init=2,
                  local=4, H=36, Dqk=576, Dv=512, seed=83)
    X = device_inputs(wl)
    return wl, X


@pytest.mark.parametrize("Lq", [1, 7])
def test_dense_attention_matches_oracle(Lq):
    """indices == NULL: attention over every position 0..p (decode) / causal (prefill)."""
    wl, X = _dense_case(Lq)
    lse = torch.empty(wl.B, Lq, wl.H, dtype=torch.float32, device="cuda")
    if Lq == 1:
        out = lsa.lsa_sparse_mla_decode(X["q0"][:, 0], X["kv0"], None, None, X["seqlens"], wl.Dv,
                                        wl.scale, lse=lse[:, 0])[:, None]
    else:
        out = lsa.lsa_sparse_mla_prefill(X["q0"], X["kv0"], None, None, X["seqlens"], wl.Dv,
                                         wl.scale, lse=lse)
    torch.cuda.synchronize()
    for b in range(wl.B):
        q = host_slice(wl, "q0", b)[None]
        kv = host_slice(wl, "kv0", b)[None]
        ref, ref_lse = oracle.sparse_mla(q, kv, None, None, np.array([wl.seqlens[b]], np.int32),
                                         wl.Dv, wl.scale)
        assert_attention_close(bf16_to_f64(out[b]), ref[0], f"dense b={b}")
        assert np.abs(lse[b].cpu().numpy() - ref_lse[0]).max() <= 5e-3


def test_attention_largest_selection():
    """topk at its largest (131072, every split of the launch at its LDS slice limit): one row
    lists all 131072 positions of its cache in shuffled order, so it equals dense attention; a
    second row lists 65536 distinct positions of its 100000, and the list entries past n_sel
    hold out-of-range values that must be ignored.  Both rows against the oracle."""
    topk = 131072
    wl = Workload("max_selection", B=2, S_max=topk, Lq=1, seqlens=(topk, 100000), Hi=4, Di=32,
                  topk=topk, init=0, local=0, H=4, seed=86)
    print("case attention topk=131072", flush=True)
    X = device_inputs(wl)
    rng = np.random.default_rng(86)
    idx = np.empty((2, topk), np.int32)
    idx[0] = rng.permutation(topk)
    idx[1, :65536] = rng.choice(100000, 65536, replace=False)
    idx[1, 65536::2] = -7
    idx[1, 65537::2] = 1 << 30
    nsel = np.array([topk, 65536], np.int32)
    lse = torch.empty(wl.B, wl.H, dtype=torch.float32, device="cuda")
    out = lsa.lsa_sparse_mla_decode(X["q0"][:, 0], X["kv0"], torch.from_numpy(idx).cuda(),
                                    torch.from_numpy(nsel).cuda(), X["seqlens"], wl.Dv, wl.scale,
                                    lse=lse)
    dense = lsa.lsa_sparse_mla_decode(X["q0"][:, 0], X["kv0"], None, None, X["seqlens"], wl.Dv,
                                      wl.scale)
    torch.cuda.synchronize()
    for b in range(wl.B):
        q = host_slice(wl, "q0", b)[None]
        kv = host_slice(wl, "kv0", b)[None]
        ref, ref_lse = oracle.sparse_mla(q, kv, idx[b][None, None], nsel[b][None, None],
                                         np.array([wl.seqlens[b]], np.int32), wl.Dv, wl.scale)
        assert_attention_close(bf16_to_f64(out[b][None]), ref[0], f"max selection b={b}")
        assert np.abs(lse[b].cpu().numpy() - ref_lse[0, 0]).max() <= 5e-3
    assert_attention_close(bf16_to_f64(out[0][None]), bf16_to_f64(dense[0][None]),
                           "max selection row 0 against dense attention")


def test_dense_fallback_equals_dense_attention():
    """n <= topk: the selection is 0..n-1, and attention with it equals indices == NULL."""
    wl = Workload("fallback", B=2, S_max=300, Lq=1, seqlens=(200, 256), Hi=4, Di=32, topk=256,
                  init=4, local=64, H=4, Dqk=80, Dv=64, seed=84)
    X = device_inputs(wl)
    sc, idx, nsel, outs, _ = run_path(wl, X)
    dense = lsa.lsa_sparse_mla_decode(X["q0"][:, 0], X["kv0"], None, None, X["seqlens"], wl.Dv,
                                      wl.scale)
    torch.cuda.synchronize()
    assert nsel[:, 0].tolist() == [200, 256]
    d = (outs[0][:, 0].float() - dense.float()).abs().max().item()
    assert d <= 1e-2 * dense.float().abs().max().item()


def test_deterministic_and_inputs_untouched():
    wl = Workload("det", B=4, S_max=20000, Lq=1, seqlens=(20000, 19999, 5000, 3000), Hi=32, Di=128,
                  topk=2048, init=16, local=1024, H=32, mla_calls=2, seed=85)
    X = device_inputs(wl)

    def digest(t):
        return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()

    before = {k: digest(v) for k, v in X.items()}
    r1 = run_path(wl, X)
    torch.cuda.synchronize()
    idx_hash = digest(r1[1])
    r2 = run_path(wl, X)
    torch.cuda.synchronize()
    assert {k: digest(v) for k, v in X.items()} == before, "inputs were modified"
    assert digest(r1[1]) == idx_hash, "indices modified by the attention calls"
    for b, n in enumerate(wl.seqlens):  # scores past the query are never written
        assert torch.equal(r1[0][b, 0, :n].view(torch.int32), r2[0][b, 0, :n].view(torch.int32))
    for a, c in zip([r1[1], r1[2]] + r1[3] + r1[4], [r2[1], r2[2]] + r2[3] + r2[4]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32))


def test_unnormal_index_inputs_scores_close():
    """Unit-variance (non-dyadic) index inputs: fp32 accumulation differs from the oracle's
    fp64 only by rounding; scores agree to a relative 1e-5 of the row's largest score."""
    wl = Workload("normal_idx", B=2, S_max=4096, Lq=1, seqlens=(4096, 1000), Hi=32, Di=128,
                  topk=256, init=4, local=64, seed=86)
    gpu_q = gen.device_tensor(wl.seed, 21, (wl.B, 1, wl.Hi, wl.Di), gen.NORMAL)
    gpu_k = gen.device_tensor(wl.seed, 22, (wl.B, wl.S_max, wl.Di), gen.NORMAL)
    w = gen.device_tensor(wl.seed, 23, (wl.B, 1, wl.Hi), gen.WEIGHT)
    sl = torch.tensor(wl.seqlens, dtype=torch.int32, device="cuda")
    sc = lsa.lsa_index_scores(gpu_q, w, gpu_k, sl)
    torch.cuda.synchronize()
    q = gen.host_tensor(wl.seed, 21, (wl.B, 1, wl.Hi, wl.Di), gen.NORMAL)
    k = gen.host_tensor(wl.seed, 22, (wl.B, wl.S_max, wl.Di), gen.NORMAL)
    wh = gen.host_tensor(wl.seed, 23, (wl.B, 1, wl.Hi), gen.WEIGHT)
    ref = oracle.index_scores(q, wh, k, np.array(wl.seqlens, np.int32), 1)
    for b in range(wl.B):
        n = wl.seqlens[b]
        got = sc[b, 0, :n].cpu().numpy().astype(np.float64)
        want = ref[b, 0, :n].astype(np.float64)
        assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


def test_workspace_too_small_is_rejected_before_launch():
    wl = dataclasses.replace(SMALL[4])
    X = device_inputs(wl)
    sc = lsa.lsa_index_scores(X["qidx"], X["w"], X["kidx"], X["seqlens"])
    need = lsa.lsa_topk_workspace_bytes(wl.B, 1, wl.S_max, wl.topk, wl.init, wl.local)
    assert need > 0
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_topk_select(sc, X["seqlens"], wl.topk, wl.init, wl.local, workspace=small)
    assert e.value.status == 4


def test_attention_buffers_without_16_byte_alignment():
    """The attention epilogue writes 16-byte pieces when the destination allows it and falls back
    to 2-byte stores otherwise: a workspace offset by 8 bytes (split partials, decode) and an
    `out` offset by one element (direct rows, prefill) give bit-identical results."""
    wl = Workload("align", B=2, S_max=3000, Lq=1, seqlens=(3000, 2500), Hi=8, Di=128, topk=512,
                  init=4, local=64, H=32, Dqk=576, Dv=512, seed=91)
    X = device_inputs(wl)
    _, idx, nsel, _, _ = run_path(wl, X)
    need = lsa.lsa_mla_workspace_bytes(wl.B, 1, wl.H, wl.Dv, wl.S_max, wl.topk, False)
    assert need > 0  # split partials go through the workspace
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    args = (X["q0"][:, 0], X["kv0"], idx[:, 0], nsel[:, 0], X["seqlens"], wl.Dv, wl.scale)
    ref = lsa.lsa_sparse_mla_decode(*args, workspace=ws[:need])
    odd = lsa.lsa_sparse_mla_decode(*args, workspace=ws[8:8 + need])
    torch.cuda.synchronize()
    assert torch.equal(ref, odd)

    # 512 query rows: one workgroup per row, so the rows go straight to `out`
    wp = Workload("align_p", B=1, S_max=700, Lq=512, seqlens=(700,), Hi=4, Di=32, topk=128, init=2,
                  local=8, H=32, Dqk=576, Dv=512, seed=92)
    Xp = device_inputs(wp)
    _, idxp, nselp, _, _ = run_path(wp, Xp)
    assert lsa.lsa_mla_workspace_bytes(wp.B, wp.Lq, wp.H, wp.Dv, wp.S_max, wp.topk, False) == 0
    refp = lsa.lsa_sparse_mla_prefill(Xp["q0"], Xp["kv0"], idxp, nselp, Xp["seqlens"], wp.Dv, wp.scale)
    n = refp.numel()
    buf = torch.zeros(n + 1, dtype=torch.bfloat16, device="cuda")
    outp = buf[1:].view(refp.shape)
    assert outp.data_ptr() % 16 != 0
    lsa.lsa_sparse_mla_prefill(Xp["q0"], Xp["kv0"], idxp, nselp, Xp["seqlens"], wp.Dv, wp.scale,
                               out=outp)
    torch.cuda.synchronize()
    assert torch.equal(refp, outp)


def test_selection_workspace_at_an_odd_address():
    """The top-k and fused calls place their candidate lists from the workspace's first 256-byte
    boundary: a workspace that starts 3 bytes past one gives the same indices, bit for bit."""
    wl = SMALL[5]  # several top-k chunks per row
    X = device_inputs(wl)
    sc = lsa.lsa_index_scores(X["qidx"], X["w"], X["kidx"], X["seqlens"])
    for query, call in (
            (lsa.lsa_topk_workspace_bytes,
             lambda ws: lsa.lsa_topk_select(sc, X["seqlens"], wl.topk, wl.init, wl.local,
                                            workspace=ws)),
            (lsa.lsa_index_topk_workspace_bytes,
             lambda ws: lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk,
                                           wl.init, wl.local, workspace=ws))):
        need = query(wl.B, wl.Lq, wl.S_max, wl.topk, wl.init, wl.local)
        buf = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
        ref_idx, ref_n = call(buf[:need])
        odd_idx, odd_n = call(buf[3:3 + need])
        torch.cuda.synchronize()
        assert torch.equal(ref_idx, odd_idx) and torch.equal(ref_n, odd_n)


def test_prefill_rows_equal_decode_calls():
    """Row i of a prefill chunk (query-blocked scan, Di = 128) selects exactly what a decode call
    at seqlen p + 1 selects for the same query, and its attention agrees within tolerance (the
    two calls split the work differently)."""
    wl = Workload("pd", B=1, S_max=3000, Lq=20, seqlens=(3000,), Hi=8, Di=128, topk=256, init=4,
                  local=32, H=4, Dqk=576, Dv=512, seed=95)
    X = device_inputs(wl)
    _, idx, nsel, outs, _ = run_path(wl, X)
    torch.cuda.synchronize()
    for i in range(wl.Lq):
        p = wl.seqlens[0] - wl.Lq + i
        sl = torch.tensor([p + 1], dtype=torch.int32, device="cuda")
        di, dn = lsa.lsa_index_topk(X["qidx"][:, i:i + 1].contiguous(), X["w"][:, i:i + 1].contiguous(),
                                    X["kidx"], sl, wl.topk, wl.init, wl.local)
        out = lsa.lsa_sparse_mla_decode(X["q0"][:, i].contiguous(), X["kv0"], di[:, 0], dn[:, 0], sl,
                                        wl.Dv, wl.scale)
        torch.cuda.synchronize()
        assert int(dn[0, 0]) == int(nsel[0, i])
        assert torch.equal(di[0, 0], idx[0, i]), f"row {i}"
        assert_attention_close(bf16_to_f64(out[0]), bf16_to_f64(outs[0][0, i]), f"row {i}")


def test_attention_workspace_reused_across_calls():
    """One attention workspace, holding the previous call's partials, serves calls of different
    shapes in a row (split and dense, 32 and 40 heads): every call equals the same call on a
    fresh workspace, bit for bit."""
    big = Workload("reuse_big", B=8, S_max=5000, Lq=1, seqlens=(5000, 4000, 3000, 2100, 5000, 4999,
                                                            2500, 4097), Hi=8, Di=64, topk=1024,
                   init=16, local=256, H=32, Dqk=576, Dv=512, seed=98)
    small = Workload("reuse_small", B=3, S_max=3000, Lq=1, seqlens=(3000, 2000, 2600), Hi=8, Di=64,
                     topk=512, init=4, local=64, H=40, Dqk=576, Dv=512, seed=99)
    cases = []
    for wl in (big, small):
        X = device_inputs(wl)
        _, idx, nsel, _, _ = run_path(wl, X)
        cases.append((wl, X, idx, nsel))
    need = max(lsa.lsa_mla_workspace_bytes(wl.B, 1, wl.H, wl.Dv, wl.S_max, wl.topk, dense)
               for wl, _, _, _ in cases for dense in (False, True))
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for wl, X, idx, nsel in cases:
            for dense in (False, True):
                print(f"case reuse {wl.name} dense={dense} round {rnd}", flush=True)
                args = (X["q0"][:, 0], X["kv0"], None if dense else idx[:, 0],
                        None if dense else nsel[:, 0], X["seqlens"], wl.Dv, wl.scale)
                lse_a = torch.empty(wl.B, wl.H, dtype=torch.float32, device="cuda")
                lse_b = torch.empty_like(lse_a)
                a = lsa.lsa_sparse_mla_decode(*args, lse=lse_a, workspace=ws)
                b = lsa.lsa_sparse_mla_decode(*args, lse=lse_b)  # a fresh workspace
                torch.cuda.synchronize()
                assert torch.equal(a, b) and torch.equal(lse_a, lse_b), (wl.name, dense)
