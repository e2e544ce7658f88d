"""GPU multi-token-prediction draft attention (lsa_mtp_draft_attention) against the oracle: a
shared index pass (seeded synthetic selections with the sink and window a pass forces) and the
positions appended since, for draft steps 0..3; outputs and lse within the attention tolerance.
Also: with nothing appended it equals lsa_sparse_mla_decode bit for bit; the max_appended clamp;
a plan where the appended positions need a second split (sampled rows)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import inputs as gen
from long_context_sparse_lightning_amd import lsa
from lsa_check import LSE_ABS, assert_attention_close

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    B: int
    H: int
    Dqk: int
    Dv: int
    S_max: int
    topk: int
    S0: int
    seed: int
    sample: int = 0  # rows compared against the oracle (0: all)


CASES = [
    Case("decode_shape", 8, 32, 576, 512, 8256, 2048, 8000, 601),
    Case("ragged_heads", 5, 40, 80, 64, 600, 64, 500, 602),
    Case("one_row", 1, 32, 576, 512, 4200, 2048, 4100, 603),
    # 512 rows of one split of 2048: the appended positions push the plan to two splits
    Case("split_growth", 512, 32, 80, 64, 4200, 2048, 4100, 604, sample=12),
]


def shared_pass(c: Case, rng):
    """Per sequence: an ascending selection of [0, S0) with the sink (16) and window (64 or
    fewer) positions and random middle ones; n_sel = topk, except a short row (dense-like)."""
    idx = np.full((c.B, c.topk), -1, np.int32)
    nsel = np.zeros(c.B, np.int32)
    for b in range(c.B):
        n = c.topk if b % 4 != 3 else min(c.topk, c.S0) // 2
        forced = set(range(min(16, n // 4))) | set(range(c.S0 - min(64, n // 4), c.S0))
        middle = rng.choice(np.setdiff1d(np.arange(c.S0), list(forced)), n - len(forced),
                            replace=False)
        sel = np.sort(np.concatenate([np.array(sorted(forced), np.int64), middle]))
        idx[b, :n] = sel
        nsel[b] = n
    return idx, nsel


def make(c: Case):
    t = lambda name, shape: gen.device_tensor(c.seed, gen.TAGS[name], shape, gen.NORMAL, device="cuda")
    q = t("q", (c.B, c.H, c.Dqk))
    kv = t("kv0", (c.B, c.S_max, c.Dqk))
    idx, nsel = shared_pass(c, np.random.default_rng(c.seed))
    return q, kv, idx, nsel


def bits(x):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def compare(c, q, kv, idx, nsel, iseq, seq, app, out, lse, what):
    rows = np.arange(c.B) if not c.sample else np.unique(
        np.r_[0, c.B - 1, np.random.default_rng(c.seed + 1).integers(0, c.B, c.sample)])
    scale = 1.0 / np.sqrt(192.0)
    r_out, r_lse = oracle.mtp_draft_attention(bits(q)[rows], bits(kv)[rows], idx[rows], nsel[rows],
                                              iseq[rows], seq[rows], app, c.Dv, scale)
    assert_attention_close(out.float().cpu().numpy()[rows], r_out, what)
    assert np.max(np.abs(lse.cpu().numpy()[rows] - r_lse)) <= LSE_ABS, what


@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_draft_steps_match_oracle(c):
    q, kv, idx, nsel = make(c)
    d_idx, d_nsel = torch.from_numpy(idx).cuda(), torch.from_numpy(nsel).cuda()
    iseq = np.full(c.B, c.S0, np.int32)
    d_iseq = torch.from_numpy(iseq).cuda()
    scale = 1.0 / np.sqrt(192.0)
    for j in range(4):  # draft step j: j positions appended since the pass
        seq = iseq + j
        lse = torch.empty(c.B, c.H, dtype=torch.float32, device="cuda")
        out = lsa.lsa_mtp_draft_attention(q, kv, d_idx, d_nsel, d_iseq, torch.from_numpy(seq).cuda(),
                                          c.Dv, scale, max_appended=3, lse=lse)
        torch.cuda.synchronize()
        compare(c, q, kv, idx, nsel, iseq, seq, 3, out, lse, f"{c.name} step {j}")


def test_largest_selection_and_most_appended():
    """The largest pass the draft call takes (topk = 65536) with the most appended positions
    (max_appended = 64): draft steps with 0, 1 and 64 positions appended, and 70 (clamped to
    64), against the oracle.  The appended positions ride in the last split, which stays within
    its LDS slice."""
    c = Case("max_selection", 2, 4, 576, 512, 65700, 65536, 65600, 605)
    q, kv, idx, nsel = make(c)
    d_idx, d_nsel = torch.from_numpy(idx).cuda(), torch.from_numpy(nsel).cuda()
    iseq = np.full(c.B, c.S0, np.int32)
    d_iseq = torch.from_numpy(iseq).cuda()
    scale = 1.0 / np.sqrt(192.0)
    for j in (0, 1, 64, 70):
        print(f"case draft topk=65536 appended={j}", flush=True)
        seq = iseq + j
        lse = torch.empty(c.B, c.H, dtype=torch.float32, device="cuda")
        out = lsa.lsa_mtp_draft_attention(q, kv, d_idx, d_nsel, d_iseq, torch.from_numpy(seq).cuda(),
                                          c.Dv, scale, max_appended=64, lse=lse)
        torch.cuda.synchronize()
        compare(c, q, kv, idx, nsel, iseq, seq, 64, out, lse, f"max selection, {j} appended")


def test_nothing_appended_equals_decode():
    c = CASES[0]
    q, kv, idx, nsel = make(c)
    d_idx, d_nsel = torch.from_numpy(idx).cuda(), torch.from_numpy(nsel).cuda()
    seq = torch.full((c.B,), c.S0, dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(192.0)
    a = lsa.lsa_mtp_draft_attention(q, kv, d_idx, d_nsel, seq, seq, c.Dv, scale, max_appended=3)
    b = lsa.lsa_sparse_mla_decode(q, kv, d_idx, d_nsel, seq, c.Dv, scale)
    z = lsa.lsa_mtp_draft_attention(q, kv, d_idx, d_nsel, seq - 2, seq, c.Dv, scale, max_appended=0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(z, b)


def test_appended_beyond_the_maximum_are_not_attended():
    c = CASES[1]
    q, kv, idx, nsel = make(c)
    iseq = np.full(c.B, c.S0, np.int32)
    iseq[1] = c.S0 + 9  # a pass "after" the query: nothing appended
    seq = np.full(c.B, c.S0 + 5, np.int32)
    lse = torch.empty(c.B, c.H, dtype=torch.float32, device="cuda")
    out = lsa.lsa_mtp_draft_attention(q, kv, torch.from_numpy(idx).cuda(), torch.from_numpy(nsel).cuda(),
                                      torch.from_numpy(iseq).cuda(), torch.from_numpy(seq).cuda(),
                                      c.Dv, 1.0 / np.sqrt(192.0), max_appended=2, lse=lse)
    torch.cuda.synchronize()
    compare(c, q, kv, idx, nsel, iseq, seq, 2, out, lse, "clamp")


def test_dense_pass_then_drafts_is_dense_attention():
    """A sequence shorter than topk: the index pass keeps every position, so each draft step's
    selection is every position up to its own, i.e. dense attention (oracle, indices = None)."""
    B, H, Dqk, Dv, S_max, topk, S0 = 3, 32, 576, 512, 3000, 2048, 1500
    t = lambda name, shape: gen.device_tensor(611, gen.TAGS[name], shape, gen.NORMAL, device="cuda")
    q, kv = t("q", (B, H, Dqk)), t("kv0", (B, S_max, Dqk))
    idx = torch.full((B, topk), -1, dtype=torch.int32)
    idx[:, :S0] = torch.arange(S0, dtype=torch.int32)
    idx, nsel = idx.cuda(), torch.full((B,), S0, dtype=torch.int32, device="cuda")
    iseq = torch.full((B,), S0, dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(192.0)
    for j in range(3):
        seq = iseq + j
        lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
        out = lsa.lsa_mtp_draft_attention(q, kv, idx, nsel, iseq, seq, Dv, scale, max_appended=3, lse=lse)
        torch.cuda.synchronize()
        r_out, r_lse = oracle.sparse_mla(bits(q)[:, None], bits(kv), None, None, seq.cpu().numpy(), Dv, scale)
        assert_attention_close(out.float().cpu().numpy(), r_out[:, 0], f"dense draft {j}")
        assert np.max(np.abs(lse.cpu().numpy() - r_lse[:, 0])) <= LSE_ABS
