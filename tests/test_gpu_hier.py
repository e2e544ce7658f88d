"""GPU hierarchical indexing (lsa_block_keys, lsa_hier_index_topk) against the oracle on dyadic
index queries and keys (every score and block mean is exact in fp32 and bf16, so selections
compare bit for bit): block keys equal the bf16 block means; selections equal the oracle's for
dense rows, rows whose blocks are all kept, kept blocks holding exactly the middle budget, block
sizes 8 to 1024, a 1M-token context (candidate lists of 16384 positions); with every block kept
the result is lsa_index_topk's; too few kept tokens for the budget is refused."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import inputs as gen
from long_context_sparse_lightning_amd import lsa

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    B: int
    S_max: int
    seqlens: tuple
    Hi: int
    Di: int
    topk: int
    init: int
    local: int
    Bk: int
    M: int
    seed: int


CASES = [
    # rows: long, all blocks kept (nb <= M), dense (n <= topk)
    Case("small", 3, 4096, (4096, 700, 200), 4, 32, 256, 4, 64, 16, 24, 701),
    # M * Bk = topk - local: with block 0 kept, exactly the middle budget of candidates
    Case("exact_fill", 2, 4096, (4096, 3001), 4, 32, 256, 4, 64, 16, 12, 702),
    Case("bk8", 2, 2048, (2048, 1999), 8, 64, 128, 2, 16, 8, 20, 703),
    Case("bk1024", 2, 16384, (16384, 9000), 32, 128, 2048, 16, 1024, 1024, 4, 704),
    Case("decode_32k", 8, 32768, tuple(32768 - 97 * j for j in range(8)), 32, 128, 2048, 16, 1024,
         64, 32, 705),
    Case("context_1m", 2, 1 << 20, (1 << 20, 700001), 32, 128, 2048, 16, 1024, 64, 32, 706),
]


def make(c):
    t = lambda name, shape, kind: gen.device_tensor(c.seed, gen.TAGS[name], shape, kind, device="cuda")
    q = t("qidx", (c.B, c.Hi, c.Di), gen.DYADIC)
    w = t("w", (c.B, c.Hi), gen.WEIGHT)
    k = t("kidx", (c.B, c.S_max, c.Di), gen.DYADIC)
    seq = torch.tensor(c.seqlens, dtype=torch.int32, device="cuda")
    return q, w, k, seq


def bits(x):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("c", CASES[:3], ids=lambda c: c.name)
def test_block_keys_are_bf16_means(c):
    q, w, k, seq = make(c)
    bk = lsa.lsa_block_keys(k, seq, c.Bk)
    torch.cuda.synchronize()
    kv = gen.as_bf16_f64(bits(k))
    for b in range(c.B):
        nb = c.seqlens[b] // c.Bk
        means = kv[b, : nb * c.Bk].reshape(nb, c.Bk, c.Di).mean(axis=1)  # exact: dyadic keys
        assert np.array_equal(bits(bk[b, :nb]), gen.f32_to_bf16_bits(means.astype(np.float32))), b
        assert torch.all(bk[b, nb:] == 0)  # blocks not complete are not written


@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_selection_matches_oracle(c):
    q, w, k, seq = make(c)
    bk = lsa.lsa_block_keys(k, seq, c.Bk)
    idx, nsel = lsa.lsa_hier_index_topk(q, w, k, bk, seq, c.topk, c.init, c.local, c.Bk, c.M)
    torch.cuda.synchronize()
    r_idx, r_nsel = oracle.hier_topk(bits(q), w.cpu().numpy(), bits(k), np.array(c.seqlens, np.int32),
                                     c.topk, c.init, c.local, c.Bk, c.M)
    assert np.array_equal(nsel.cpu().numpy(), r_nsel)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    # deterministic, and the workspace contents on entry do not matter
    ws = torch.full((lsa.lsa_hier_workspace_bytes(c.B, c.S_max, c.Bk, c.topk, c.init, c.local, c.M),),
                    255, dtype=torch.uint8, device="cuda")
    idx2, nsel2 = lsa.lsa_hier_index_topk(q, w, k, bk, seq, c.topk, c.init, c.local, c.Bk, c.M,
                                          workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(nsel, nsel2)


def test_every_block_kept_equals_the_exact_pass():
    c = CASES[4]
    q, w, k, seq = make(c)
    bk = lsa.lsa_block_keys(k, seq, c.Bk)
    idx, nsel = lsa.lsa_hier_index_topk(q, w, k, bk, seq, c.topk, c.init, c.local, c.Bk,
                                        c.S_max // c.Bk)
    e_idx, e_nsel = lsa.lsa_index_topk(q[:, None], w[:, None], k, seq, c.topk, c.init, c.local)
    torch.cuda.synchronize()
    assert torch.equal(nsel, e_nsel[:, 0]) and torch.equal(idx, e_idx[:, 0])


def test_incremental_block_keys():
    """Summarising a growing cache block by block gives the same keys as one pass."""
    c = CASES[0]
    q, w, k, seq = make(c)
    full = lsa.lsa_block_keys(k, seq, c.Bk)
    part = lsa.lsa_block_keys(k, seq - 100, c.Bk)
    part = lsa.lsa_block_keys(k, seq, c.Bk, block_keys=part,
                              first_block=(c.seqlens[2] - 100) // c.Bk)
    torch.cuda.synchronize()
    assert torch.equal(full, part)


def test_too_few_kept_tokens_is_refused():
    c = CASES[0]
    q, w, k, seq = make(c)
    bk = lsa.lsa_block_keys(k, seq, c.Bk)
    with pytest.raises(lsa.LsaError):  # 11 * 16 = 176 < topk - local = 192
        lsa.lsa_hier_index_topk(q, w, k, bk, seq, c.topk, c.init, c.local, c.Bk, 11)


def test_all_scores_tied():
    """Every key equal: every block and token score ties, so the lowest blocks are kept and the
    lowest candidate positions chosen, as in the oracle."""
    c = Case("tied", 3, 8192, (8192, 5000, 3001), 8, 64, 512, 8, 128, 32, 16, 707)
    q, w, _, seq = make(c)
    k = gen.device_tensor(c.seed, gen.TAGS["kidx"], (1, 1, c.Di), gen.DYADIC).expand(
        c.B, c.S_max, c.Di).contiguous()
    bk = lsa.lsa_block_keys(k, seq, c.Bk)
    idx, nsel = lsa.lsa_hier_index_topk(q, w, k, bk, seq, c.topk, c.init, c.local, c.Bk, c.M)
    torch.cuda.synchronize()
    r_idx, r_nsel = oracle.hier_topk(bits(q), w.cpu().numpy(), bits(k), np.array(c.seqlens, np.int32),
                                     c.topk, c.init, c.local, c.Bk, c.M)
    assert np.array_equal(nsel.cpu().numpy(), r_nsel) and np.array_equal(idx.cpu().numpy(), r_idx)
