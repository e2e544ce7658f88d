"""GPU indexer front end (lsa_index_frontend) against the oracle: index queries and new keys
(bf16) within the tolerance used for attention, head weights (fp32) within the worst-case fp32
summation bound, only the current tokens' cache rows written, deterministic.  Shapes: ragged
token counts and output tiles, reduction splits, the decode_128k shape at positions near 2^17,
a 256-token prefill chunk, and the query projection's rotated epilogue (ragged, and a full
4096-token chunk on sampled tokens)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from long_context_sparse_lightning_amd import inputs as gen
from long_context_sparse_lightning_amd import lsa
from lsa_check import assert_attention_close

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@dataclasses.dataclass(frozen=True)
class Case:
    name: str
    B: int
    Lq: int
    seqlens: tuple
    S_max: int
    q_lora: int
    hidden: int
    Hi: int
    Di: int
    R: int
    theta: float = 1e6
    eps: float = 1e-6
    seed: int = 500


CASES = [
    Case("ragged", 3, 5, (20, 7, 300), 512, 64, 96, 5, 64, 32, seed=501),
    Case("tiles", 2, 40, (4096, 1000), 4096, 128, 256, 32, 128, 64, seed=502),
    Case("no_rotation", 2, 3, (9, 64), 64, 32, 48, 3, 32, 0, eps=0.0, seed=503),
    Case("decode_128k", 32, 1, tuple(131072 - 37 * j for j in range(32)), 131072, 1536, 3072, 32,
         128, 64, seed=504),
    Case("prefill_chunk", 1, 256, (131072,), 131072, 1536, 3072, 32, 128, 64, seed=505),
    # no reduction split with LDS tiles: the query projection rotates in its epilogue; ragged
    # token tiles, heads that straddle 32-output blocks
    Case("rotated_epilogue", 2, 150, (150, 4000), 4096, 192, 128, 5, 48, 16, seed=507),
    # the two projections take different tilings (q_lora not a multiple of 64): two launches
    Case("mixed_tiling", 1, 130, (500,), 512, 80, 128, 4, 64, 32, seed=509),
]


def make(c: Case):
    dev = "cuda"
    T = (c.B, c.Lq)
    t = lambda name, shape, kind: gen.device_tensor(c.seed, gen.TAGS[name], shape, kind, device=dev)
    X = {"cq": t("cq", T + (c.q_lora,), gen.NORMAL), "hid": t("hid", T + (c.hidden,), gen.NORMAL),
         "wq_b": t("wq_b", (c.Hi * c.Di, c.q_lora), gen.NORMAL),
         "wk": t("wk", (c.Di, c.hidden), gen.NORMAL),
         "w_proj": t("w_proj", (c.Hi, c.hidden), gen.NORMAL),
         "k_gain": t("k_gain", (c.Di,), gen.WEIGHT),
         "seqlens": torch.tensor(c.seqlens, dtype=torch.int32, device=dev)}
    return X


def bits(x):
    return x.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("c", CASES, ids=lambda c: c.name)
def test_frontend_matches_oracle(c):
    X = make(c)
    cache = torch.full((c.B, c.S_max, c.Di), 1.5, dtype=torch.bfloat16, device="cuda")
    q, w = lsa.lsa_index_frontend(X["cq"], X["hid"], X["wq_b"], X["wk"], X["k_gain"], X["w_proj"],
                                  X["seqlens"], cache, rope_dim=c.R, rope_theta=c.theta,
                                  norm_eps=c.eps)
    torch.cuda.synchronize()
    rq, rw, rk = oracle.index_frontend(bits(X["cq"]), bits(X["hid"]), bits(X["wq_b"]), bits(X["wk"]),
                                       X["k_gain"].cpu().numpy(), bits(X["w_proj"]),
                                       np.array(c.seqlens, np.int32), c.Hi, c.Di, c.R, c.theta, c.eps)
    assert_attention_close(q.float().cpu().numpy(), rq, f"{c.name} q_idx")
    # head weights: fp32 sums of exact bf16 products; any order stays within gamma_K * sum|a w|
    hid = gen.as_bf16_f64(bits(X["hid"]))
    wp = gen.as_bf16_f64(bits(X["w_proj"]))
    mag = np.einsum("blj,hj->blh", np.abs(hid), np.abs(wp))
    u = 2.0 ** -24
    gam = c.hidden * u / (1 - c.hidden * u)
    assert np.all(np.abs(w.cpu().numpy().astype(np.float64) - rw) <= gam * mag + 1e-30)
    # keys: written at each token's position, every other row untouched
    pos = [(b, c.seqlens[b] - c.Lq + i) for b in range(c.B) for i in range(c.Lq)]
    got_k = np.stack([cache[b, p].float().cpu().numpy() for b, p in pos]).reshape(c.B, c.Lq, c.Di)
    assert_attention_close(got_k, rk, f"{c.name} k")
    if c.S_max * c.B <= 1 << 16:
        mask = torch.ones(c.B, c.S_max, dtype=torch.bool)
        for b, p in pos:
            mask[b, p] = False
        assert torch.all(cache.cpu()[mask] == 1.5)
    # deterministic
    q2, w2 = lsa.lsa_index_frontend(X["cq"], X["hid"], X["wq_b"], X["wk"], X["k_gain"],
                                    X["w_proj"], X["seqlens"], cache.clone(), rope_dim=c.R,
                                    rope_theta=c.theta, norm_eps=c.eps)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(w, w2)


def test_frontend_prefill_4096_sampled():
    """A 4096-token prefill chunk at 128K (the query projection's rotated epilogue, full-size
    weights): sampled tokens against the oracle, each evaluated as a one-token sequence at the
    same position; tile edges and the first and last tokens included."""
    c = Case("prefill_4096", 1, 4096, (131072,), 131072, 1536, 3072, 32, 128, 64, seed=508)
    X = make(c)
    cache = torch.zeros(c.B, c.S_max, c.Di, dtype=torch.bfloat16, device="cuda")
    q, w = lsa.lsa_index_frontend(X["cq"], X["hid"], X["wq_b"], X["wk"], X["k_gain"], X["w_proj"],
                                  X["seqlens"], cache, rope_dim=c.R, rope_theta=c.theta,
                                  norm_eps=c.eps)
    torch.cuda.synchronize()
    rng = np.random.default_rng(c.seed)
    toks = sorted(set([0, 1, 127, 128, 129, 2047, 2048, 4094, 4095]) |
                  set(rng.integers(0, c.Lq, 23).tolist()))
    pos = [c.seqlens[0] - c.Lq + i for i in toks]
    sel = lambda x: x[0, toks].unsqueeze(1)  # [n, 1, ...]: one-token sequences
    rq, rw, rk = oracle.index_frontend(bits(sel(X["cq"])), bits(sel(X["hid"])), bits(X["wq_b"]),
                                       bits(X["wk"]), X["k_gain"].cpu().numpy(), bits(X["w_proj"]),
                                       np.array([p + 1 for p in pos], np.int32), c.Hi, c.Di, c.R,
                                       c.theta, c.eps)
    assert_attention_close(sel(q).float().cpu().numpy(), rq, "prefill_4096 q_idx")
    hid = gen.as_bf16_f64(bits(sel(X["hid"])))
    mag = np.einsum("blj,hj->blh", np.abs(hid), np.abs(gen.as_bf16_f64(bits(X["w_proj"]))))
    gam = c.hidden * 2.0 ** -24 / (1 - c.hidden * 2.0 ** -24)
    assert np.all(np.abs(sel(w).cpu().numpy().astype(np.float64) - rw) <= gam * mag + 1e-30)
    got_k = cache[0, pos].float().cpu().numpy().reshape(len(toks), 1, c.Di)
    assert_attention_close(got_k, rk, "prefill_4096 k")


def test_frontend_feeds_the_indexer():
    """The front end's outputs are the indexer's inputs: scoring the cache it wrote gives the
    oracle's scores of the oracle's own front-end outputs (rounded to bf16 the same way) within
    the score tolerance of non-dyadic inputs."""
    c = Case("chain", 2, 1, (300, 257), 512, 64, 96, 4, 32, 16, seed=506)
    X = make(c)
    # a cache of earlier keys, plus the rows the front end writes
    cache = gen.device_tensor(c.seed, gen.TAGS["kidx"], (c.B, c.S_max, c.Di), gen.NORMAL)
    q, w = lsa.lsa_index_frontend(X["cq"], X["hid"], X["wq_b"], X["wk"], X["k_gain"], X["w_proj"],
                                  X["seqlens"], cache, rope_dim=c.R, rope_theta=c.theta,
                                  norm_eps=c.eps)
    sc = lsa.lsa_index_scores(q, w, cache, X["seqlens"])
    torch.cuda.synchronize()
    ref = oracle.index_scores(bits(q), w.cpu().numpy(), bits(cache), np.array(c.seqlens, np.int32), 1)
    for b in range(c.B):
        n = c.seqlens[b]
        got = sc[b, 0, :n].cpu().numpy().astype(np.float64)
        want = ref[b, 0, :n].astype(np.float64)
        assert np.max(np.abs(got - want)) <= 1e-5 * max(np.max(np.abs(want)), 1.0)
