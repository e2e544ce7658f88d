"""Pins of the oracle's hierarchical indexing (block scores, then the token selection inside
the kept blocks; page "LongCat Sparse Attention技术深度解析", "分层索引"): against the exact
selection when every block is kept, a brute force written with Python loops and exact
fractions on small inputs, and the dense fallback.  Parity against the pages is unpinned: they
give no block size and no block score (the readings are in the oracle's header)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from long_context_sparse_lightning_amd import inputs as gen


def dyadic(rng, shape):
    return gen.f32_to_bf16_bits(rng.integers(-3, 4, size=shape).astype(np.float32) / 4.0)


def make(seed, B, S, Hi, Di):
    rng = np.random.default_rng(seed)
    q = dyadic(rng, (B, Hi, Di))
    w = ((rng.integers(0, 4, size=(B, Hi)) + 1) / 8.0).astype(np.float32)
    k = dyadic(rng, (B, S, Di))
    return q, w, k


def test_every_block_kept_is_the_exact_selection():
    B, S, Hi, Di, topk, init, local, Bk = 3, 300, 4, 16, 40, 3, 10, 8
    q, w, k = make(41, B, S, Hi, Di)
    seq = np.array([300, 257, 41], np.int32)
    got, gn = oracle.hier_topk(q, w, k, seq, topk, init, local, Bk, M=S // Bk)
    sc = oracle.index_scores(q[:, None], w[:, None], k, seq, 1)
    want, wn = oracle.topk_select(sc, seq, topk, init, local)
    assert np.array_equal(gn, wn[:, 0]) and np.array_equal(got, want[:, 0])


def brute(q, w, k, p, topk, init, local, Bk, M):
    """One row by the reading, with exact fractions for the block means and plain sorting."""
    Hi, Di = q.shape
    val = lambda bits: [Fraction(float(x)) for x in gen.as_bf16_f64(bits)]
    qv = [val(q[h]) for h in range(Hi)]
    wv = [Fraction(float(x)) for x in w]

    def score(key):
        tot = sum(wv[h] * max(Fraction(0), sum(a * b for a, b in zip(qv[h], key))) for h in range(Hi))
        return float(np.float32(float(tot)))

    n = p + 1
    if n <= topk:
        return list(range(n))
    w0 = max(p - local + 1, 0)
    nb = w0 // Bk
    blocks = []
    for j in range(nb):
        mean = [sum(val(k[j * Bk + t])[d] for t in range(Bk)) / Bk for d in range(Di)]
        key = [Fraction(float(x)) for x in gen.as_bf16_f64(gen.f32_to_bf16_bits(
            np.array([float(m) for m in mean], np.float32)))]
        blocks.append((-score(key), j))
    kept = {j for _, j in sorted(blocks)[:M]}
    ranked = []
    for s in range(n):
        if s < init or s > p - local:
            key = float("inf")
        elif s >= nb * Bk or s // Bk in kept:
            key = score(val(k[s]))
        else:
            key = float("-inf")
        ranked.append((-key, s))
    return sorted(s for _, s in sorted(ranked)[:topk])


@pytest.mark.parametrize("M", [1, 3, 6])
def test_brute_force(M):
    B, S, Hi, Di, topk, init, local, Bk = 2, 64, 2, 4, 12, 2, 4, 4
    q, w, k = make(42 + M, B, S, Hi, Di)
    seq = np.array([64, 40], np.int32)
    got, gn = oracle.hier_topk(q, w, k, seq, topk, init, local, Bk, M)
    for b in range(B):
        want = brute(q[b], w[b], k[b], int(seq[b]) - 1, topk, init, local, Bk, M)
        assert gn[b] == len(want) and got[b, :gn[b]].tolist() == want, (M, b)


def test_dense_fallback_and_block_means():
    q, w, k = make(43, 1, 64, 2, 4)
    got, gn = oracle.hier_topk(q, w, k, np.array([12], np.int32), 12, 2, 4, 4, 1)
    assert gn[0] == 12 and got[0].tolist() == list(range(12))
    # a block whose keys are all equal has that key as its mean: keeping one block out of two
    # with equal-key blocks picks the one whose (shared) token score is higher
    Di = 4
    k = np.zeros((1, 24, Di), np.uint16)
    one = gen.f32_to_bf16_bits(np.array([0.25, 0.5, -0.25, 0.75], np.float32))
    two = gen.f32_to_bf16_bits(np.array([0.5, 0.5, 0.5, 0.5], np.float32))
    k[0, 0:4], k[0, 4:8] = one, two
    q = gen.f32_to_bf16_bits(np.ones((1, 1, Di), np.float32))
    w = np.ones((1, 1), np.float32)
    # p = 23, local 4 -> window from 20, nb = 5 blocks; keep M = 1: block 1 (score 2) beats
    # block 0 (1.25); blocks 2-4 score 0.  topk 8 leaves a middle budget of 4: block 1 exactly
    got, gn = oracle.hier_topk(q, w, k, np.array([24], np.int32), 8, 0, 4, 4, 1)
    assert got[0, :gn[0]].tolist() == [4, 5, 6, 7, 20, 21, 22, 23]
    # a larger budget than the kept tokens: the rest are -inf, taken from the lowest position
    got, gn = oracle.hier_topk(q, w, k, np.array([24], np.int32), 10, 0, 4, 4, 1)
    assert got[0, :gn[0]].tolist() == [0, 1, 4, 5, 6, 7, 20, 21, 22, 23]
