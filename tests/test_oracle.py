"""Pins for the CPU oracle: each check is something other than the oracle itself (exact integer
arithmetic, NumPy brute force in a different formulation, a hand-worked fixture, closed forms
and invariants), chosen so that a dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them."""
import json
import os

import numpy as np
import pytest

import oracle
from long_context_sparse_lightning_amd import inputs as gen


def _dyadic(seed, tag, shape):
    return gen.ref_tensor(seed, tag, shape, gen.DYADIC)


def _weights(seed, tag, shape):
    return gen.ref_tensor(seed, tag, shape, gen.WEIGHT)


def _normal(seed, tag, shape):
    return gen.ref_tensor(seed, tag, shape, gen.NORMAL)


def _vals(bits):
    return gen.as_bf16_f64(bits)


# ------------------------------------------------------------------------------ indexer scores
@pytest.mark.parametrize("B,Lq,Hi,Di,S,seqlens", [
    (2, 1, 4, 32, 96, [96, 57]),
    (1, 5, 3, 16, 40, [40]),
    (3, 2, 8, 32, 33, [2, 33, 17]),
])
def test_scores_exact_integer_bruteforce(B, Lq, Hi, Di, S, seqlens):
    """Dyadic inputs scaled to integers: q*4, k*4 and w*8 are integers, so 128*score is an
    integer computed exactly with int64 matmuls (no float rounding anywhere)."""
    seed = 11
    q = _dyadic(seed, 1, (B, Lq, Hi, Di))
    k = _dyadic(seed, 3, (B, S, Di))
    w = _weights(seed, 2, (B, Lq, Hi))
    sl = np.array(seqlens, dtype=np.int32)
    got = oracle.index_scores(q, w, k, sl, Lq)

    qi = np.rint(_vals(q) * 4).astype(np.int64)
    ki = np.rint(_vals(k) * 4).astype(np.int64)
    wi = np.rint(w.astype(np.float64) * 8).astype(np.int64)
    for b in range(B):
        for i in range(Lq):
            p = sl[b] - Lq + i
            g = qi[b, i] @ ki[b, : p + 1].T                       # [Hi, p+1] int64
            s_int = (wi[b, i][:, None] * np.maximum(g, 0)).sum(0)  # units of 2^-7
            want = s_int.astype(np.float64) / 128.0
            np.testing.assert_array_equal(got[b, i, : p + 1].astype(np.float64), want)
            assert np.isnan(got[b, i, p + 1:]).all(), "positions after the query must stay unwritten"


def test_scores_single_head_is_relu_dot():
    """Hi = 1, w = 1 reduces the score to max(0, q.k), a plain dot product."""
    q = _dyadic(5, 1, (1, 1, 1, 64))
    k = _dyadic(5, 3, (1, 300, 64))
    w = np.ones((1, 1, 1), np.float32)
    got = oracle.index_scores(q, w, k, np.array([300], np.int32), 1)[0, 0]
    want = np.maximum(_vals(k[0]) @ _vals(q[0, 0, 0]), 0.0)
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_scores_nonpositive_dots_give_zero():
    """If every q.k is <= 0 the ReLU removes every term: all scores are exactly 0."""
    k = np.abs(_vals(_dyadic(6, 3, (1, 50, 32))))
    q = -np.abs(_vals(_dyadic(6, 1, (1, 1, 4, 32))))
    kb = gen.f32_to_bf16_bits(k.astype(np.float32))
    qb = gen.f32_to_bf16_bits(q.astype(np.float32))
    w = _weights(6, 2, (1, 1, 4))
    got = oracle.index_scores(qb, w, kb, np.array([50], np.int32), 1)
    assert (got[0, 0] == 0.0).all()


def test_scores_weight_sign_and_head_sum():
    """Scores are linear in w per head: a negative weight subtracts that head's ReLU term."""
    q = _dyadic(7, 1, (1, 1, 2, 32))
    k = _dyadic(7, 3, (1, 64, 32))
    sl = np.array([64], np.int32)
    e0 = oracle.index_scores(q, np.array([[[1.0, 0.0]]], np.float32), k, sl, 1)
    e1 = oracle.index_scores(q, np.array([[[0.0, 1.0]]], np.float32), k, sl, 1)
    mixw = oracle.index_scores(q, np.array([[[0.5, -2.0]]], np.float32), k, sl, 1)
    np.testing.assert_array_equal(mixw, (0.5 * e0.astype(np.float64) - 2.0 * e1).astype(np.float32))


# ------------------------------------------------------------------------------ top-k
def _bruteforce_topk(row, n, topk, init, local):
    """Independent formulation: NumPy lexsort on (position asc) within (key desc)."""
    p = n - 1
    if n <= topk:
        return np.arange(n)
    pos = np.arange(n)
    key = row[:n].astype(np.float64).copy()
    key[(pos < init) | (pos >= p - local + 1)] = np.inf
    order = np.lexsort((pos, -key))
    return np.sort(order[:topk])


def test_topk_golden_fixture(golden_dir):
    with open(os.path.join(golden_dir, "topk_tiny_p1_constants.json")) as f:
        g = json.load(f)
    scores = np.array(g["scores"], dtype=np.float32)
    S = scores.size
    for case in g["cases"]:
        sl = np.array([case["seqlen"]], np.int32)
        idx, nsel = oracle.topk_select(scores[None, None, :], sl, g["topk"], g["init_tokens"],
                                       g["local_tokens"])
        assert idx[0, 0].tolist() == case["indices"], case["why"]
        assert nsel[0, 0] == case["n_sel"]
    assert S == 14


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_lexsort_bruteforce(seed):
    rng = np.random.default_rng(seed)
    topk = int(rng.choice([8, 16, 32]))
    init = int(rng.integers(0, topk // 2 + 1))
    local = int(rng.integers(0, topk - init + 1))
    S = int(rng.integers(1, 120))
    Lq = int(rng.integers(1, 4))
    B = 2
    # few distinct values -> many ties, plus zeros and negative weights' negative scores
    scores = rng.integers(-3, 5, size=(B, Lq, S)).astype(np.float32) * np.float32(0.5)
    sl = rng.integers(Lq, S + 1, size=B).astype(np.int32)
    idx, nsel = oracle.topk_select(scores, sl, topk, init, local)
    for b in range(B):
        for i in range(Lq):
            n = sl[b] - Lq + i + 1
            want = _bruteforce_topk(scores[b, i], n, topk, init, local)
            assert nsel[b, i] == len(want)
            assert idx[b, i, : len(want)].tolist() == want.tolist()
            assert (idx[b, i, len(want):] == -1).all()


def test_topk_invariants_large_row():
    rng = np.random.default_rng(3)
    topk, init, local = 256, 4, 64
    S = 4096
    scores = (rng.integers(0, 64, size=(1, 1, S)) * 0.125).astype(np.float32)
    for n in (200, 256, 257, 1000, 4096):
        idx, nsel = oracle.topk_select(scores, np.array([n], np.int32), topk, init, local)
        sel = idx[0, 0, : nsel[0, 0]]
        assert nsel[0, 0] == min(n, topk)
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < n
        if n <= topk:
            continue
        p = n - 1
        forced = np.r_[np.arange(init), np.arange(p - local + 1, n)]
        assert np.isin(forced, sel).all()
        middle = np.arange(init, p - local + 1)
        chosen = np.isin(middle, sel)
        s_mid = scores[0, 0, middle]
        thr = s_mid[chosen].min()
        assert thr >= s_mid[~chosen].max()
        tied_in = middle[chosen & (s_mid == thr)]
        tied_out = middle[~chosen & (s_mid == thr)]
        if tied_out.size:
            assert tied_in.max() < tied_out.min(), "ties must go to the lowest positions"


def test_topk_rejects_forced_overflow():
    with pytest.raises(ValueError):
        oracle.topk_select(np.zeros((1, 1, 32), np.float32), np.array([32], np.int32), 8, 5, 4)


def test_topk_equal_scores_take_lowest_positions():
    scores = np.zeros((1, 1, 100), np.float32)
    idx, nsel = oracle.topk_select(scores, np.array([100], np.int32), 16, 2, 4)
    assert idx[0, 0].tolist() == list(range(12)) + [96, 97, 98, 99]


# ------------------------------------------------------------------------------ attention
def _dense_masked_reference(qv, kvv, mask, scale, Dv):
    """Independent formulation: full-length logits with -inf outside the mask, softmax by
    NumPy over the whole cache length (the prefill mask form)."""
    logits = scale * (qv @ kvv.T)                                  # [H, S]
    logits = np.where(mask[None, :], logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    out = (e / z) @ kvv[:, :Dv]
    lse = (m + np.log(z))[:, 0]
    return out, lse


@pytest.mark.parametrize("B,Lq,H,Dqk,Dv,S,topk", [
    (2, 1, 4, 80, 64, 50, 16),
    (1, 4, 3, 24, 16, 40, 8),
    (2, 3, 2, 40, 32, 64, 64),
])
def test_attention_matches_dense_masked_softmax(B, Lq, H, Dqk, Dv, S, topk):
    rng = np.random.default_rng(B * 100 + Lq)
    q = _normal(21, 4, (B, Lq, H, Dqk))
    kv = _normal(21, 5, (B, S, Dqk))
    sl = rng.integers(Lq, S + 1, size=B).astype(np.int32)
    scale = 1.0 / np.sqrt(Dqk)
    idx = np.full((B, Lq, topk), -1, np.int32)
    nsel = np.zeros((B, Lq), np.int32)
    for b in range(B):
        for i in range(Lq):
            p = sl[b] - Lq + i
            c = min(topk, p + 1)
            pick = np.sort(rng.choice(p + 1, size=c, replace=False))
            idx[b, i, :c] = pick
            nsel[b, i] = c
    out, lse = oracle.sparse_mla(q, kv, idx, nsel, sl, Dv, scale)
    outd, lsed = oracle.sparse_mla(q, kv, None, None, sl, Dv, scale)
    qv, kvv = _vals(q), _vals(kv)
    for b in range(B):
        for i in range(Lq):
            p = sl[b] - Lq + i
            mask = np.zeros(S, bool)
            mask[idx[b, i, : nsel[b, i]]] = True
            want, wl = _dense_masked_reference(qv[b, i], kvv[b], mask, scale, Dv)
            np.testing.assert_allclose(out[b, i], want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, i], wl, rtol=1e-12)
            causal = np.arange(S) <= p
            want, wl = _dense_masked_reference(qv[b, i], kvv[b], causal, scale, Dv)
            np.testing.assert_allclose(outd[b, i], want, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lsed[b, i], wl, rtol=1e-12)


def test_attention_two_keys_closed_form():
    """Two selected rows: the weights are a logistic function of the logit difference."""
    q = _normal(3, 4, (1, 1, 2, 16))
    kv = _normal(3, 5, (1, 10, 16))
    idx = np.array([[[2, 7]]], np.int32)
    out, lse = oracle.sparse_mla(q, kv, idx, np.array([[2]], np.int32), np.array([10], np.int32),
                                 8, 0.5)
    qv, kvv = _vals(q)[0, 0], _vals(kv)[0]
    for h in range(2):
        d = 0.5 * (qv[h] @ (kvv[2] - kvv[7]))
        a = 1.0 / (1.0 + np.exp(-d))
        np.testing.assert_allclose(out[0, 0, h], a * kvv[2, :8] + (1 - a) * kvv[7, :8], rtol=1e-12,
                                   atol=1e-14)
        l2, l7 = 0.5 * qv[h] @ kvv[2], 0.5 * qv[h] @ kvv[7]
        np.testing.assert_allclose(lse[0, 0, h], np.logaddexp(l2, l7), rtol=1e-13)


def test_attention_special_cases():
    S, Dqk, Dv, H = 30, 24, 16, 3
    q = _normal(8, 4, (1, 1, H, Dqk))
    kv = _normal(8, 5, (1, S, Dqk))
    sl = np.array([S], np.int32)
    idx = np.array([[[1, 4, 9, 16, 25, 29]]], np.int32)
    nsel = np.array([[6]], np.int32)
    # identical rows -> output is that row's value vector
    same = np.repeat(kv[:, :1], S, axis=1)
    out, _ = oracle.sparse_mla(q, same, idx, nsel, sl, Dv, 0.3)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(_vals(same)[0, 0, :Dv], (H, Dv)),
                               rtol=1e-14)
    # q = 0 -> uniform weights -> mean of the selected value vectors, lse = log(count)
    zq = np.zeros_like(q)
    out, lse = oracle.sparse_mla(zq, kv, idx, nsel, sl, Dv, 0.3)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(_vals(kv)[0, idx[0, 0], :Dv].mean(0),
                                                          (H, Dv)), rtol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(6.0), rtol=1e-14)
    # set semantics: the order of the index list does not matter
    out1, lse1 = oracle.sparse_mla(q, kv, idx, nsel, sl, Dv, 0.3)
    perm = idx[:, :, ::-1].copy()
    out2, lse2 = oracle.sparse_mla(q, kv, perm, nsel, sl, Dv, 0.3)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse1, lse2, rtol=1e-14)
    # exp(l - lse) sums to one
    qv, kvv = _vals(q)[0, 0], _vals(kv)[0, idx[0, 0]]
    lg = 0.3 * qv @ kvv.T
    np.testing.assert_allclose(np.exp(lg - lse1[0, 0][:, None]).sum(1), 1.0, rtol=1e-13)


def test_sparse_equals_dense_when_short():
    """n <= topk: the selection keeps everything, so sparse attention equals dense attention."""
    S, topk = 200, 256
    qi = _dyadic(4, 1, (1, 1, 4, 32))
    ki = _dyadic(4, 3, (1, S, 32))
    w = _weights(4, 2, (1, 1, 4))
    sl = np.array([S], np.int32)
    sc = oracle.index_scores(qi, w, ki, sl, 1)
    idx, nsel = oracle.topk_select(sc, sl, topk, 4, 64)
    assert nsel[0, 0] == S
    q = _normal(4, 4, (1, 1, 4, 80))
    kv = _normal(4, 5, (1, S, 80))
    a, la = oracle.sparse_mla(q, kv, idx, nsel, sl, 64, 80 ** -0.5)
    b, lb = oracle.sparse_mla(q, kv, None, None, sl, 64, 80 ** -0.5)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14)


def test_prefill_rows_equal_decode_calls():
    """A prefill row at position p equals a decode call on a cache of p + 1 tokens
    (cached forward == full forward)."""
    S, Lq, topk = 48, 6, 16
    qi = _dyadic(9, 1, (1, Lq, 4, 32))
    ki = _dyadic(9, 3, (1, S, 32))
    w = _weights(9, 2, (1, Lq, 4))
    q = _normal(9, 4, (1, Lq, 4, 40))
    kv = _normal(9, 5, (1, S, 40))
    sl = np.array([S], np.int32)
    sc = oracle.index_scores(qi, w, ki, sl, Lq)
    idx, nsel = oracle.topk_select(sc, sl, topk, 2, 4)
    out, lse = oracle.sparse_mla(q, kv, idx, nsel, sl, 32, 0.2)
    for i in range(Lq):
        p = S - Lq + i
        sl1 = np.array([p + 1], np.int32)
        sc1 = oracle.index_scores(qi[:, i:i + 1], w[:, i:i + 1], ki, sl1, 1)
        np.testing.assert_array_equal(sc1[0, 0, : p + 1], sc[0, i, : p + 1])
        idx1, nsel1 = oracle.topk_select(sc1, sl1, topk, 2, 4)
        np.testing.assert_array_equal(idx1[0, 0], idx[0, i])
        o1, l1 = oracle.sparse_mla(q[:, i:i + 1], kv, idx1, nsel1, sl1, 32, 0.2)
        np.testing.assert_array_equal(o1[0, 0], out[0, i])
        np.testing.assert_array_equal(l1[0, 0], lse[0, i])


def test_rejects_out_of_range_index():
    q = _normal(1, 4, (1, 1, 1, 8))
    kv = _normal(1, 5, (1, 10, 8))
    with pytest.raises(ValueError):
        oracle.sparse_mla(q, kv, np.array([[[3, 9]]], np.int32), np.array([[2]], np.int32),
                          np.array([5], np.int32), 8, 1.0)
