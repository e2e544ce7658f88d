"""CPU oracle for the LSA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The GPU library never loads it, and it shares no code with the GPU path:
the arithmetic lives in ``lsa_oracle.c`` (plain C, fp64, naive loops), and this module only
marshals numpy arrays to it.  See the header of ``lsa_oracle.c`` for the passages each
function follows and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB = os.path.join(_HERE, "liblsa_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (-O2, IEEE semantics: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.lsa_oracle_index_scores.argtypes = [P, P, P, P, I, I, I, I, I, P]
        L.lsa_oracle_index_scores.restype = I
        L.lsa_oracle_topk.argtypes = [P, P, I, I, I, I, I, I, P, P]
        L.lsa_oracle_topk.restype = I
        L.lsa_oracle_sparse_mla.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_double,
                                            P, P]
        L.lsa_oracle_sparse_mla.restype = I
        L.lsa_oracle_index_frontend.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                                ctypes.c_double, ctypes.c_double, P, P, P]
        L.lsa_oracle_index_frontend.restype = I
        L.lsa_oracle_hier_topk.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I, P, P]
        L.lsa_oracle_hier_topk.restype = I
        L.lsa_oracle_set_threads.argtypes = [I]
        L.lsa_oracle_max_threads.restype = I
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    lib().lsa_oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().lsa_oracle_max_threads())


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def index_scores(q_idx, w, k_idx, seqlens, Lq: int) -> np.ndarray:
    """q_idx bf16 bits [B,Lq,Hi,Di], w f32 [B,Lq,Hi], k_idx bf16 bits [B,S_max,Di] ->
    f32 scores [B,Lq,S_max] (NaN where s > p)."""
    q_idx = _c(q_idx, np.uint16)
    w = _c(w, np.float32)
    k_idx = _c(k_idx, np.uint16)
    seqlens = _c(seqlens, np.int32)
    B, Lq_, Hi, Di = q_idx.shape
    assert Lq_ == Lq and w.shape == (B, Lq, Hi) and k_idx.shape[0] == B and k_idx.shape[2] == Di
    S_max = k_idx.shape[1]
    out = np.full((B, Lq, S_max), np.nan, dtype=np.float32)
    rc = lib().lsa_oracle_index_scores(q_idx.ctypes.data, w.ctypes.data, k_idx.ctypes.data,
                                       seqlens.ctypes.data, B, Lq, Hi, Di, S_max, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"lsa_oracle_index_scores: bad input ({rc})")
    return out


def topk_select(scores, seqlens, topk: int, init_tokens: int, local_tokens: int):
    """scores f32 [B,Lq,S_max] -> (indices int32 [B,Lq,topk] ascending, -1 padded; n_sel [B,Lq])."""
    scores = _c(scores, np.float32)
    seqlens = _c(seqlens, np.int32)
    B, Lq, S_max = scores.shape
    idx = np.empty((B, Lq, topk), dtype=np.int32)
    nsel = np.empty((B, Lq), dtype=np.int32)
    rc = lib().lsa_oracle_topk(scores.ctypes.data, seqlens.ctypes.data, B, Lq, S_max, topk,
                               init_tokens, local_tokens, idx.ctypes.data, nsel.ctypes.data)
    if rc != 0:
        raise ValueError(f"lsa_oracle_topk: bad input ({rc})")
    return idx, nsel


def sparse_mla(q, kv, indices, n_sel, seqlens, Dv: int, scale: float):
    """q bf16 bits [B,Lq,H,Dqk]; kv bf16 bits [B,S_max,Dqk]; indices int32 [B,Lq,topk] or None
    (dense over [0,p]); n_sel int32 [B,Lq] -> (out f64 [B,Lq,H,Dv], lse f64 [B,Lq,H])."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    seqlens = _c(seqlens, np.int32)
    B, Lq, H, Dqk = q.shape
    assert kv.shape[0] == B and kv.shape[2] == Dqk and 0 < Dv <= Dqk
    S_max = kv.shape[1]
    if indices is not None:
        indices = _c(indices, np.int32)
        n_sel = _c(n_sel, np.int32)
        topk = indices.shape[2]
        assert indices.shape[:2] == (B, Lq) and n_sel.shape == (B, Lq)
        ip, np_ = indices.ctypes.data, n_sel.ctypes.data
    else:
        topk, ip, np_ = 0, None, None
    out = np.empty((B, Lq, H, Dv), dtype=np.float64)
    lse = np.empty((B, Lq, H), dtype=np.float64)
    rc = lib().lsa_oracle_sparse_mla(q.ctypes.data, kv.ctypes.data, ip, np_, seqlens.ctypes.data,
                                     B, Lq, H, Dqk, Dv, S_max, topk, float(scale),
                                     out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"lsa_oracle_sparse_mla: bad input ({rc})")
    return out, lse


def hier_topk(q_idx, w, k_idx, seqlens, topk: int, init_tokens: int, local_tokens: int, Bk: int,
              M: int):
    """Hierarchical indexing of decode rows (see lsa_oracle_hier_topk): q_idx bf16 bits
    [B,Hi,Di], w f32 [B,Hi], k_idx bf16 bits [B,S_max,Di] -> (indices int32 [B,topk] ascending,
    -1 padded; n_sel int32 [B])."""
    q_idx = _c(q_idx, np.uint16)
    w = _c(w, np.float32)
    k_idx = _c(k_idx, np.uint16)
    seqlens = _c(seqlens, np.int32)
    B, Hi, Di = q_idx.shape
    S_max = k_idx.shape[1]
    assert w.shape == (B, Hi) and k_idx.shape == (B, S_max, Di)
    idx = np.empty((B, topk), dtype=np.int32)
    nsel = np.empty(B, dtype=np.int32)
    rc = lib().lsa_oracle_hier_topk(q_idx.ctypes.data, w.ctypes.data, k_idx.ctypes.data,
                                    seqlens.ctypes.data, B, Hi, Di, S_max, topk, init_tokens,
                                    local_tokens, Bk, M, idx.ctypes.data, nsel.ctypes.data)
    if rc != 0:
        raise ValueError(f"lsa_oracle_hier_topk: bad input ({rc})")
    return idx, nsel


def mtp_draft_indices(indices, n_sel, index_seqlens, seqlens, max_appended: int):
    """Selection of a multi-token-prediction draft step on a shared index pass (page "LongCat
    Sparse Attention技术深度解析", "技术实现细节": the three draft steps share one index pass).
    indices int32 [B,topk] and n_sel int32 [B] of the pass made at index_seqlens [B]; the query
    sits at p = seqlens[b] - 1.  Per sequence: the pass's first min(n_sel, topk) entries, then
    the positions appended since, index_seqlens[b] .. p (at most max_appended of them).
    Returns (indices int32 [B,1,topk+max_appended], -1 padded; n_sel int32 [B,1]).  Where the
    shared pass runs (here: at the first draft step) is parity unpinned against the pages."""
    indices = np.asarray(indices, np.int32)
    B, topk = indices.shape
    out = np.full((B, 1, topk + max_appended), -1, np.int32)
    cnt = np.zeros((B, 1), np.int32)
    for b in range(B):
        base = indices[b, :max(0, min(int(n_sel[b]), topk))]
        first = max(int(index_seqlens[b]), 0)
        app = np.arange(first, min(int(seqlens[b]), first + max_appended), dtype=np.int32)
        sel = np.concatenate([base, app])
        out[b, 0, :len(sel)] = sel
        cnt[b, 0] = len(sel)
    return out, cnt


def mtp_draft_attention(q, kv, indices, n_sel, index_seqlens, seqlens, max_appended: int, Dv: int,
                        scale: float):
    """Attention of a draft step (q bf16 bits [B,H,Dqk]) over mtp_draft_indices' selection:
    the attention of sparse_mla.  Returns (out f64 [B,H,Dv], lse f64 [B,H])."""
    idx, cnt = mtp_draft_indices(indices, n_sel, index_seqlens, seqlens, max_appended)
    q = np.asarray(q)
    out, lse = sparse_mla(q[:, None], kv, idx, cnt, seqlens, Dv, scale)
    return out[:, 0], lse[:, 0]


def index_frontend(cq, hid, wq_b, wk, gain, w_proj, seqlens, Hi: int, Di: int, rope_dim: int,
                   theta: float, eps: float):
    """cq bf16 bits [B,Lq,q_lora]; hid bf16 bits [B,Lq,hidden]; wq_b bf16 bits [Hi*Di,q_lora];
    wk bf16 bits [Di,hidden]; gain f32 [Di]; w_proj bf16 bits [Hi,hidden] ->
    (q f64 [B,Lq,Hi,Di], w f64 [B,Lq,Hi], k f64 [B,Lq,Di]): the index query, head weights and
    the key written at each token's position."""
    cq = _c(cq, np.uint16)
    hid = _c(hid, np.uint16)
    wq_b = _c(wq_b, np.uint16)
    wk = _c(wk, np.uint16)
    gain = _c(gain, np.float32)
    w_proj = _c(w_proj, np.uint16)
    seqlens = _c(seqlens, np.int32)
    B, Lq, q_lora = cq.shape
    hidden = hid.shape[2]
    assert hid.shape[:2] == (B, Lq) and wq_b.shape == (Hi * Di, q_lora)
    assert wk.shape == (Di, hidden) and gain.shape == (Di,) and w_proj.shape == (Hi, hidden)
    q = np.empty((B, Lq, Hi, Di), dtype=np.float64)
    w = np.empty((B, Lq, Hi), dtype=np.float64)
    k = np.empty((B, Lq, Di), dtype=np.float64)
    rc = lib().lsa_oracle_index_frontend(cq.ctypes.data, hid.ctypes.data, wq_b.ctypes.data,
                                         wk.ctypes.data, gain.ctypes.data, w_proj.ctypes.data,
                                         seqlens.ctypes.data, B, Lq, q_lora, hidden, Hi, Di,
                                         rope_dim, float(theta), float(eps), q.ctypes.data,
                                         w.ctypes.data, k.ctypes.data)
    if rc != 0:
        raise ValueError(f"lsa_oracle_index_frontend: bad input ({rc})")
    return q, w, k
