"""Thin ctypes binding of ``liblsa.so`` (C ABI in ``include/lsa.h``).

Argument marshalling only: shapes come from the tensors, pointers from ``data_ptr()`` and the
stream from ``torch.cuda.current_stream()``; every step of the hot path runs in the library's
HIP kernels.  PyTorch provides device memory (including workspaces) and streams, nothing else.
The binding refuses to run without the built library -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblsa.so")

LSA_OK = 0
STATUS = {0: "LSA_OK", 1: "LSA_ERR_NULL_ARG", 2: "LSA_ERR_BAD_SHAPE", 3: "LSA_ERR_UNSUPPORTED",
          4: "LSA_ERR_WORKSPACE", 5: "LSA_ERR_LAUNCH"}

EXPORTED = ["lsa_status_str", "lsa_last_error", "lsa_index_scores", "lsa_topk_workspace_bytes",
            "lsa_topk_select", "lsa_index_topk_workspace_bytes", "lsa_index_topk",
            "lsa_mla_workspace_bytes", "lsa_sparse_mla_decode", "lsa_sparse_mla_prefill",
            "lsa_index_frontend_workspace_bytes", "lsa_index_frontend",
            "lsa_mtp_draft_workspace_bytes", "lsa_mtp_draft_attention", "lsa_block_keys",
            "lsa_hier_workspace_bytes", "lsa_hier_index_topk", "lsa_index_topk_noalloc",
            "lsa_check_seqlens"]

INDEX_TOPK_SCRATCH_BYTES = 16 << 20  # LSA_INDEX_TOPK_SCRATCH_BYTES


class LsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """Load liblsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with "
                               "`python -m long_context_sparse_lightning_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.lsa_status_str.argtypes = [I]
        L.lsa_status_str.restype = ctypes.c_char_p
        L.lsa_last_error.argtypes = []
        L.lsa_last_error.restype = ctypes.c_char_p
        L.lsa_check_seqlens.argtypes = [P, I, I, I]
        L.lsa_check_seqlens.restype = I
        L.lsa_index_scores.argtypes = [P, P, P, P, I, I, I, I, I, P, P]
        L.lsa_index_scores.restype = I
        L.lsa_topk_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.lsa_topk_workspace_bytes.restype = Z
        L.lsa_topk_select.argtypes = [P, P, I, I, I, I, I, I, P, P, P, Z, P]
        L.lsa_topk_select.restype = I
        L.lsa_index_topk_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.lsa_index_topk_workspace_bytes.restype = Z
        L.lsa_index_topk.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, P, P, Z, P]
        L.lsa_index_topk.restype = I
        L.lsa_index_topk_noalloc.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, P, P, P]
        L.lsa_index_topk_noalloc.restype = I
        L.lsa_mla_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.lsa_mla_workspace_bytes.restype = Z
        L.lsa_sparse_mla_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, P]
        L.lsa_sparse_mla_decode.restype = I
        L.lsa_sparse_mla_prefill.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, Z, P]
        L.lsa_sparse_mla_prefill.restype = I
        L.lsa_index_frontend_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.lsa_index_frontend_workspace_bytes.restype = Z
        L.lsa_index_frontend.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, F, I, P, P, P,
                                         P, Z, P]
        L.lsa_index_frontend.restype = I
        L.lsa_mtp_draft_workspace_bytes.argtypes = [I, I, I, I, I, I]
        L.lsa_mtp_draft_workspace_bytes.restype = Z
        L.lsa_mtp_draft_attention.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, Z, P]
        L.lsa_mtp_draft_attention.restype = I
        L.lsa_block_keys.argtypes = [P, P, I, I, I, I, I, P, P]
        L.lsa_block_keys.restype = I
        L.lsa_hier_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        L.lsa_hier_workspace_bytes.restype = Z
        L.lsa_hier_index_topk.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, P, P, Z, P]
        L.lsa_hier_index_topk.restype = I
        _lib = L
    return _lib


def check_seqlens(seqlens, Lq, S_max) -> int:
    """The device-side precondition Lq <= seqlens[b] <= S_max on a host copy of the lengths:
    the first b that violates it, or -1 (the check LSA_DEBUG_BOUNDS=1 makes on every call)."""
    import numpy as np

    h = np.ascontiguousarray(np.asarray(seqlens.cpu() if hasattr(seqlens, "cpu") else seqlens,
                                        dtype=np.int32))
    return int(lib().lsa_check_seqlens(h.ctypes.data_as(ctypes.c_void_p), h.size, Lq, S_max))


def _check(status: int) -> None:
    if status != LSA_OK:
        raise LsaError(status, lib().lsa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _want(t, name, dtype, ndim):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _want_shape(t, name, dtype, shape):
    """A tensor that must match exactly: dtype, shape, contiguous, on a device."""
    _want(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(name, *ts):
    """Every tensor given is a device tensor, all on one device (checked after the shapes)."""
    devs = {t.device for t in ts if t is not None}
    if any(d.type != "cuda" for d in devs):
        raise ValueError(f"{name}: every tensor must be a device tensor, got {sorted(map(str, devs))}")
    if len(devs) > 1:
        raise ValueError(f"{name}: tensors on different devices {sorted(map(str, devs))}")


def _index_inputs(fn, q_idx, w, k_idx, seqlens):
    """Shapes of the indexer inputs, checked against each other: (B, Lq, Hi, Di, S_max)."""
    _want(q_idx, "q_idx", torch.bfloat16, 4)
    B, Lq, Hi, Di = q_idx.shape
    _want_shape(w, "w", torch.float32, (B, Lq, Hi))
    _want(k_idx, "k_idx", torch.bfloat16, 3)
    if k_idx.shape[0] != B or k_idx.shape[2] != Di:
        raise ValueError(f"{fn}: k_idx shape {tuple(k_idx.shape)} does not match q_idx "
                         f"{tuple(q_idx.shape)} (expected [{B}, S_max, {Di}])")
    _want_shape(seqlens, "seqlens", torch.int32, (B,))
    return B, Lq, Hi, Di, k_idx.shape[1]


def _selection_outputs(indices, n_sel, B, Lq, topk, dev):
    """Caller-supplied (or new) indices [B, Lq, topk] and n_sel [B, Lq]."""
    if indices is None:
        indices = torch.empty(B, Lq, topk, dtype=torch.int32, device=dev)
    _want_shape(indices, "indices", torch.int32, (B, Lq, topk))
    if n_sel is None:
        n_sel = torch.empty(B, Lq, dtype=torch.int32, device=dev)
    _want_shape(n_sel, "n_sel", torch.int32, (B, Lq))
    return indices, n_sel


def _workspace(workspace, need, dev):
    """The caller's workspace (contents on entry do not matter), or a new one."""
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None and (workspace.device.type != "cuda" or not workspace.is_contiguous()):
        raise ValueError("workspace: must be a contiguous device tensor")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, wbytes


def lsa_index_scores(q_idx, w, k_idx, seqlens, scores=None):
    """q_idx bf16 [B,Lq,Hi,Di], w f32 [B,Lq,Hi], k_idx bf16 [B,S_max,Di], seqlens i32 [B]
    -> scores f32 [B,Lq,S_max] (entries after each query's position are left untouched)."""
    B, Lq, Hi, Di, S_max = _index_inputs("lsa_index_scores", q_idx, w, k_idx, seqlens)
    if scores is None:
        scores = torch.empty(B, Lq, S_max, dtype=torch.float32, device=q_idx.device)
    _want_shape(scores, "scores", torch.float32, (B, Lq, S_max))
    _same_device("lsa_index_scores", q_idx, w, k_idx, seqlens, scores)
    _check(lib().lsa_index_scores(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(seqlens), B, Lq, Hi, Di,
                                  S_max, _ptr(scores), _stream(q_idx)))
    return scores


def lsa_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens) -> int:
    return int(lib().lsa_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens))


def lsa_topk_select(scores, seqlens, topk, init_tokens, local_tokens, indices=None, n_sel=None,
                    workspace=None):
    """scores f32 [B,Lq,S_max] -> (indices i32 [B,Lq,topk] ascending, -1 padded; n_sel i32 [B,Lq])."""
    _want(scores, "scores", torch.float32, 3)
    B, Lq, S_max = scores.shape
    _want_shape(seqlens, "seqlens", torch.int32, (B,))
    dev = scores.device
    indices, n_sel = _selection_outputs(indices, n_sel, B, Lq, topk, dev)
    _same_device("lsa_topk_select", scores, seqlens, indices, n_sel)
    need = lsa_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens)
    workspace, wbytes = _workspace(workspace, need, dev)
    _check(lib().lsa_topk_select(_ptr(scores), _ptr(seqlens), B, Lq, S_max, topk, init_tokens,
                                 local_tokens, _ptr(indices), _ptr(n_sel), _ptr(workspace), wbytes,
                                 _stream(scores)))
    return indices, n_sel


def lsa_index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens) -> int:
    return int(lib().lsa_index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens))


def lsa_index_topk(q_idx, w, k_idx, seqlens, topk, init_tokens, local_tokens, indices=None,
                   n_sel=None, workspace=None):
    """Indexer + top-k in one pass (no score array): the inputs of lsa_index_scores ->
    (indices i32 [B,Lq,topk] ascending, -1 padded; n_sel i32 [B,Lq])."""
    B, Lq, Hi, Di, S_max = _index_inputs("lsa_index_topk", q_idx, w, k_idx, seqlens)
    dev = q_idx.device
    indices, n_sel = _selection_outputs(indices, n_sel, B, Lq, topk, dev)
    _same_device("lsa_index_topk", q_idx, w, k_idx, seqlens, indices, n_sel)
    need = lsa_index_topk_workspace_bytes(B, Lq, S_max, topk, init_tokens, local_tokens)
    workspace, wbytes = _workspace(workspace, need, dev)
    _check(lib().lsa_index_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(seqlens), B, Lq, Hi, Di,
                                S_max, topk, init_tokens, local_tokens, _ptr(indices), _ptr(n_sel),
                                _ptr(workspace), wbytes, _stream(q_idx)))
    return indices, n_sel


def lsa_index_topk_noalloc(q_idx, w, k_idx, seqlens, topk, init_tokens, local_tokens, indices,
                           n_sel):
    """lsa_index_topk with the library's static per-device workspace instead of a caller one
    (no allocation at all: indices and n_sel must be given).  Calls overlapping on one device
    race on that workspace."""
    B, Lq, Hi, Di, S_max = _index_inputs("lsa_index_topk_noalloc", q_idx, w, k_idx, seqlens)
    _want_shape(indices, "indices", torch.int32, (B, Lq, topk))
    _want_shape(n_sel, "n_sel", torch.int32, (B, Lq))
    _same_device("lsa_index_topk_noalloc", q_idx, w, k_idx, seqlens, indices, n_sel)
    _check(lib().lsa_index_topk_noalloc(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(seqlens), B, Lq, Hi,
                                        Di, S_max, topk, init_tokens, local_tokens, _ptr(indices),
                                        _ptr(n_sel), _stream(q_idx)))
    return indices, n_sel


def lsa_mla_workspace_bytes(B, Lq, H, Dv, S_max, topk, dense) -> int:
    return int(lib().lsa_mla_workspace_bytes(B, Lq, H, Dv, S_max, topk, 1 if dense else 0))


def _mla(decode, q, kv, indices, n_sel, seqlens, Dv, softmax_scale, out, lse, workspace):
    if decode:
        _want(q, "q", torch.bfloat16, 3)
        B, H, Dqk = q.shape
        Lq = 1
        rows = (B,)
    else:
        _want(q, "q", torch.bfloat16, 4)
        B, Lq, H, Dqk = q.shape
        rows = (B, Lq)
    _want(kv, "kv", torch.bfloat16, 3)
    if kv.shape[0] != B or kv.shape[2] != Dqk:
        raise ValueError(f"kv: shape {tuple(kv.shape)} does not match q {tuple(q.shape)} "
                         f"(expected [{B}, S_max, {Dqk}])")
    _want_shape(seqlens, "seqlens", torch.int32, (B,))
    S_max = kv.shape[1]
    dense = indices is None
    topk = 0
    if not dense:
        _want(indices, "indices", torch.int32, len(rows) + 1)
        topk = indices.shape[-1]
        _want_shape(indices, "indices", torch.int32, rows + (topk,))
        if n_sel is None:
            raise ValueError("n_sel: required with indices")
        _want_shape(n_sel, "n_sel", torch.int32, rows)
    dev = q.device
    if out is None:
        out = torch.empty(rows + (H, Dv), dtype=torch.bfloat16, device=dev)
    _want_shape(out, "out", torch.bfloat16, rows + (H, Dv))
    if lse is not None:
        _want_shape(lse, "lse", torch.float32, rows + (H,))
    _same_device("attention", q, kv, seqlens, indices, n_sel, out, lse)
    need = lsa_mla_workspace_bytes(B, Lq, H, Dv, S_max, topk, dense)
    workspace, wbytes = _workspace(workspace, need, dev)
    if decode:
        st = lib().lsa_sparse_mla_decode(_ptr(q), _ptr(kv), _ptr(indices), _ptr(n_sel),
                                         _ptr(seqlens), B, H, Dqk, Dv, S_max, topk,
                                         float(softmax_scale), _ptr(out), _ptr(lse),
                                         _ptr(workspace), wbytes, _stream(q))
    else:
        st = lib().lsa_sparse_mla_prefill(_ptr(q), _ptr(kv), _ptr(indices), _ptr(n_sel),
                                          _ptr(seqlens), B, Lq, H, Dqk, Dv, S_max, topk,
                                          float(softmax_scale), _ptr(out), _ptr(lse),
                                          _ptr(workspace), wbytes, _stream(q))
    _check(st)
    return out


def lsa_sparse_mla_decode(q, kv, indices, n_sel, seqlens, Dv, softmax_scale, out=None, lse=None,
                          workspace=None):
    """q bf16 [B,H,Dqk], kv bf16 [B,S_max,Dqk], indices i32 [B,topk] (or None: dense over
    [0, p]), n_sel i32 [B] -> out bf16 [B,H,Dv] (lse f32 [B,H] written if given)."""
    return _mla(True, q, kv, indices, n_sel, seqlens, Dv, softmax_scale, out, lse, workspace)


def lsa_sparse_mla_prefill(q, kv, indices, n_sel, seqlens, Dv, softmax_scale, out=None, lse=None,
                           workspace=None):
    """q bf16 [B,Lq,H,Dqk], kv bf16 [B,S_max,Dqk], indices i32 [B,Lq,topk] (or None: dense
    causal), n_sel i32 [B,Lq] -> out bf16 [B,Lq,H,Dv] (lse f32 [B,Lq,H] written if given)."""
    return _mla(False, q, kv, indices, n_sel, seqlens, Dv, softmax_scale, out, lse, workspace)


def lsa_mtp_draft_workspace_bytes(B, H, Dv, S_max, topk, max_appended) -> int:
    return int(lib().lsa_mtp_draft_workspace_bytes(B, H, Dv, S_max, topk, max_appended))


def lsa_mtp_draft_attention(q, kv, indices, n_sel, index_seqlens, seqlens, Dv, softmax_scale,
                            max_appended=3, out=None, lse=None, workspace=None):
    """A draft step on a shared index pass: q bf16 [B,H,Dqk], kv bf16 [B,S_max,Dqk], indices i32
    [B,topk] and n_sel i32 [B] of the pass made at index_seqlens i32 [B]; the query sits at
    seqlens[b] - 1 and also attends to the positions appended since (at most max_appended)
    -> out bf16 [B,H,Dv] (lse f32 [B,H] written if given)."""
    _want(q, "q", torch.bfloat16, 3)
    B, H, Dqk = q.shape
    _want(kv, "kv", torch.bfloat16, 3)
    if kv.shape[0] != B or kv.shape[2] != Dqk:
        raise ValueError(f"kv: shape {tuple(kv.shape)} does not match q {tuple(q.shape)} "
                         f"(expected [{B}, S_max, {Dqk}])")
    _want(indices, "indices", torch.int32, 2)
    S_max, topk = kv.shape[1], indices.shape[1]
    _want_shape(indices, "indices", torch.int32, (B, topk))
    _want_shape(n_sel, "n_sel", torch.int32, (B,))
    _want_shape(index_seqlens, "index_seqlens", torch.int32, (B,))
    _want_shape(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        out = torch.empty(B, H, Dv, dtype=torch.bfloat16, device=q.device)
    _want_shape(out, "out", torch.bfloat16, (B, H, Dv))
    if lse is not None:
        _want_shape(lse, "lse", torch.float32, (B, H))
    _same_device("lsa_mtp_draft_attention", q, kv, indices, n_sel, index_seqlens, seqlens, out, lse)
    need = lsa_mtp_draft_workspace_bytes(B, H, Dv, S_max, topk, max_appended)
    workspace, wbytes = _workspace(workspace, need, q.device)
    _check(lib().lsa_mtp_draft_attention(_ptr(q), _ptr(kv), _ptr(indices), _ptr(n_sel),
                                         _ptr(index_seqlens), _ptr(seqlens), B, H, Dqk, Dv, S_max,
                                         topk, int(max_appended), float(softmax_scale), _ptr(out),
                                         _ptr(lse), _ptr(workspace), wbytes, _stream(q)))
    return out


def lsa_block_keys(k_idx, seqlens, Bk, block_keys=None, first_block=0):
    """k_idx bf16 [B,S_max,Di], seqlens i32 [B] -> block_keys bf16 [B,S_max//Bk,Di] (rows
    first_block .. seqlens[b]//Bk - 1 written: the bf16 means of complete blocks of Bk keys)."""
    _want(k_idx, "k_idx", torch.bfloat16, 3)
    _want(seqlens, "seqlens", torch.int32, 1)
    B, S_max, Di = k_idx.shape
    if block_keys is None:
        block_keys = torch.zeros(B, S_max // Bk, Di, dtype=torch.bfloat16, device=k_idx.device)
    _want(block_keys, "block_keys", torch.bfloat16, 3)
    if block_keys.shape != (B, S_max // Bk, Di) or seqlens.shape[0] != B:
        raise ValueError("lsa_block_keys: inconsistent shapes")
    _same_device("lsa_block_keys", k_idx, seqlens, block_keys)
    _check(lib().lsa_block_keys(_ptr(k_idx), _ptr(seqlens), B, S_max, Di, int(Bk), int(first_block),
                                _ptr(block_keys), _stream(k_idx)))
    return block_keys


def lsa_hier_workspace_bytes(B, S_max, Bk, topk, init_tokens, local_tokens, M) -> int:
    return int(lib().lsa_hier_workspace_bytes(B, S_max, Bk, topk, init_tokens, local_tokens, M))


def lsa_hier_index_topk(q_idx, w, k_idx, block_keys, seqlens, topk, init_tokens, local_tokens, Bk,
                        M, indices=None, n_sel=None, workspace=None):
    """Hierarchical indexer + top-k of decode rows: q_idx bf16 [B,Hi,Di], w f32 [B,Hi], k_idx
    bf16 [B,S_max,Di], block_keys bf16 [B,S_max//Bk,Di] (lsa_block_keys) -> (indices i32
    [B,topk], n_sel i32 [B])."""
    _want(q_idx, "q_idx", torch.bfloat16, 3)
    _want(w, "w", torch.float32, 2)
    _want(k_idx, "k_idx", torch.bfloat16, 3)
    _want(block_keys, "block_keys", torch.bfloat16, 3)
    _want(seqlens, "seqlens", torch.int32, 1)
    B, Hi, Di = q_idx.shape
    S_max = k_idx.shape[1]
    if w.shape != (B, Hi) or k_idx.shape != (B, S_max, Di) or seqlens.shape[0] != B \
            or block_keys.shape != (B, S_max // Bk, Di):
        raise ValueError("lsa_hier_index_topk: inconsistent shapes")
    dev = q_idx.device
    if indices is None:
        indices = torch.empty(B, topk, dtype=torch.int32, device=dev)
    _want_shape(indices, "indices", torch.int32, (B, topk))
    if n_sel is None:
        n_sel = torch.empty(B, dtype=torch.int32, device=dev)
    _want_shape(n_sel, "n_sel", torch.int32, (B,))
    _same_device("lsa_hier_index_topk", q_idx, w, k_idx, block_keys, seqlens, indices, n_sel)
    need = lsa_hier_workspace_bytes(B, S_max, Bk, topk, init_tokens, local_tokens, M)
    workspace, wbytes = _workspace(workspace, need, dev)
    _check(lib().lsa_hier_index_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), _ptr(block_keys),
                                     _ptr(seqlens), B, Hi, Di, S_max, topk, init_tokens, local_tokens,
                                     int(Bk), int(M), _ptr(indices), _ptr(n_sel), _ptr(workspace),
                                     wbytes, _stream(q_idx)))
    return indices, n_sel


def lsa_index_frontend_workspace_bytes(B, Lq, q_lora, hidden, Hi, Di) -> int:
    return int(lib().lsa_index_frontend_workspace_bytes(B, Lq, q_lora, hidden, Hi, Di))


def lsa_index_frontend(cq, hid, wq_b, wk, k_norm_gain, w_proj, seqlens, k_cache, rope_dim=64,
                       rope_theta=1e6, norm_eps=1e-6, q_idx=None, w=None, workspace=None):
    """cq bf16 [B,Lq,q_lora], hid bf16 [B,Lq,hidden], wq_b bf16 [Hi*Di,q_lora], wk bf16
    [Di,hidden], k_norm_gain f32 [Di], w_proj bf16 [Hi,hidden], seqlens i32 [B], k_cache bf16
    [B,S_max,Di] (row p of each current token is written) -> (q_idx bf16 [B,Lq,Hi,Di], w f32
    [B,Lq,Hi])."""
    _want(cq, "cq", torch.bfloat16, 3)
    _want(hid, "hid", torch.bfloat16, 3)
    _want(wq_b, "wq_b", torch.bfloat16, 2)
    _want(wk, "wk", torch.bfloat16, 2)
    _want(k_norm_gain, "k_norm_gain", torch.float32, 1)
    _want(w_proj, "w_proj", torch.bfloat16, 2)
    _want(seqlens, "seqlens", torch.int32, 1)
    _want(k_cache, "k_cache", torch.bfloat16, 3)
    B, Lq, q_lora = cq.shape
    hidden = hid.shape[2]
    Di = wk.shape[0]
    Hi = w_proj.shape[0]
    S_max = k_cache.shape[1]
    if hid.shape[:2] != (B, Lq) or wq_b.shape != (Hi * Di, q_lora) or wk.shape[1] != hidden \
            or w_proj.shape[1] != hidden or k_norm_gain.shape[0] != Di \
            or k_cache.shape[0] != B or k_cache.shape[2] != Di or seqlens.shape[0] != B:
        raise ValueError("lsa_index_frontend: inconsistent shapes")
    dev = cq.device
    if q_idx is None:
        q_idx = torch.empty(B, Lq, Hi, Di, dtype=torch.bfloat16, device=dev)
    _want_shape(q_idx, "q_idx", torch.bfloat16, (B, Lq, Hi, Di))
    if w is None:
        w = torch.empty(B, Lq, Hi, dtype=torch.float32, device=dev)
    _want_shape(w, "w", torch.float32, (B, Lq, Hi))
    _same_device("lsa_index_frontend", cq, hid, wq_b, wk, k_norm_gain, w_proj, seqlens, k_cache,
                 q_idx, w)
    need = lsa_index_frontend_workspace_bytes(B, Lq, q_lora, hidden, Hi, Di)
    workspace, wbytes = _workspace(workspace, need, dev)
    _check(lib().lsa_index_frontend(_ptr(cq), _ptr(hid), _ptr(wq_b), _ptr(wk), _ptr(k_norm_gain),
                                    _ptr(w_proj), _ptr(seqlens), B, Lq, q_lora, hidden, Hi, Di,
                                    rope_dim, rope_theta, norm_eps, S_max, _ptr(q_idx), _ptr(w),
                                    _ptr(k_cache), _ptr(workspace), wbytes, _stream(cq)))
    return q_idx, w
