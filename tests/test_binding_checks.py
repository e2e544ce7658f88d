"""The Python binding checks caller tensors against each other before any pointer reaches the C
ABI: a mismatched shape, dtype or length raises ValueError/TypeError instead of turning into
out-of-range device accesses.  Host tensors are used on purpose: every check below fires before
the device check, so these run without a GPU (the library is loaded only for workspace sizes)."""
import pytest
import torch

from long_context_sparse_lightning_amd import lsa

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
B, Lq, Hi, Di, S, K = 2, 1, 4, 32, 64, 16
H, DQK, DV = 4, 80, 64


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def idx_inputs(**over):
    a = dict(q_idx=z(B, Lq, Hi, Di), w=z(B, Lq, Hi, dtype=f32), k_idx=z(B, S, Di),
             seqlens=z(B, dtype=i32))
    a.update(over)
    return a


@pytest.mark.parametrize("over", [
    dict(w=z(B, Lq, Hi + 1, dtype=f32)),
    dict(w=z(B, Lq, Hi, dtype=bf)),
    dict(k_idx=z(B + 1, S, Di)),
    dict(k_idx=z(B, S, Di * 2)),
    dict(seqlens=z(B + 1, dtype=i32)),
    dict(seqlens=z(B, dtype=torch.int64)),
    dict(q_idx=z(B, Lq, Hi, Di).transpose(2, 3)),
])
def test_index_inputs_mismatch(over):
    with pytest.raises((ValueError, TypeError)):
        lsa.lsa_index_scores(**idx_inputs(**over))
    with pytest.raises((ValueError, TypeError)):
        lsa.lsa_index_topk(**idx_inputs(**over), topk=K, init_tokens=2, local_tokens=4)


def test_index_outputs_mismatch():
    with pytest.raises(ValueError, match="scores"):
        lsa.lsa_index_scores(**idx_inputs(), scores=z(B, Lq, S + 1, dtype=f32))
    for bad in (dict(indices=z(B, Lq, K + 1, dtype=i32)), dict(n_sel=z(B, Lq + 1, dtype=i32)),
                dict(indices=z(B, Lq, K, dtype=torch.int64))):
        with pytest.raises((ValueError, TypeError)):
            lsa.lsa_index_topk(**idx_inputs(), topk=K, init_tokens=2, local_tokens=4, **bad)
        with pytest.raises((ValueError, TypeError)):
            lsa.lsa_topk_select(z(B, Lq, S, dtype=f32), z(B, dtype=i32), K, 2, 4, **bad)
    with pytest.raises(ValueError, match="seqlens"):
        lsa.lsa_topk_select(z(B, Lq, S, dtype=f32), z(B + 1, dtype=i32), K, 2, 4)


def test_host_tensors_refused():
    with pytest.raises(ValueError, match="device"):
        lsa.lsa_index_scores(**idx_inputs())


def mla_args(**over):
    a = dict(q=z(B, H, DQK), kv=z(B, S, DQK), indices=z(B, K, dtype=i32), n_sel=z(B, dtype=i32),
             seqlens=z(B, dtype=i32), Dv=DV, softmax_scale=0.1)
    a.update(over)
    return a


@pytest.mark.parametrize("over", [
    dict(kv=z(B + 1, S, DQK)),
    dict(kv=z(B, S, DQK + 16)),
    dict(indices=z(B + 1, K, dtype=i32)),
    dict(indices=z(B, 1, K, dtype=i32)),
    dict(n_sel=z(B + 1, dtype=i32)),
    dict(n_sel=None),
    dict(seqlens=z(B - 1, dtype=i32)),
    dict(out=z(B, H, DV + 1)),
    dict(out=z(B, H, DV, dtype=f32)),
    dict(lse=z(B, H + 1, dtype=f32)),
    dict(lse=z(B, H, dtype=bf)),
])
def test_decode_attention_mismatch(over):
    with pytest.raises((ValueError, TypeError)):
        lsa.lsa_sparse_mla_decode(**mla_args(**over))


@pytest.mark.parametrize("over", [
    dict(q=z(B, Lq + 1, H, DQK), kv=z(B, S, DQK), indices=z(B, Lq, K, dtype=i32)),
    dict(out=z(B, 2, H, DV + 1)),
    dict(lse=z(B, 2, H + 1, dtype=f32)),
    dict(n_sel=z(B, 3, dtype=i32)),
])
def test_prefill_attention_mismatch(over):
    a = dict(q=z(B, 2, H, DQK), kv=z(B, S, DQK), indices=z(B, 2, K, dtype=i32),
             n_sel=z(B, 2, dtype=i32), seqlens=z(B, dtype=i32), Dv=DV, softmax_scale=0.1)
    a.update(over)
    with pytest.raises((ValueError, TypeError)):
        lsa.lsa_sparse_mla_prefill(**a)


@pytest.mark.parametrize("over", [
    dict(index_seqlens=z(B + 1, dtype=i32)),
    dict(n_sel=z(B, 1, dtype=i32)),
    dict(kv=z(B, S, DQK - 16)),
    dict(out=z(B, H + 1, DV)),
])
def test_draft_attention_mismatch(over):
    a = dict(q=z(B, H, DQK), kv=z(B, S, DQK), indices=z(B, K, dtype=i32), n_sel=z(B, dtype=i32),
             index_seqlens=z(B, dtype=i32), seqlens=z(B, dtype=i32), Dv=DV, softmax_scale=0.1)
    a.update(over)
    with pytest.raises((ValueError, TypeError)):
        lsa.lsa_mtp_draft_attention(**a)


def test_hier_outputs_mismatch():
    a = dict(q_idx=z(B, Hi, Di), w=z(B, Hi, dtype=f32), k_idx=z(B, S, Di),
             block_keys=z(B, S // 8, Di), seqlens=z(B, dtype=i32), topk=K, init_tokens=2,
             local_tokens=4, Bk=8, M=4)
    for bad in (dict(indices=z(B, K + 1, dtype=i32)), dict(n_sel=z(B + 1, dtype=i32)),
                dict(block_keys=z(B, S // 8 + 1, Di))):
        with pytest.raises(ValueError):
            lsa.lsa_hier_index_topk(**{**a, **bad})


def test_frontend_outputs_mismatch():
    a = dict(cq=z(B, Lq, 32), hid=z(B, Lq, 48), wq_b=z(Hi * Di, 32), wk=z(Di, 48),
             k_norm_gain=z(Di, dtype=f32), w_proj=z(Hi, 48), seqlens=z(B, dtype=i32),
             k_cache=z(B, S, Di))
    for bad in (dict(q_idx=z(B, Lq, Hi, Di + 2)), dict(w=z(B, Lq, Hi + 1, dtype=f32)),
                dict(k_cache=z(B, S, Di + 2)), dict(wq_b=z(Hi * Di + 1, 32))):
        with pytest.raises(ValueError):
            lsa.lsa_index_frontend(**{**a, **bad})
