"""Host-only checks of the C ABI: the library loads, exports every function include/lsa.h
declares, and rejects bad arguments before enqueueing anything (no GPU needed: every call
below returns during argument checking)."""
import ctypes
import os
import re

import pytest

from long_context_sparse_lightning_amd import lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "lsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for f in ("lsa_index_scores", "lsa_topk_select", "lsa_sparse_mla_decode",
              "lsa_sparse_mla_prefill"):
        assert f in names


def test_library_exports_every_declared_symbol():
    L = lsa.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} not exported by liblsa.so"
    assert sorted(lsa.EXPORTED) == declared_functions()


def test_status_strings():
    L = lsa.lib()
    for code, name in lsa.STATUS.items():
        assert L.lsa_status_str(code).decode() == name
    assert L.lsa_status_str(99).decode() == "LSA_ERR_UNKNOWN"


def _err():
    return lsa.lib().lsa_last_error().decode()


def test_index_scores_argument_errors():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    assert L.lsa_index_scores(None, None, None, None, 2, 1, 32, 128, 100, None, None) == 1
    assert "NULL" in _err()
    assert L.lsa_index_scores(p, p, p, p, -1, 1, 32, 128, 100, p, None) == 2
    assert L.lsa_index_scores(p, p, p, p, 1, 1, 0, 128, 100, p, None) == 2
    assert L.lsa_index_scores(p, p, p, p, 1, 1, 33, 128, 100, p, None) == 3
    assert L.lsa_index_scores(p, p, p, p, 1, 1, 32, 96, 100, p, None) == 3
    assert "Di=96" in _err()
    # empty batch: valid no-op even with NULL pointers
    assert L.lsa_index_scores(None, None, None, None, 0, 1, 32, 128, 100, None, None) == 0
    assert _err() == ""


def test_topk_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    assert L.lsa_topk_select(p, p, 1, 1, 4096, 8, 5, 4, p, p, None, 0, None) == 2  # init+local>topk
    # positions beyond the LDS bitmap of one row are rejected
    assert L.lsa_topk_select(p, p, 1, 1, (1 << 20) + 1, 2048, 16, 1024, p, p, None, 0, None) == 3
    assert "S_max" in _err()
    assert L.lsa_topk_select(None, p, 1, 1, 4096, 256, 4, 64, p, p, None, 0, None) == 1
    need = L.lsa_topk_workspace_bytes(32, 1, 131072, 2048, 16, 1024)
    assert need > 0
    assert L.lsa_topk_select(p, p, 32, 1, 131072, 2048, 16, 1024, p, p, None, 0, None) == 4
    assert L.lsa_topk_select(p, p, 32, 1, 131072, 2048, 16, 1024, p, p, p, need - 1, None) == 4
    assert "need" in _err()
    assert L.lsa_topk_workspace_bytes(1, 1, 4096, 8, 5, 4) == 0  # invalid -> 0
    assert L.lsa_topk_workspace_bytes(1, 1, (1 << 20) + 1, 2048, 16, 1024) == 0


def test_index_topk_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    f = L.lsa_index_topk
    assert f(p, p, p, p, 1, 1, 33, 128, 4096, 256, 4, 64, p, p, p, 1 << 30, None) == 3  # Hi > 32
    assert f(p, p, p, p, 1, 1, 32, 96, 4096, 256, 4, 64, p, p, p, 1 << 30, None) == 3  # Di
    assert f(p, p, p, p, 1, 1, 32, 128, 4096, 8, 5, 4, p, p, p, 1 << 30, None) == 2  # init+local
    assert f(p, p, p, p, 1, 1, 32, 128, (1 << 20) + 1, 2048, 16, 1024, p, p, p, 1 << 30, None) == 3
    assert f(p, None, p, p, 1, 1, 32, 128, 4096, 256, 4, 64, p, p, p, 1 << 30, None) == 1
    need = L.lsa_index_topk_workspace_bytes(32, 1, 131072, 2048, 16, 1024)
    assert need > 0
    assert f(p, p, p, p, 32, 1, 32, 128, 131072, 2048, 16, 1024, p, p, p, need - 1, None) == 4
    assert "need" in _err()
    assert f(None, None, None, None, 0, 1, 32, 128, 4096, 256, 4, 64, None, None, None, 0, None) == 0
    assert L.lsa_index_topk_workspace_bytes(1, 1, 4096, 8, 5, 4) == 0  # invalid -> 0


def test_index_topk_noalloc_argument_errors():
    """The static-workspace variant checks like lsa_index_topk and refuses sizes whose workspace
    exceeds LSA_INDEX_TOPK_SCRATCH_BYTES, all before touching a device."""
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    f = L.lsa_index_topk_noalloc
    assert f(p, p, p, p, 1, 1, 33, 128, 4096, 256, 4, 64, p, p, None) == 3  # Hi > 32
    assert f(p, p, p, p, 1, 1, 32, 128, 4096, 8, 5, 4, p, p, None) == 2  # init + local > topk
    assert f(p, None, p, p, 1, 1, 32, 128, 4096, 256, 4, 64, p, p, None) == 1
    assert f(None, None, None, None, 0, 1, 32, 128, 4096, 256, 4, 64, None, None, None) == 0
    big = L.lsa_index_topk_workspace_bytes(256, 1, 131072, 2048, 16, 1024)
    assert big > lsa.INDEX_TOPK_SCRATCH_BYTES
    assert f(p, p, p, p, 256, 1, 32, 128, 131072, 2048, 16, 1024, p, p, None) == 4
    assert "static" in _err()
    # the bench shapes fit
    for B, S in ((32, 131072), (8, 32768), (4, 983040)):
        assert L.lsa_index_topk_workspace_bytes(B, 1, S, 2048, 16, 1024) <= lsa.INDEX_TOPK_SCRATCH_BYTES


def test_mla_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    dec = L.lsa_sparse_mla_decode
    assert dec(p, p, p, p, p, 4, 32, 576, 640, 1000, 64, 0.1, p, None, p, 1 << 30, None) == 2
    assert dec(p, p, p, p, p, 4, 32, 512, 448, 1000, 64, 0.1, p, None, p, 1 << 30, None) == 3
    assert dec(p, p, p, None, p, 4, 32, 576, 512, 1000, 64, 0.1, p, None, p, 1 << 30, None) == 1
    assert dec(p, p, p, p, p, 4, 32, 576, 512, 1000, 0, 0.1, p, None, p, 1 << 30, None) == 2
    assert dec(p, p, p, p, p, 4, 32, 576, 512, 1000, 64, float("nan"), p, None, p, 1 << 30,
               None) == 2
    assert dec(p, p, p, p, p, 4, 32, 576, 512, 1 << 20, 131073, 0.1, p, None, p, 1 << 30, None) == 3
    assert L.lsa_mla_workspace_bytes(4, 1, 32, 512, 1 << 20, 131073, 0) == 0
    need = L.lsa_mla_workspace_bytes(32, 1, 32, 512, 131072, 2048, 0)
    assert need > 0
    assert dec(p, p, p, p, p, 32, 32, 576, 512, 131072, 2048, 0.07, p, None, None, 0, None) == 4
    pre = L.lsa_sparse_mla_prefill
    assert pre(p, p, None, None, p, 0, 10, 32, 576, 512, 100, 0, 0.1, None, None, None, 0,
               None) == 0
    # many query rows: one workgroup per row, no partials -> no workspace
    assert L.lsa_mla_workspace_bytes(1, 4096, 32, 512, 131072, 2048, 0) == 0


def test_hierarchical_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    bk = L.lsa_block_keys
    assert bk(p, p, 2, 4096, 128, 48, 0, p, None) == 3  # not a power of two
    assert bk(p, p, 2, 4096, 128, 4, 0, p, None) == 3 and bk(p, p, 2, 4096, 128, 2048, 0, p, None) == 3
    assert bk(p, p, 2, 4096, 120, 64, 0, p, None) == 3 and bk(p, p, 2, 32, 128, 64, 0, p, None) == 3
    assert bk(p, p, 2, 4096, 128, 64, -1, p, None) == 2 and bk(p, None, 2, 4096, 128, 64, 0, p, None) == 1
    h = L.lsa_hier_index_topk

    def call(Hi=32, Di=128, topk=2048, init=16, local=1024, Bk=64, M=32, bk_=p, ws=p, wbytes=1 << 30):
        return h(p, p, p, bk_, p, 4, Hi, Di, 131072, topk, init, local, Bk, M, p, p, ws, wbytes, None)

    assert call(Hi=33) == 3 and call(Di=120) == 3 and call(Bk=96) == 3
    assert call(M=0) == 2 and call(M=2049) == 2 and call(init=1500) == 2
    assert call(M=15) == 2  # 15 * 64 < topk - local: too few candidates
    assert call(bk_=None) == 1
    need = L.lsa_hier_workspace_bytes(4, 131072, 64, 2048, 16, 1024, 32)
    assert 0 < need < 16 << 20
    assert call(wbytes=need - 1) == 4 and call(ws=None, wbytes=0) == 4
    assert L.lsa_hier_workspace_bytes(4, 131072, 64, 2048, 16, 1024, 0) == 0


def test_index_frontend_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    fe = L.lsa_index_frontend

    def call(B=2, Lq=1, ql=1536, hd=3072, Hi=32, Di=128, R=64, theta=1e6, eps=1e-6, gain=p,
             ws=p, wbytes=1 << 30):
        return fe(p, p, p, p, gain, p, p, B, Lq, ql, hd, Hi, Di, R, theta, eps, 100, p, p, p, ws,
                  wbytes, None)

    assert call(R=63) == 2 and call(R=130) == 2 and call(Di=127, R=64) == 2
    assert call(ql=1530) == 3 and call(Di=256, R=64) == 3 and call(Hi=33) == 3
    assert call(theta=0.0) == 2 and call(theta=float("inf")) == 2 and call(eps=-1.0) == 2
    assert call(eps=float("nan")) == 2
    assert call(gain=None) == 1
    need = L.lsa_index_frontend_workspace_bytes(32, 1, 1536, 3072, 32, 128)
    assert 0 < need < 64 << 20
    assert call(B=32, wbytes=need - 1) == 4 and call(B=32, ws=None, wbytes=0) == 4
    assert fe(None, None, None, None, None, None, None, 0, 1, 1536, 3072, 32, 128, 64, 1e6, 1e-6,
              100, None, None, None, None, 0, None) == 0
    assert L.lsa_index_frontend_workspace_bytes(32, 1, 1530, 3072, 32, 128) == 0
    # prefill-sized calls stay modest: the query is rotated in its projection's epilogue, so only
    # the key/weight partials and the angle table remain
    assert L.lsa_index_frontend_workspace_bytes(1, 4096, 1536, 3072, 32, 128) <= 32 << 20


def test_mtp_draft_argument_errors_and_workspace():
    L = lsa.lib()
    p = ctypes.c_void_p(16)
    f = L.lsa_mtp_draft_attention

    def call(B=4, Dqk=576, Dv=512, topk=2048, app=3, idx=p, nsel=p, iseq=p, ws=p, wbytes=1 << 30):
        return f(p, p, idx, nsel, iseq, p, B, 32, Dqk, Dv, 131072, topk, app, 0.07, p, None, ws,
                 wbytes, None)

    assert call(app=-1) == 2 and call(app=65) == 2 and call(topk=0) == 2
    assert call(topk=65537) == 3 and L.lsa_mtp_draft_workspace_bytes(4, 32, 512, 1 << 20, 65537, 3) == 0
    assert call(Dqk=512, Dv=448) == 3
    assert call(idx=None) == 1 and call(nsel=None) == 1 and call(iseq=None) == 1
    need = L.lsa_mtp_draft_workspace_bytes(32, 32, 512, 131072, 2048, 3)
    assert need > 0 and need == L.lsa_mla_workspace_bytes(32, 1, 32, 512, 131072, 2048, 0)
    assert call(B=32, wbytes=need - 1) == 4 and call(B=32, ws=None, wbytes=0) == 4
    assert f(None, None, None, None, None, None, 0, 32, 576, 512, 100, 64, 3, 0.1, None, None,
             None, 0, None) == 0
    assert L.lsa_mtp_draft_workspace_bytes(32, 32, 512, 131072, 2048, 65) == 0
    # one split per row of 2048 at 512 rows: the appended positions push it to two
    assert L.lsa_mtp_draft_workspace_bytes(512, 32, 512, 131072, 2048, 3) > 0
    assert L.lsa_mla_workspace_bytes(512, 1, 32, 512, 131072, 2048, 0) == 0


@pytest.mark.parametrize("name", ["tiny_decode", "decode_32k", "decode_128k", "prefill_128k",
                                  "decode_1m"])
def test_workspace_sizes_are_modest(name):
    from long_context_sparse_lightning_amd.workloads import WORKLOADS

    wl = WORKLOADS[name]
    t = lsa.lsa_topk_workspace_bytes(wl.B, wl.Lq, wl.S_max, wl.topk, wl.init, wl.local)
    f = lsa.lsa_index_topk_workspace_bytes(wl.B, wl.Lq, wl.S_max, wl.topk, wl.init, wl.local)
    m = lsa.lsa_mla_workspace_bytes(wl.B, wl.Lq, wl.H, wl.Dv, wl.S_max, wl.topk, False)
    # the standalone top-k groups rows under a 1 GiB candidate budget (plus list lengths and
    # bounds); the fused call and the attention stay far smaller
    assert 0 <= t <= (1 << 30) + (16 << 20) and 0 < f <= 512 << 20 and 0 <= m <= 256 << 20


def test_binding_rejects_host_tensors():
    import torch

    with pytest.raises(ValueError):
        lsa.lsa_index_scores(torch.zeros(1, 1, 4, 32, dtype=torch.bfloat16),
                             torch.zeros(1, 1, 4), torch.zeros(1, 64, 32, dtype=torch.bfloat16),
                             torch.tensor([64], dtype=torch.int32))


def test_check_seqlens_host_side():
    """The precondition check of LSA_DEBUG_BOUNDS mode on host arrays: Lq <= seqlens[b] <= S_max."""
    assert lsa.check_seqlens([5, 100, 1000], 1, 1000) == -1
    assert lsa.check_seqlens([5, 100, 1001], 1, 1000) == 2     # beyond the cache
    assert lsa.check_seqlens([5, 0, 1000], 1, 1000) == 1       # no room for the query
    assert lsa.check_seqlens([50, 49], 50, 100) == 1           # prefill chunk longer than seq
    assert lsa.check_seqlens([-3], 0, 10) == 0
    assert lsa.check_seqlens([], 1, 10) == -1
    assert lsa.check_seqlens([0, 10], 0, 10) == -1             # block keys: Lq = 0
