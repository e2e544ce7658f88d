"""Named synthetic workloads of the LSA hot path and their seeded inputs.

Shapes follow the pages' model configuration (index_n_heads 32, index_head_dim 128,
index_topk 2048, index_init_tokens 16, index_local_tokens 1024; 32 attention heads with a
512-wide latent plus 64 rope dims, softmax scale 1/sqrt(128 + 64)) and their long-context
settings (128K decode, 128K chunked prefill, 983040-token context).  Inputs come from the
counter-based generator in ``inputs.py``: index queries/keys are dyadic (so scores are exact
in fp32 and index sets can be compared bit for bit), weights are positive dyadic, the MLA
query and latent cache are unit-variance bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import inputs as gen


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S_max: int
    Lq: int
    seqlens: tuple
    Hi: int = 32
    Di: int = 128
    topk: int = 2048
    init: int = 16
    local: int = 1024
    H: int = 32
    Dqk: int = 576
    Dv: int = 512
    scale: float = 1.0 / math.sqrt(192.0)
    mla_calls: int = 1
    # multi-token-prediction draft steps on one index pass (0: none).  Draft step c runs at
    # length seqlens[b] + c on cache kv0 with its own query q{c}.
    draft_steps: int = 0
    # hierarchical indexing: block size and blocks kept (0: the exact indexer)
    hier_block: int = 0
    hier_keep: int = 0
    seed: int = 1000
    notes: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.B * self.Lq

    @property
    def decode(self) -> bool:
        return self.Lq == 1

    @property
    def attn_calls(self) -> int:
        """Attention calls per step (draft steps share one cache; sub-blocks have their own)."""
        return self.draft_steps or self.mla_calls

    def attn_inputs(self, c: int):
        """(query, cache, positions appended since the index pass) of attention call c."""
        return f"q{c}", ("kv0" if self.draft_steps else f"kv{c}"), (c if self.draft_steps else 0)


def _wl(name, B, S, Lq=1, seqlens=None, **kw):
    return Workload(name=name, B=B, S_max=S, Lq=Lq,
                    seqlens=tuple(seqlens if seqlens is not None else [S] * B), **kw)


TINY = dict(Hi=4, Di=32, topk=256, init=4, local=64, H=4, Dqk=80, Dv=64, scale=1.0 / math.sqrt(80.0))

WORKLOADS = {
    # 1 cache of 4096 tokens, 4 decode queries at the last positions, plus a short sequence of
    # 200 tokens (n <= topk: dense fallback)
    "tiny_decode": _wl("tiny_decode", 5, 4096, seqlens=[4093, 4094, 4095, 4096, 200], seed=1000,
                       **TINY),
    "decode_32k": _wl("decode_32k", 8, 32768, seed=1001),
    # the headline: one index + top-k pass shared by the layer's two attention sub-blocks
    "decode_128k": _wl("decode_128k", 32, 131072, mla_calls=2, seed=1002),
    "prefill_128k": _wl("prefill_128k", 1, 131072, Lq=4096, seed=1003),
    "decode_1m": _wl("decode_1m", 4, 983040, seed=1004),
    # multi-token prediction: one index pass at 131070 tokens serves three draft steps (lengths
    # 131070, 131071, 131072), each attending to the selection plus the tokens drafted since
    "mtp_decode_128k": _wl("mtp_decode_128k", 32, 131072, seqlens=[131070] * 32, draft_steps=3,
                           seed=1005),
    # hierarchical indexing on the decode_128k shapes: blocks of 64 keys, the 32 best kept (twice
    # the middle budget of 2048 - 16 - 1024 tokens); same inputs as decode_128k
    "hier_decode_128k": _wl("hier_decode_128k", 32, 131072, mla_calls=2, hier_block=64,
                            hier_keep=32, seed=1002),
}


def tensor_specs(wl: Workload):
    """name -> (tag, shape, kind) of every input tensor."""
    specs = {
        "qidx": (gen.TAGS["qidx"], (wl.B, wl.Lq, wl.Hi, wl.Di), gen.DYADIC),
        "w": (gen.TAGS["w"], (wl.B, wl.Lq, wl.Hi), gen.WEIGHT),
        "kidx": (gen.TAGS["kidx"], (wl.B, wl.S_max, wl.Di), gen.DYADIC),
        "q0": (gen.TAGS["q"], (wl.B, wl.Lq, wl.H, wl.Dqk), gen.NORMAL),
        "kv0": (gen.TAGS["kv0"], (wl.B, wl.S_max, wl.Dqk), gen.NORMAL),
    }
    if wl.mla_calls > 1:
        specs["q1"] = (gen.TAGS["q1"], (wl.B, wl.Lq, wl.H, wl.Dqk), gen.NORMAL)
        specs["kv1"] = (gen.TAGS["kv1"], (wl.B, wl.S_max, wl.Dqk), gen.NORMAL)
    for c in range(1, wl.draft_steps):
        specs[f"q{c}"] = (gen.TAGS[f"q{c}"], (wl.B, wl.Lq, wl.H, wl.Dqk), gen.NORMAL)
    return specs


def device_inputs(wl: Workload, device="cuda"):
    """All inputs generated directly in device memory; q tensors are [B, Lq, H, Dqk]."""
    import torch

    X = {}
    for name, (tag, shape, kind) in tensor_specs(wl).items():
        X[name] = gen.device_tensor(wl.seed, tag, shape, kind, device=device)
    X["seqlens"] = torch.tensor(wl.seqlens, dtype=torch.int32, device=device)
    return X


def host_slice(wl: Workload, name: str, b: int) -> np.ndarray:
    """Sequence b of input `name` generated on the host (same bits as the device tensor)."""
    tag, shape, kind = tensor_specs(wl)[name]
    per = int(np.prod(shape[1:]))
    return gen.host_tensor(wl.seed, tag, shape[1:], kind, start=b * per)


def host_kv_rows(wl: Workload, name: str, b: int, positions) -> np.ndarray:
    """Latent rows `positions` of sequence b of cache `name` -> [len(positions), Dqk] bf16 bits."""
    tag, shape, kind = tensor_specs(wl)[name]
    rows = np.asarray(positions, dtype=np.int64) + b * wl.S_max
    return gen.host_rows(wl.seed, tag, rows, wl.Dqk, kind)
