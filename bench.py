#!/usr/bin/env python3
"""Benchmark of the LSA hot path on one MI355X: lightning indexer -> top-2048 (sink/window
forced) -> sparse absorbed-MLA over the selected latent rows, through the C ABI.

Default workload: 128K-context decode, batch 32, one index + top-k pass shared by the layer's
two attention sub-blocks (two MLA calls).  A step is one pass of the whole path over the
batch; inputs are generated in HBM before timing.  Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--path fused|split]
                  [--no-cpu-baseline]

--path fused (the default for decode workloads) runs the indexer and the top-k in one call
(lsa_index_topk: the scores never leave the chip); --path split (the default for prefill
workloads, where the query-blocked scan is the faster indexer) runs lsa_index_scores then
lsa_topk_select.  Both give the same indices bit for bit.

Passes: (1) the headline, K steps between two events; (2) the same K steps with an event at
every call boundary (per-call durations, roofline, spread); (3) up to 50 steps each preceded by a
1 GiB read that evicts the caches (cold-cache figure, and the read's rate as context); (4) the
indexer front end (lsa_index_frontend) at the same shape, reported under `stages` only.  The CPU-oracle leg also re-checks parity on the sampled rows of the timed
run's output buffers.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "LSA decode queries/s @128K ctx (indexer+top-2048+MLA); % HBM peak GB/s"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, public spec
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_128k")
    ap.add_argument("--path", choices=("fused", "split"), default=None,
                    help="default: fused for decode workloads, split for prefill ones (the "
                         "query-blocked prefill scan writes the scores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="query rows the oracle times (0: auto)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this size (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(wl):
    """Bytes the method must move per step (per query row, summed): index keys of the visible
    positions, index query and weights, index write; per MLA call the selected latent rows, the
    query, the output and the index read.  The fp32 score round trip between the first two
    stages is excluded (reported separately)."""
    tot = 0
    score_rt = 0
    for b in range(wl.B):
        for i in range(wl.Lq):
            n = wl.seqlens[b] - wl.Lq + i + 1
            tot += index_keys_read(wl, n) * wl.Di * 2 + wl.Hi * wl.Di * 2 + wl.Hi * 4 + wl.topk * 4
            tot += sum(attn_row_bytes(wl, n, c) for c in range(wl.attn_calls))
            score_rt += 2 * n * 4
    return tot, score_rt


def index_keys_read(wl, n):
    """Key rows the index pass of a row with n visible positions must read: all n, or with
    hierarchical indexing the block keys before the window plus the tokens scored (the kept
    blocks and the partial block before the window; the sink and window are forced)."""
    if not wl.hier_block or n <= wl.topk:
        return n if not wl.hier_block else 0
    w0 = max(n - wl.local, 0)
    nb = w0 // wl.hier_block
    return nb + min(wl.hier_keep, nb) * wl.hier_block + (w0 - nb * wl.hier_block)


def attn_row_bytes(wl, n, c):
    """Attention call c of one query row whose index pass saw n positions: the selected latent
    rows (plus the draft positions appended since the pass), the query, the output and the
    index list."""
    rows = min(n, wl.topk) + wl.attn_inputs(c)[2]
    return rows * wl.Dqk * 2 + wl.H * wl.Dqk * 2 + wl.H * wl.Dv * 2 + wl.topk * 4


def attention_call_bytes(wl, c=0):
    """Algorithmic bytes of attention call c over the whole batch (decode rows)."""
    return sum(attn_row_bytes(wl, wl.seqlens[b] - wl.Lq + i + 1, c)
               for b in range(wl.B) for i in range(wl.Lq))


def indexer_bytes(wl):
    """Algorithmic bytes of one indexer launch: keys of the visible positions, the index query
    and weights, and the fp32 score written per visible position."""
    tot = 0
    for b in range(wl.B):
        for i in range(wl.Lq):
            n = wl.seqlens[b] - wl.Lq + i + 1
            tot += n * wl.Di * 2 + wl.Hi * wl.Di * 2 + wl.Hi * 4 + n * 4
    return tot


def indexer_flops(wl):
    """Algorithmic matrix-core flops of one indexer launch: the q.k products of every index head
    over every visible (query, key) pair, 2*Hi*Di each (the ReLU-weighted head sum is not counted)."""
    pairs = sum(wl.seqlens[b] - wl.Lq + i + 1 for b in range(wl.B) for i in range(wl.Lq))
    return 2 * wl.Hi * wl.Di * pairs


def query_blocked(wl):
    """True when lsa_index_scores runs the query-blocked scan for this shape (16 query rows per
    workgroup share each key tile; a dense contraction, bound by the matrix cores)."""
    return wl.Di == 128 and wl.Lq >= 16


def hier_call_bytes(wl):
    """Algorithmic bytes of one lsa_hier_index_topk call: the block keys and token keys it must
    score, the index query and weights, the indices and n_sel."""
    return sum(index_keys_read(wl, wl.seqlens[b]) * wl.Di * 2 + wl.Hi * wl.Di * 2 + wl.Hi * 4
               + wl.topk * 4 + 4 for b in range(wl.B))


def fused_call_bytes(wl):
    """Algorithmic bytes of one lsa_index_topk call: keys of the visible positions, the index
    query and weights, and the indices and n_sel written."""
    tot = 0
    for b in range(wl.B):
        for i in range(wl.Lq):
            n = wl.seqlens[b] - wl.Lq + i + 1
            tot += n * wl.Di * 2 + wl.Hi * wl.Di * 2 + wl.Hi * 4 + wl.topk * 4 + 4
    return tot


FE_Q_LORA, FE_HIDDEN, FE_ROPE = 1536, 3072, 64  # q_lora_rank, hidden_size, qk_rope_head_dim


def frontend_cost(wl):
    """Algorithmic bytes and flops of one lsa_index_frontend call at the workload's shape: the
    three weight matrices, the token activations, the outputs (q_idx, w, the new keys)."""
    T = wl.B * wl.Lq
    wbytes = (wl.Hi * wl.Di * FE_Q_LORA + (wl.Di + wl.Hi) * FE_HIDDEN) * 2
    act = T * (FE_Q_LORA + FE_HIDDEN) * 2
    out = T * (wl.Hi * wl.Di * 2 + wl.Hi * 4 + wl.Di * 2)
    flops = 2 * T * (wl.Hi * wl.Di * FE_Q_LORA + (wl.Di + wl.Hi) * FE_HIDDEN)
    return wbytes + act + out, flops


def time_frontend(wl, dev, stream, calls=20):
    """Average duration (ms) of lsa_index_frontend at the workload's shape, on its own cache."""
    import torch

    from long_context_sparse_lightning_amd import inputs as gen
    from long_context_sparse_lightning_amd import lsa

    T = (wl.B, wl.Lq)
    t = lambda name, shape, kind: gen.device_tensor(wl.seed, gen.TAGS[name], shape, kind, device=dev)
    cq, hid = t("cq", T + (FE_Q_LORA,), gen.NORMAL), t("hid", T + (FE_HIDDEN,), gen.NORMAL)
    wq_b = t("wq_b", (wl.Hi * wl.Di, FE_Q_LORA), gen.NORMAL)
    wk, w_proj = t("wk", (wl.Di, FE_HIDDEN), gen.NORMAL), t("w_proj", (wl.Hi, FE_HIDDEN), gen.NORMAL)
    gain = t("k_gain", (wl.Di,), gen.WEIGHT)
    seqlens = torch.tensor(wl.seqlens, dtype=torch.int32, device=dev)
    cache = torch.empty(wl.B, wl.S_max, wl.Di, dtype=torch.bfloat16, device=dev)
    q = torch.empty(wl.B, wl.Lq, wl.Hi, wl.Di, dtype=torch.bfloat16, device=dev)
    w = torch.empty(wl.B, wl.Lq, wl.Hi, dtype=torch.float32, device=dev)
    ws = torch.empty(lsa.lsa_index_frontend_workspace_bytes(wl.B, wl.Lq, FE_Q_LORA, FE_HIDDEN, wl.Hi,
                                                            wl.Di), dtype=torch.uint8, device=dev)

    def call():
        lsa.lsa_index_frontend(cq, hid, wq_b, wk, gain, w_proj, seqlens, cache, rope_dim=FE_ROPE,
                               q_idx=q, w=w, workspace=ws)

    for _ in range(3):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(calls):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / calls


def host_cpu():
    """Model name and logical CPU count of the host (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            names = [l.split(":", 1)[1].strip() for l in f if l.startswith("model name")]
    except OSError:
        names = []
    return f"{names[0] if names else 'unknown CPU'} ({os.cpu_count()} logical CPUs on the host)"


def cpu_baseline(wl, sample_rows, gpu=None):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload.  With `gpu`
    (host copies of the timed run's indices, n_sel and attention outputs) also re-check parity
    on the sampled rows: indices bit for bit, attention within max|err| <= 1e-2 max|ref| and
    relative L2 <= 5e-3."""
    import numpy as np

    import oracle
    from long_context_sparse_lightning_amd.workloads import host_kv_rows, host_slice

    every = [(b, i) for b in range(wl.B) for i in range(wl.Lq)]
    if sample_rows >= len(every):  # whole steps, repeated
        rows = [every[j % len(every)] for j in range(sample_rows)]
    else:
        step = max(1, len(every) // sample_rows)
        rows = every[::step][:sample_rows]
    # inputs first (not timed)
    prepared = []
    for b, i in rows:
        p = wl.seqlens[b] - wl.Lq + i
        prepared.append((b, i, p, host_slice(wl, "qidx", b)[i:i + 1][None],
                         host_slice(wl, "w", b)[i:i + 1][None],
                         host_slice(wl, "kidx", b)[None, : p + 1],
                         [host_slice(wl, wl.attn_inputs(c)[0], b)[i][None, None]
                          for c in range(wl.attn_calls)]))
    cores = oracle.max_threads()
    t_total = 0.0
    checked, idx_equal, worst_max, worst_l2 = set(), True, 0.0, 0.0
    for b, i, p, qi, w, k, qs in prepared:
        n = p + 1
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        if wl.hier_block:
            hi, hn = oracle.hier_topk(qi[:, 0], w[:, 0], k, sl, wl.topk, wl.init, wl.local,
                                      wl.hier_block, wl.hier_keep)
            idx, nsel = hi[:, None], hn[:, None]
        else:
            sc = oracle.index_scores(qi, w, k, sl, 1)
            idx, nsel = oracle.topk_select(sc, sl, wl.topk, wl.init, wl.local)
        t_total += time.perf_counter() - t0
        # each call's selection: the pass's, plus the positions drafted since (draft steps)
        sels = [oracle.mtp_draft_indices(idx[:, 0], nsel[:, 0], sl, sl + wl.attn_inputs(c)[2],
                                         wl.draft_steps)[0][0, 0] if wl.draft_steps
                else idx[0, 0] for c in range(wl.attn_calls)]
        sels = [s_[s_ >= 0] if wl.draft_steps else s_[: nsel[0, 0]] for s_ in sels]
        kvs = [host_kv_rows(wl, wl.attn_inputs(c)[1], b, sels[c])[None] for c in range(wl.attn_calls)]
        t0 = time.perf_counter()
        refs = [oracle.sparse_mla(qs[c], kvs[c], np.arange(sels[c].size, dtype=np.int32)[None, None],
                                  np.array([[sels[c].size]], np.int32),
                                  np.array([sels[c].size], np.int32), wl.Dv, wl.scale)[0]
                for c in range(wl.attn_calls)]
        t_total += time.perf_counter() - t0
        if gpu is not None and (b, i) not in checked:  # not timed
            checked.add((b, i))
            g_idx, g_nsel, g_outs = gpu
            idx_equal &= bool(int(g_nsel[b, i]) == int(nsel[0, 0])
                              and np.array_equal(g_idx[b, i].cpu().numpy(), idx[0, 0]))
            for c in range(wl.attn_calls):
                ref = refs[c][0, 0]
                err = g_outs[c][b, i].float().cpu().numpy().astype(np.float64) - ref
                worst_max = max(worst_max, float(np.abs(err).max() / max(np.abs(ref).max(), 1e-300)))
                worst_l2 = max(worst_l2, float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300)))
    res = {"value": len(rows) / t_total, "unit": "queries/s", "cores": cores, "kind": "oracle",
           "cpu": host_cpu(),
           "sample": f"{len(rows)} query-row evaluations over the {len(every)} query rows of "
                     f"{wl.name} (each: full indexer scan, top-k and {wl.attn_calls} MLA call(s)); "
                     f"{t_total:.2f} s wall on {cores} threads"}
    if gpu is not None:
        res["parity_on_timed_buffers"] = {
            "rows": len(checked), "indices_bit_exact": idx_equal,
            "attention_max_err_over_max_ref": float(f"{worst_max:.3e}"),
            "attention_rel_l2": float(f"{worst_l2:.3e}"),
            "pass": bool(idx_equal and worst_max <= 1e-2 and worst_l2 <= 5e-3)}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        return 2

    import torch

    from long_context_sparse_lightning_amd import lsa
    from long_context_sparse_lightning_amd.pmc import load_traffic
    from long_context_sparse_lightning_amd.workloads import WORKLOADS, device_inputs

    wl = WORKLOADS[args.workload]
    if wl.hier_block:
        args.path = "hier"
    elif args.path is None:
        args.path = "fused" if wl.decode else "split"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    X = device_inputs(wl, device=dev)
    B, Lq = wl.B, wl.Lq
    scores = None if args.path in ("fused", "hier") else torch.empty(B, Lq, wl.S_max, dtype=torch.float32,
                                                             device=dev)
    idx = torch.empty(B, Lq, wl.topk, dtype=torch.int32, device=dev)
    nsel = torch.empty(B, Lq, dtype=torch.int32, device=dev)
    fused = args.path == "fused"
    hier = args.path == "hier"
    if hier:
        # the block summary of the cache: built once here, maintained block by block as a cache
        # grows (one block completes every hier_block decode steps)
        bkeys = torch.zeros(B, wl.S_max // wl.hier_block, wl.Di, dtype=torch.bfloat16, device=dev)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lsa.lsa_block_keys(X["kidx"], X["seqlens"], wl.hier_block, block_keys=bkeys)
        torch.cuda.synchronize()
        ev0.record()
        lsa.lsa_block_keys(X["kidx"], X["seqlens"], wl.hier_block, block_keys=bkeys)
        ev1.record()
        torch.cuda.synchronize()
        block_keys_ms = ev0.elapsed_time(ev1)
        tws = torch.empty(lsa.lsa_hier_workspace_bytes(B, wl.S_max, wl.hier_block, wl.topk, wl.init,
                                                       wl.local, wl.hier_keep), dtype=torch.uint8,
                          device=dev)
    elif fused:
        tws = torch.empty(max(1, lsa.lsa_index_topk_workspace_bytes(B, Lq, wl.S_max, wl.topk, wl.init,
                                                                    wl.local)), dtype=torch.uint8, device=dev)
    else:
        tws = torch.empty(max(1, lsa.lsa_topk_workspace_bytes(B, Lq, wl.S_max, wl.topk, wl.init,
                                                              wl.local)), dtype=torch.uint8, device=dev)
    if wl.draft_steps:
        mws_bytes = lsa.lsa_mtp_draft_workspace_bytes(B, wl.H, wl.Dv, wl.S_max, wl.topk, wl.draft_steps)
        draft_seqlens = [X["seqlens"] + c for c in range(wl.draft_steps)]
    else:
        mws_bytes = lsa.lsa_mla_workspace_bytes(B, Lq, wl.H, wl.Dv, wl.S_max, wl.topk, False)
    mws = torch.empty(max(1, mws_bytes), dtype=torch.uint8, device=dev)
    outs = [torch.empty(B, Lq, wl.H, wl.Dv, dtype=torch.bfloat16, device=dev)
            for _ in range(wl.attn_calls)]
    lses = [torch.empty(B, Lq, wl.H, dtype=torch.float32, device=dev) for _ in range(wl.attn_calls)]
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        # ev: events recorded on the launch stream at the stage boundaries of this step:
        # [start, after the indexer call, after top-k, after each attention call]
        if ev is not None:
            ev[0].record(stream)
        if hier:
            lsa.lsa_hier_index_topk(X["qidx"][:, 0], X["w"][:, 0], X["kidx"], bkeys, X["seqlens"],
                                    wl.topk, wl.init, wl.local, wl.hier_block, wl.hier_keep,
                                    indices=idx[:, 0], n_sel=nsel[:, 0], workspace=tws)
        elif fused:
            lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init,
                               wl.local, indices=idx, n_sel=nsel, workspace=tws)
        else:
            lsa.lsa_index_scores(X["qidx"], X["w"], X["kidx"], X["seqlens"], scores=scores)
        if ev is not None:
            ev[1].record(stream)
        if not fused and not hier:
            lsa.lsa_topk_select(scores, X["seqlens"], wl.topk, wl.init, wl.local, indices=idx,
                                n_sel=nsel, workspace=tws)
        if ev is not None:
            ev[2].record(stream)
        for c in range(wl.attn_calls):
            if wl.draft_steps:  # draft step c on the shared index pass
                lsa.lsa_mtp_draft_attention(X[f"q{c}"][:, 0], X["kv0"], idx[:, 0], nsel[:, 0],
                                            X["seqlens"], draft_seqlens[c], wl.Dv, wl.scale,
                                            max_appended=wl.draft_steps, out=outs[c][:, 0],
                                            lse=lses[c][:, 0], workspace=mws)
            elif wl.decode:
                lsa.lsa_sparse_mla_decode(X[f"q{c}"][:, 0], X[f"kv{c}"], idx[:, 0], nsel[:, 0],
                                          X["seqlens"], wl.Dv, wl.scale, out=outs[c][:, 0],
                                          lse=lses[c][:, 0], workspace=mws)
            else:
                lsa.lsa_sparse_mla_prefill(X[f"q{c}"], X[f"kv{c}"], idx, nsel, X["seqlens"], wl.Dv,
                                           wl.scale, out=outs[c], lse=lses[c], workspace=mws)
            if ev is not None:
                ev[3 + c].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: warmup done", file=sys.stderr, flush=True)

    # Pass 1 (the headline): K steps between two events and nothing else on the stream.  A
    # timing event between kernels costs a few microseconds of queue bubble on this stack, so
    # the per-call boundaries are taken in pass 2.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = t_start.elapsed_time(t_end)
    print(f"[bench] timed {args.steps} steps: {elapsed_ms:.3f} ms (host wall {wall * 1e3:.3f} ms)",
          file=sys.stderr, flush=True)

    # Pass 2: the same K steps with an event at every call boundary, for the per-call durations
    # (roofline, stages) and the spread of step times.  The last stage of step s ends where step
    # s+1's first event is recorded (the same stream position).
    n_ev = 3 + wl.attn_calls
    step_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(step_ev[s])
    torch.cuda.synchronize()
    stage_ms = [[ev[j].elapsed_time(ev[j + 1]) for j in range(n_ev - 1)] for ev in step_ev]
    k1_ms = sum(st[0] for st in stage_ms) / args.steps
    step_list = sorted(step_ev[s][0].elapsed_time(step_ev[s + 1][0]) for s in range(args.steps - 1))

    recall = None
    if hier:
        # share of the exact selection (lsa_index_topk on the same inputs) the hierarchical one
        # keeps; synthetic keys have no block structure, so this is a floor
        e_idx, _ = lsa.lsa_index_topk(X["qidx"], X["w"], X["kidx"], X["seqlens"], wl.topk, wl.init,
                                      wl.local)
        torch.cuda.synchronize()
        hits = sum(len(set(idx[b, 0].tolist()) & set(e_idx[b, 0].tolist())) for b in range(B))
        recall = round(hits / (B * wl.topk), 4)

    ms_per_step = elapsed_ms / args.steps
    queries = B * Lq * (wl.draft_steps or 1)  # draft steps: one query per step and sequence
    value = queries * args.steps / (elapsed_ms / 1e3)
    alg, score_rt = algorithmic_bytes(wl)
    k1_bytes = (hier_call_bytes(wl) if hier else fused_call_bytes(wl) if fused
                else indexer_bytes(wl))
    k1_gbs = k1_bytes / (k1_ms / 1e3) / 1e9
    step_gbs = alg / (ms_per_step / 1e3) / 1e9
    mla_bytes = [attention_call_bytes(wl, c) for c in range(wl.attn_calls)]
    if hier:
        # the index pass reads a small fraction of the keys; the attention call dominates
        att_ms = sum(st[2 + c] for st in stage_ms for c in range(wl.attn_calls)) / (
            args.steps * wl.attn_calls)
        att_gbs = mla_bytes[0] / (att_ms / 1e3) / 1e9
        roofline = {"kernel": "lsa_sparse_mla_decode (sparse_mla_kernel<576,512,true> + "
                              "mla_combine_kernel)",
                    "bound": "hbm", "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_ms": round(att_ms, 5), "alg_bytes_per_launch": mla_bytes[0]}
    elif fused:
        roofline = {"kernel": "lsa_index_topk (index_scores_kernel<128,true> + topk_merge_kernel)",
                    "bound": "hbm", "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(wl.name, args.path), "avg_launch_ms": round(k1_ms, 5),
                    "alg_bytes_per_launch": k1_bytes}
    elif query_blocked(wl):
        flops = indexer_flops(wl)
        tfs = flops / (k1_ms / 1e3) / 1e12
        roofline = {"kernel": "lsa_index_scores (index_scores_qb_kernel)", "bound": "mfma",
                    "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "avg_launch_ms": round(k1_ms, 5), "alg_flops_per_launch": flops}
    else:
        roofline = {"kernel": "lsa_index_scores (index_scores_kernel<128,false>)", "bound": "hbm",
                    "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(wl.name, args.path), "avg_launch_ms": round(k1_ms, 5),
                    "alg_bytes_per_launch": k1_bytes}

    # Pass 3 (cold cache): each step preceded by a 1 GiB read (torch's sum reduction) that evicts
    # the L2 and the Infinity Cache with clean lines (a written flush would leave 1 GiB of dirty
    # lines for the next key stream to write back), events around each step (so each figure also
    # carries an event's queue bubble, as in pass 2).  The read's own rate is reported as
    # context; torch's reduction is not a tuned streaming kernel.
    flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    n_cold = min(args.steps, 50)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_cold)]
    torch.cuda.synchronize()
    for ev in cold_ev:
        ev[0].record(stream)
        torch.sum(flush, dim=0, out=sink)
        ev[1].record(stream)
        step()
        ev[2].record(stream)
    torch.cuda.synchronize()
    cold_ms = sorted(ev[1].elapsed_time(ev[2]) for ev in cold_ev)
    read_ms = sorted(ev[0].elapsed_time(ev[1]) for ev in cold_ev)
    del flush

    # Pass 4: the indexer front end (the next row after the hot path; not part of the headline
    # step) at the same shape, back to back
    fe_ms = time_frontend(wl, dev, stream)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        bcopy = torch.empty_like(a)
        torch.cuda.synchronize()
        bcopy.copy_(a)
        torch.cuda.synchronize()
        del a, bcopy

    def mean(j):
        return sum(st[j] for st in stage_ms) / args.steps

    mla_ms = [mean(2 + c) for c in range(wl.attn_calls)]

    def pct(q):
        return round(step_list[min(len(step_list) - 1, int(q * len(step_list)))], 5) if step_list else None

    # per-stage algorithmic bytes: the indexer call as in the roofline; top-k (split path) reads
    # the visible scores and writes the indices; an attention call gathers the selected rows and
    # moves q, out and the index list
    topk_bytes = sum((wl.seqlens[b] - wl.Lq + i + 1) * 4 + wl.topk * 4 + 4
                     for b in range(wl.B) for i in range(wl.Lq))
    # (rates only for decode: prefill rows share keys and selected rows, so per-row byte counts
    # do not measure HBM there)
    stages = {"index_call_ms": round(mean(0), 5)}
    if wl.decode:
        stages["index_call_gbs"] = round(k1_bytes / (mean(0) / 1e3) / 1e9, 1)
    if hier:
        stages["block_keys_build_ms"] = round(block_keys_ms, 5)
        stages["selection_recall_vs_exact"] = recall
    elif not fused:
        stages["topk_call_ms"] = round(mean(1), 5)
        stages["topk_call_gbs"] = round(topk_bytes / (mean(1) / 1e3) / 1e9, 1)
    for c in range(wl.attn_calls):
        stages[f"mla{c}_call_ms"] = round(mla_ms[c], 5)
        if wl.decode:
            stages[f"mla{c}_call_gbs"] = round(mla_bytes[c] / (mla_ms[c] / 1e3) / 1e9, 1)
    att_traffic = load_traffic(wl.name, "attention") if wl.decode and not wl.draft_steps else None
    if att_traffic:  # counter-measured HBM bytes of one attention call (current sources only)
        stages["mla_call_traffic_bytes"] = att_traffic
        stages["mla_call_traffic_over_alg"] = round(att_traffic / mla_bytes[0], 4)
    # the same step with one attention call (the shape of configurations with one sub-block)
    stages["one_mla_step_ms"] = round(mean(0) + mean(1) + mean(2), 5)
    # spread of step times in pass 2 (which carries the boundary events)
    stages["instrumented_step_ms_p10_p50_p90"] = [pct(0.1), pct(0.5), pct(0.9)]
    stages["cold_cache_step_ms_p10_p50_p90"] = [round(cold_ms[int(q * (n_cold - 1))], 5)
                                                 for q in (0.1, 0.5, 0.9)]
    fe_bytes, fe_flops = frontend_cost(wl)
    stages["frontend_call_ms"] = round(fe_ms, 5)
    stages["frontend_alg_bytes"] = fe_bytes
    if wl.decode:
        stages["frontend_gbs"] = round(fe_bytes / (fe_ms / 1e3) / 1e9, 1)
    else:
        stages["frontend_tflops"] = round(fe_flops / (fe_ms / 1e3) / 1e12, 1)
    stages["flush_torch_sum_1gib_gbs"] = round((1 << 30) / (read_ms[n_cold // 2] / 1e3) / 1e9, 1)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64; dyadic index q/k, unit-variance bf16 latent cache)",
        "config": {"workload": wl.name, "path": args.path, "batch": B, "context": wl.S_max, "query_tokens": Lq,
                   "index_heads": wl.Hi, "index_dim": wl.Di, "topk": wl.topk,
                   "init_tokens": wl.init, "local_tokens": wl.local, "mla_heads": wl.H,
                   "qk_dim": wl.Dqk, "v_dim": wl.Dv, "mla_calls_per_step": wl.attn_calls,
                   "draft_steps": wl.draft_steps, "hier_block": wl.hier_block,
                   "hier_keep": wl.hier_keep},
        "roofline": roofline,
        "stages": stages,
    }
    if wl.decode:
        # per-row byte accounting; in prefill the rows of one sequence share their keys, so a
        # per-row sum would count every key Lq times and is not reported
        line["hbm_frac_step"] = round(step_gbs / HBM_PEAK_GBS, 4)
        line["step_alg_bytes"] = alg
        line["step_score_roundtrip_bytes"] = score_rt
    if not args.no_cpu_baseline:
        # about 10 s of oracle work: three passes over the 32 decode rows of the 128K step
        sample = args.cpu_sample or (3 * B * Lq if wl.decode and B * Lq <= 64 else 64)
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, sample, gpu=(idx, nsel, outs))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    sys.exit(main())
