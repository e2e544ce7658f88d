/*
 * lsa.h -- C ABI of the MI355X (gfx950) LongCat Sparse Attention hot path.
 *
 * Four operations, in the order one attention layer calls them:
 *   lsa_index_scores       lightning-indexer scores of every cached key        (stage 1)
 *   lsa_topk_select        top-k positions with sink/window columns forced      (stage 2)
 *   lsa_sparse_mla_decode  absorbed-MLA attention over the selected latent rows (stage 3)
 *   lsa_sparse_mla_prefill the same for a chunk of Lq query tokens, causal      (stage 3)
 * and lsa_index_topk, stages 1 and 2 in one pass without the score array.
 *
 * Sources: the page "MLX-VLM 的 LongCat-Flash-Lite-Sparse 支持LSA 稀疏注意力、n-gram
 * 融合与预填充优化解析", sections "LSA" (indexer, top-k with forced columns, dense fallback,
 * decode gather, prefill mask, one index pass shared by both attention sub-blocks of a layer)
 * and "架构总览" (absorbed MLA, kv_lora_rank 512, rope 64); and the page "LongCat Sparse
 * Attention技术深度解析", section "模型架构配置" (index_n_heads 32, index_head_dim 128,
 * index_topk 2048, index_init_tokens 16, index_local_tokens 1024).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless stated otherwise; all are owned by the caller.  The
 *   library allocates nothing on these paths and keeps no pointer after returning.  Buffers
 *   must stay alive until the enqueued work has finished.
 * - `stream` is a hipStream_t (NULL = the legacy default stream).  Every call only enqueues
 *   work on it and returns without synchronising; order between calls is stream order, so
 *   the caller appends the current token's index key and latent row before calling.
 * - Sequences: B sequences, the cache of sequence b holds seqlens[b] tokens (device int32),
 *   the last Lq of which are the current queries.  Query i of sequence b sits at position
 *   p = seqlens[b] - Lq + i and may see keys [0, p] (n = p + 1 keys).
 *   Caller preconditions (device-side, not checked): Lq <= seqlens[b] <= S_max.  With the
 *   environment variable LSA_DEBUG_BOUNDS set (to anything but "0"), every entry point copies
 *   seqlens (and index_seqlens) to the host, waits for them and returns LSA_ERR_BAD_SHAPE when a
 *   precondition fails, before launching anything: a debugging mode that synchronises the stream.
 * - bf16 tensors are passed as raw 16-bit storage (`const void*`).  All layouts are dense,
 *   row-major, with the last dimension contiguous.
 * - Errors: host-checkable problems return a non-zero status BEFORE anything is enqueued, and
 *   lsa_last_error() then describes them (thread-local).  A zero-sized batch (B == 0 or
 *   Lq == 0) is a valid no-op.  A kernel-launch failure returns LSA_ERR_LAUNCH.  Faults in
 *   device memory surface at the caller's next synchronisation, as usual for HIP.
 * - Workspaces are device buffers of at least the size the matching *_workspace_bytes query
 *   returns, at any address (the sizes include the slack the library needs to align its
 *   regions inside); their contents on entry do not matter, and two calls in flight must not
 *   share one.
 * - Results are deterministic: identical inputs give bit-identical outputs.
 * - No global mutable state except the thread-local error text and the static workspace of
 *   lsa_index_topk_noalloc (one per device).
 */
#ifndef LSA_H_
#define LSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int lsa_status;
#define LSA_OK 0
#define LSA_ERR_NULL_ARG 1    /* a required pointer is NULL */
#define LSA_ERR_BAD_SHAPE 2   /* a size is negative/zero where it must be positive, or inconsistent */
#define LSA_ERR_UNSUPPORTED 3 /* a size outside the compiled set (see each entry point) */
#define LSA_ERR_WORKSPACE 4   /* workspace missing or smaller than the query function says */
#define LSA_ERR_LAUNCH 5      /* the HIP runtime rejected a kernel launch */

/* Short constant name of a status ("LSA_OK", ...); never NULL. */
const char* lsa_status_str(lsa_status s);

/* Detail of the last failure on the calling thread ("" if none).  Valid until the next call
 * on this thread. */
const char* lsa_last_error(void);

/* The device-side precondition on sequence lengths, checked on a HOST copy: returns the first
 * b with seqlens_host[b] < Lq or seqlens_host[b] > S_max, or -1 when every length is valid.
 * (The LSA_DEBUG_BOUNDS mode applies it to each call's seqlens.) */
int lsa_check_seqlens(const int32_t* seqlens_host, int B, int Lq, int S_max);

/*
 * Lightning-indexer scores ("LSA" section; the fused epilogue of "预填充优化" accumulates
 * max(g, 0) * w over the index heads):
 *
 *   scores[b,i,s] = sum_{h<Hi} w[b,i,h] * max(0, sum_{d<Di} q_idx[b,i,h,d] * k_idx[b,s,d])
 *
 * for every s in [0, p].  One index key per cached token, shared by all index heads.
 *   q_idx   bf16 [B, Lq, Hi, Di]   index queries (already projected, rotated)
 *   w       fp32 [B, Lq, Hi]       per-head weights (any sign)
 *   k_idx   bf16 [B, S_max, Di]    index-key cache (already normalised, rotated)
 *   seqlens int32 [B]
 *   scores  fp32 [B, Lq, S_max]    output; entries s > p are left untouched
 * Products are exact in fp32 and accumulated in fp32 (bf16 matrix cores), the head sum in
 * fp32.  Supported: 1 <= Hi <= 32, Di in {32, 64, 128}; S_max >= 1.
 */
lsa_status lsa_index_scores(const void* q_idx, const float* w, const void* k_idx,
                            const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                            float* scores, void* stream);

/* Workspace (bytes) lsa_topk_select needs for these sizes (0 is possible). */
size_t lsa_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens,
                                int local_tokens);

/*
 * Top-k selection ("LSA" section: argpartition of the top index_topk scores; the
 * index_init_tokens sink columns and index_local_tokens sliding-window columns forced so they
 * are always selected; dense fallback when the cached length does not exceed index_topk).
 * For each query row with n = p + 1 valid keys:
 *   - n <= topk: indices = 0, 1, ..., n-1 (dense fallback), n_sel = n;
 *   - otherwise positions s < init_tokens and s > p - local_tokens are forced in, and the
 *     remaining topk - init_tokens - local_tokens slots go to the largest fp32 scores among
 *     positions [init_tokens, p - local_tokens]; equal scores go to the LOWEST position
 *     (-0.0 and +0.0 are equal); n_sel = topk.
 * Indices are written in ascending order; unused slots are -1.
 *   scores    fp32 [B, Lq, S_max] (only s <= p is read; values must be finite)
 *   indices   int32 [B, Lq, topk]  output
 *   n_sel     int32 [B, Lq]        output
 *   workspace device buffer of at least lsa_topk_workspace_bytes(...) bytes (may be NULL when
 *             that is 0); its contents on entry do not matter.
 * Supported: topk >= 1, init_tokens >= 0, local_tokens >= 0, init_tokens + local_tokens <= topk
 * (else LSA_ERR_BAD_SHAPE); S_max <= 1048576 (else LSA_ERR_UNSUPPORTED).
 */
lsa_status lsa_topk_select(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max,
                           int topk, int init_tokens, int local_tokens, int32_t* indices,
                           int32_t* n_sel, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace (bytes) lsa_index_topk needs for these sizes. */
size_t lsa_index_topk_workspace_bytes(int B, int Lq, int S_max, int topk, int init_tokens,
                                      int local_tokens);

/*
 * Indexer scores and top-k selection in one pass: the same indices and n_sel as
 * lsa_index_scores followed by lsa_topk_select (bit for bit), without materialising the
 * [B, Lq, S_max] score array.  Each workgroup keeps its chunk's fp32 scores on chip and emits
 * only a superset of that chunk's contribution to the row's top scores; a merge pass makes the
 * exact selection ("LSA" section: indexer, forced columns, argpartition, dense fallback; the
 * fused epilogue of "预填充优化").
 *   q_idx, w, k_idx, seqlens  as in lsa_index_scores
 *   topk, init_tokens, local_tokens, indices, n_sel  as in lsa_topk_select
 *   workspace  device buffer of at least lsa_index_topk_workspace_bytes(...) bytes
 * Supported: the union of both calls' limits (Hi <= 32, Di in {32, 64, 128}, S_max <= 1048576,
 * init_tokens + local_tokens <= topk).
 */
lsa_status lsa_index_topk(const void* q_idx, const float* w, const void* k_idx,
                          const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max, int topk,
                          int init_tokens, int local_tokens, int32_t* indices, int32_t* n_sel,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Size of the static device workspace of lsa_index_topk_noalloc (16 MiB per device). */
#define LSA_INDEX_TOPK_SCRATCH_BYTES (16u << 20)

/*
 * lsa_index_topk without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and results as lsa_index_topk (bit for bit), with its workspace in a static
 * array of LSA_INDEX_TOPK_SCRATCH_BYTES that the library holds on each device it runs on until
 * the process ends (its device address is looked up on the first call for a device).  The call
 * allocates nothing.  Every call on a device shares that device's array: calls that may overlap
 * on one device (different streams, or several host threads) race on it and must be ordered by
 * the caller.  Arguments and errors as lsa_index_topk, without workspace/workspace_bytes; sizes
 * whose lsa_index_topk_workspace_bytes exceeds LSA_INDEX_TOPK_SCRATCH_BYTES return
 * LSA_ERR_WORKSPACE before anything is enqueued.
 */
lsa_status lsa_index_topk_noalloc(const void* q_idx, const float* w, const void* k_idx,
                                  const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                                  int topk, int init_tokens, int local_tokens, int32_t* indices,
                                  int32_t* n_sel, void* stream);

/* Largest selection the attention takes: 64 partial splits of at most 2048 rows each. */
#define LSA_MLA_MAX_TOPK 131072

/* Workspace (bytes) lsa_sparse_mla_decode / _prefill need for these sizes (0 is possible).
 * `dense` is 1 when the call will pass indices == NULL. */
size_t lsa_mla_workspace_bytes(int B, int Lq, int H, int Dv, int S_max, int topk, int dense);

/*
 * Absorbed-MLA attention over selected latent rows ("LSA" section: decode gathers KV rows by
 * the top-k indices; "架构总览": latent rank 512 plus rope 64, absorbed projections).
 * For each query row (b, i) at position p and each head h:
 *   sel   = indices[b,i,0:n_sel[b,i]]   or, when indices == NULL, every position 0..p
 *   l_s   = softmax_scale * sum_{d<Dqk} q[b,i,h,d] * kv[b,s,d]        for s in sel
 *   out[b,i,h,c] = sum_s softmax(l)_s * kv[b,s,c]                       for c < Dv
 *   lse[b,i,h]   = log(sum_s exp(l_s))                                  (natural log)
 * A latent row is [latent (Dv) | rope (Dqk - Dv)]; the value vector is its first Dv entries.
 * Products are bf16 x bf16 on matrix cores with fp32 accumulation; the softmax is fp32; the
 * probabilities enter the value product as bf16; out is rounded to bf16.
 *   q       bf16 [B, H, Dqk] (decode) / [B, Lq, H, Dqk] (prefill)
 *   kv      bf16 [B, S_max, Dqk]   latent cache
 *   indices int32 [B, Lq, topk] from lsa_topk_select (ascending or not; entries >= n_sel are
 *           ignored), or NULL for dense attention over [0, p]
 *   n_sel   int32 [B, Lq] (ignored when indices == NULL)
 *   out     bf16 [B, H, Dv] / [B, Lq, H, Dv]
 *   lse     fp32 [B, H] / [B, Lq, H], or NULL
 * The same indices may serve several calls (the two attention sub-blocks of a layer share
 * one index pass); the inputs are never written.
 * Rows that select nothing get out = 0 and lse = -inf.
 * Supported: (Dqk, Dv) in {(576, 512), (80, 64)}; H >= 1 (heads are processed in groups of
 * 32); 1 <= topk <= LSA_MLA_MAX_TOPK when indices != NULL.
 */
lsa_status lsa_sparse_mla_decode(const void* q, const void* kv, const int32_t* indices,
                                 const int32_t* n_sel, const int32_t* seqlens, int B, int H,
                                 int Dqk, int Dv, int S_max, int topk, float softmax_scale,
                                 void* out, float* lse, void* workspace, size_t workspace_bytes,
                                 void* stream);

lsa_status lsa_sparse_mla_prefill(const void* q, const void* kv, const int32_t* indices,
                                  const int32_t* n_sel, const int32_t* seqlens, int B, int Lq,
                                  int H, int Dqk, int Dv, int S_max, int topk,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Most positions appended after an index pass that lsa_mtp_draft_attention takes. */
#define LSA_MTP_MAX_APPENDED 64
/* Largest selection lsa_mtp_draft_attention takes (its last split also holds the appended
 * positions). */
#define LSA_MTP_MAX_TOPK 65536

/* Workspace (bytes) lsa_mtp_draft_attention needs for these sizes (0 is possible). */
size_t lsa_mtp_draft_workspace_bytes(int B, int H, int Dv, int S_max, int topk, int max_appended);

/*
 * Attention of a multi-token-prediction draft step on a shared index pass (page "LongCat Sparse
 * Attention技术深度解析…", section "技术实现细节", multi-token prediction: the three draft steps
 * of speculative decoding share a single index pass; config key dsa_mtp_cli).  The index pass
 * ran when sequence b had index_seqlens[b] tokens; the draft steps have appended the tokens
 * since.  For the query at p = seqlens[b] - 1:
 *   sel = indices[b, 0:n_sel[b]]  followed by  index_seqlens[b], ..., p
 * (the appended positions, at most max_appended of them; later ones are not attended), then the
 * attention of lsa_sparse_mla_decode over sel.  The appended tokens are the most recent ones,
 * which the forced local window keeps at every position, so each draft step attends to them
 * without a new index pass.
 *   indices        int32 [B, topk] of the index pass (lsa_index_topk or lsa_topk_select, Lq = 1)
 *   n_sel          int32 [B]
 *   index_seqlens  int32 [B] sequence lengths at the index pass
 *   seqlens        int32 [B] current lengths
 *   q, kv, out, lse, softmax_scale, workspace, stream: as for lsa_sparse_mla_decode.
 * The inputs are never written; one index pass serves any number of calls.
 * Errors: those of lsa_sparse_mla_decode; NULL indices, n_sel or index_seqlens ->
 * LSA_ERR_NULL_ARG; max_appended outside [0, LSA_MTP_MAX_APPENDED] -> LSA_ERR_BAD_SHAPE;
 * topk > LSA_MTP_MAX_TOPK -> LSA_ERR_UNSUPPORTED.
 */
lsa_status lsa_mtp_draft_attention(const void* q, const void* kv, const int32_t* indices,
                                   const int32_t* n_sel, const int32_t* index_seqlens,
                                   const int32_t* seqlens, int B, int H, int Dqk, int Dv,
                                   int S_max, int topk, int max_appended, float softmax_scale,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Block keys for hierarchical indexing (page "LongCat Sparse Attention技术深度解析", section on
 * LSA's three strategies, "分层索引": block-level approximate scores come first, then the token
 * selection inside the chosen blocks).  The page gives no block size or block key; here block j
 * of sequence b is tokens [j*Bk, (j+1)*Bk) and its key is the mean of their index keys, rounded
 * once to bf16 (round to nearest even; the sum is taken in fp32, exact for keys on a coarse
 * dyadic grid).  Writes block_keys[b, j, :] for first_block <= j < seqlens[b] / Bk (complete
 * blocks only), so a cache that grows can be summarised block by block.
 *   k_idx       bf16 [B, S_max, Di] index-key cache
 *   block_keys  bf16 [B, S_max / Bk, Di] (caller-owned; other rows are not touched)
 * Supported: Bk a power of two in [8, 1024], Bk <= S_max; Di a multiple of 16, <= 128.
 * Errors: NULL pointers (B > 0) -> LSA_ERR_NULL_ARG; bad sizes -> LSA_ERR_BAD_SHAPE /
 * LSA_ERR_UNSUPPORTED.
 */
lsa_status lsa_block_keys(const void* k_idx, const int32_t* seqlens, int B, int S_max, int Di,
                          int Bk, int first_block, void* block_keys, void* stream);

/* Workspace (bytes) lsa_hier_index_topk needs for these sizes (0 for invalid sizes). */
size_t lsa_hier_workspace_bytes(int B, int S_max, int Bk, int topk, int init_tokens,
                                int local_tokens, int M);

/*
 * Hierarchical indexer + top-k for decode rows ("分层索引", same page): for the query at
 * p = seqlens[b] - 1 (n = p + 1 visible keys):
 *  - n <= topk: every position (the dense fallback of lsa_topk_select);
 *  - else the nb = w0 / Bk complete blocks before the sliding window (w0 = max(p - local + 1, 0))
 *    are scored like keys, I_j = sum_h w[b,h] * max(0, q_idx[b,h,:] . block_keys[b,j,:]), and
 *    the M best kept (larger score, then lower block; all when nb <= M);
 *  - tokens outside the sink [0, init), the positions from nb*Bk on (the partial block and the
 *    window) and the kept blocks get the score -inf; the others their indexer score; then the
 *    selection of lsa_topk_select (sink and window forced, ties to the lower position).
 * This is an approximation of lsa_index_topk (exact when M >= nb); with M*Bk well above
 * topk - init - local it reads about (nb + M*Bk) keys instead of n.
 *   q_idx bf16 [B, Hi, Di]; w fp32 [B, Hi]; k_idx bf16 [B, S_max, Di]; block_keys from
 *   lsa_block_keys (complete for every block below seqlens[b] / Bk); indices int32 [B, topk]
 *   ascending, -1 padded; n_sel int32 [B].
 * Supported: Hi <= 32, Di a multiple of 16 and <= 128, Bk a power of two in [8, 1024],
 * 1 <= M <= S_max / Bk with M*Bk >= topk - local_tokens (so the kept blocks always hold enough
 * candidates and no -inf token is ever selected), and the sizes lsa_topk_select takes.  Errors
 * as lsa_index_topk.
 */
lsa_status lsa_hier_index_topk(const void* q_idx, const float* w, const void* k_idx,
                               const void* block_keys, const int32_t* seqlens, int B, int Hi,
                               int Di, int S_max, int topk, int init_tokens, int local_tokens,
                               int Bk, int M, int32_t* indices, int32_t* n_sel, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Workspace (bytes) lsa_index_frontend needs for these sizes (0 for invalid sizes). */
size_t lsa_index_frontend_workspace_bytes(int B, int Lq, int q_lora, int hidden, int Hi, int Di);

/*
 * Indexer front end: the indexer inputs of the current tokens ("LSA" section: wq_b projects the
 * q-LoRA representation to index_n_heads x index_head_dim, wk projects the hidden state to the
 * index key, which is RMS-normalised, weights_proj gives one weight per index head; index queries
 * and keys take the attention's rotary settings, qk_rope_head_dim and rope_theta, "架构总览").
 * For token i of sequence b at position p = seqlens[b] - Lq + i:
 *   q_idx[b,i,h,:] = rot_p(cq[b,i,:] . wq_b[h*Di:(h+1)*Di, :]^T)
 *   w[b,i,h]       = hid[b,i,:] . w_proj[h, :]^T
 *   k_cache[b,p,:] = rot_p(gain * x / sqrt(mean(x^2) + norm_eps)),  x = hid[b,i,:] . wk^T
 * where rot_p turns pair (2m, 2m+1) of the last rope_dim entries by the angle
 * p * rope_theta^(-2m/rope_dim): (u, v) -> (u cos - v sin, u sin + v cos).  Which entries rotate
 * and how they pair is not given by the pages (the last rope_dim, adjacent pairs, is this
 * library's reading).  Products are bf16 x bf16 with fp32 accumulation; the norm and the rotation
 * run in fp32 (angles in fp64); q_idx and the key are rounded once to bf16, w stays fp32.
 *   cq      bf16 [B, Lq, q_lora]          q-LoRA representation
 *   hid     bf16 [B, Lq, hidden]          hidden state
 *   wq_b    bf16 [Hi*Di, q_lora]          (rows = outputs, as a linear layer's weight)
 *   wk      bf16 [Di, hidden]
 *   k_norm_gain fp32 [Di]
 *   w_proj  bf16 [Hi, hidden]
 *   q_idx   bf16 [B, Lq, Hi, Di]  output;  w fp32 [B, Lq, Hi]  output
 *   k_cache bf16 [B, S_max, Di]   row p of each current token is written, nothing else
 *   workspace device buffer of at least lsa_index_frontend_workspace_bytes(...) bytes
 * Supported: q_lora and hidden multiples of 16, Di even <= 128, Hi <= 32, rope_dim even <= Di,
 * rope_theta > 0, norm_eps >= 0 (else LSA_ERR_BAD_SHAPE / LSA_ERR_UNSUPPORTED).  Caller
 * precondition (device-side): 0 <= p < S_max; a token outside writes no cache row.
 */
lsa_status lsa_index_frontend(const void* cq, const void* hid, const void* wq_b, const void* wk,
                              const float* k_norm_gain, const void* w_proj, const int32_t* seqlens,
                              int B, int Lq, int q_lora, int hidden, int Hi, int Di, int rope_dim,
                              float rope_theta, float norm_eps, int S_max, void* q_idx, float* w,
                              void* k_cache, void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H_ */
