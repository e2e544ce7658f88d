/*
 * CPU oracle for the LongCat Sparse Attention (LSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg
 * may load this library.  It shares no code, header or constant with the GPU library and
 * includes no HIP header.  It is deliberately plain: fp64 arithmetic, naive loops, a library
 * sort; OpenMP only runs independent outputs (query rows, and (row, key) pairs for the
 * scores) side by side, never changing what is summed or in which order.
 *
 * Sources (the web pages this project follows):
 *  - "MLX-VLM 的 LongCat-Flash-Lite-Sparse 支持LSA 稀疏注意力、n-gram 融合与预填充优化解析"
 *    (lmnt.cn), section "LSA": the indexer score (ReLU of q.k, weighted sum over index heads),
 *    top-index_topk selection with argpartition, sink (index_init_tokens) and sliding-window
 *    (index_local_tokens) columns forced so they are always chosen, the dense fallback when the
 *    cached length does not exceed index_topk, decode gathering KV rows by index and prefill
 *    using a sparse boolean mask; section "预填充优化": the fused epilogue accumulating
 *    max(g, 0) * w over heads, and the plain fallback max(q k^T, 0) weighted sum.
 *  - "LongCat Sparse Attention技术深度解析" (wmrh.cn), "模型架构配置": index_n_heads 32,
 *    index_head_dim 128, index_topk 2048, index_init_tokens 16, index_local_tokens 1024.
 *
 * Readings where the pages are silent or garbled (each is listed in the design notes):
 *  - the forced value is +infinity (sign lost in extraction; "always selected");
 *  - the dense fallback applies when n = p + 1 <= topk (comparison operator lost);
 *  - sink = positions [0, init), window = the `local` most recent positions [p-local+1, p];
 *  - ties are broken toward the lowest position, output is ascending, padded with -1;
 *  - one index key per cached token, shared by all index heads;
 *  - scores are rounded once to fp32, and the selection ranks the fp32 values;
 *  - a latent row is [latent (Dv values) | rope]; the value vector is its first Dv entries.
 *
 * Hierarchical indexing (lsa_oracle_hier_topk, at the end of this file) follows the LSA page's
 * "分层索引"; its block size and block score are readings listed with the function, and its
 * parity against the pages is unpinned.
 *
 * The indexer front end (lsa_oracle_index_frontend, at the end of this file) follows page 1's
 * "LSA" description of wq_b, wk with RMS normalisation and weights_proj, with the attention's
 * rotary settings; its readings are listed with the function.
 *
 * Parity pins (tests/test_oracle.py, tests/test_oracle_frontend.py): exact integer brute force of
 * the scores and of the front-end projections, closed-form norms and rotations, NumPy lexsort
 * brute force of the selection, a hand-worked selection fixture (tests/golden), dense masked
 * softmax in NumPy float64, closed-form special cases and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 bit pattern -> exact double */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Position of query i of a sequence holding `seqlen` tokens of which the last Lq are queries. */
static long query_position(int32_t seqlen, int Lq, int i) { return (long)seqlen - Lq + i; }

void lsa_oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int lsa_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Indexer scores (page 1, "LSA" and "预填充优化"):
 *   I[s] = sum_h w[h] * max(0, sum_d q[h][d] * k[s][d])   for s in [0, p]
 * q_idx: bf16 [B, Lq, Hi, Di]; w: fp32 [B, Lq, Hi]; k_idx: bf16 [B, S_max, Di];
 * scores: fp32 [B, Lq, S_max], written for s <= p only.  fp64 sums, one rounding to fp32.
 * Returns 0, or -1 if some query position falls outside [0, S_max).
 */
int lsa_oracle_index_scores(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                            const int32_t* seqlens, int B, int Lq, int Hi, int Di, int S_max,
                            float* scores) {
  long rows = (long)B * Lq;
  for (long r = 0; r < rows; ++r) {
    long p = query_position(seqlens[r / Lq], Lq, (int)(r % Lq));
    if (p < 0 || p >= S_max) return -1;
  }
  /* one (row, key) pair per iteration; positions after the query are skipped */
#pragma omp parallel for collapse(2) schedule(static)
  for (long r = 0; r < rows; ++r) {
    for (long s = 0; s < S_max; ++s) {
      int b = (int)(r / Lq), i = (int)(r % Lq);
      long p = query_position(seqlens[b], Lq, i);
      if (s > p) continue;
      const uint16_t* qr = q_idx + r * (long)Hi * Di;
      const float* wr = w + r * (long)Hi;
      const uint16_t* ks = k_idx + ((long)b * S_max + s) * Di;
      double total = 0.0;
      for (int h = 0; h < Hi; ++h) {
        double g = 0.0;
        for (int d = 0; d < Di; ++d) g += bf16_value(qr[(long)h * Di + d]) * bf16_value(ks[d]);
        double relu = g > 0.0 ? g : 0.0;
        total += (double)wr[h] * relu;
      }
      scores[r * (long)S_max + s] = (float)total;
    }
  }
  return 0;
}

typedef struct {
  double key; /* fp32 score widened, or +inf for forced columns */
  int32_t pos;
} ranked_t;

/* larger key first; equal keys: lower position first */
static int cmp_rank(const void* a, const void* b) {
  const ranked_t* x = (const ranked_t*)a;
  const ranked_t* y = (const ranked_t*)b;
  if (x->key > y->key) return -1;
  if (x->key < y->key) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int cmp_int(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/*
 * Top-k selection (page 1, "LSA"): for each row with n = p + 1 valid keys
 *  - n <= topk: every position 0..n-1 (dense fallback), n_sel = n;
 *  - else: keys of positions s < init and s > p - local are +inf, the rest keep their fp32
 *    score; order by key descending then position ascending; keep the first topk;
 *    n_sel = topk.
 * indices: int32 [B, Lq, topk], ascending, padded with -1.  n_sel: int32 [B, Lq].
 * Returns 0, -1 on a bad position, -2 if init + local > topk.
 */
int lsa_oracle_topk(const float* scores, const int32_t* seqlens, int B, int Lq, int S_max, int topk,
                    int init_tokens, int local_tokens, int32_t* indices, int32_t* n_sel) {
  if (init_tokens < 0 || local_tokens < 0 || init_tokens + local_tokens > topk) return -2;
  int bad = 0;
  long rows = (long)B * Lq;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long r = 0; r < rows; ++r) {
    int b = (int)(r / Lq), i = (int)(r % Lq);
    long p = query_position(seqlens[b], Lq, i);
    int32_t* out = indices + r * (long)topk;
    if (p < 0 || p >= S_max) {
      bad |= 1;
      continue;
    }
    long n = p + 1;
    for (int j = 0; j < topk; ++j) out[j] = -1;
    if (n <= topk) {
      for (long s = 0; s < n; ++s) out[s] = (int32_t)s;
      n_sel[r] = (int32_t)n;
      continue;
    }
    ranked_t* all = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)n);
    const float* sr = scores + r * (long)S_max;
    for (long s = 0; s < n; ++s) {
      int forced = (s < init_tokens) || (s > p - local_tokens);
      all[s].key = forced ? INFINITY : (double)sr[s];
      all[s].pos = (int32_t)s;
    }
    qsort(all, (size_t)n, sizeof(ranked_t), cmp_rank);
    for (int j = 0; j < topk; ++j) out[j] = all[j].pos;
    qsort(out, (size_t)topk, sizeof(int32_t), cmp_int);
    n_sel[r] = topk;
    free(all);
  }
  return bad ? -1 : 0;
}

/*
 * Absorbed-MLA attention over a set of latent rows (page 1, "LSA": decode gathers rows by
 * the top-k indices, prefill masks; "架构总览": latent rank 512 plus rope 64).
 * For each row (b, i) with position p and each head h:
 *   sel  = indices[b,i,0:n_sel[b,i]]  (or every position 0..p when indices == NULL)
 *   l_s  = scale * sum_{d < Dqk} q[b,i,h,d] * kv[b,s,d]         (s in sel)
 *   out  = sum_s exp(l_s - m) kv[b,s,0:Dv] / sum_s exp(l_s - m),  m = max_s l_s
 *   lse  = m + log(sum_s exp(l_s - m))
 * q: bf16 [B, Lq, H, Dqk]; kv: bf16 [B, S_max, Dqk]; out: fp64 [B, Lq, H, Dv];
 * lse: fp64 [B, Lq, H] (may be NULL).  A row with nothing selected gets out = 0, lse = -inf.
 * Returns 0, -1 on a bad position, -3 on a selected index outside [0, p].
 */
int lsa_oracle_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                          const int32_t* n_sel, const int32_t* seqlens, int B, int Lq, int H,
                          int Dqk, int Dv, int S_max, int topk, double scale, double* out,
                          double* lse) {
  int bad = 0;
  long rows = (long)B * Lq;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long r = 0; r < rows; ++r) {
    int b = (int)(r / Lq), i = (int)(r % Lq);
    long p = query_position(seqlens[b], Lq, i);
    if (p < 0 || p >= S_max) {
      bad |= 1;
      continue;
    }
    long cnt;
    int32_t* sel;
    if (indices) {
      cnt = n_sel[r];
      sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(cnt > 0 ? cnt : 1));
      for (long j = 0; j < cnt; ++j) {
        int32_t s = indices[r * (long)topk + j];
        if (s < 0 || s > p) bad |= 2;
        sel[j] = s;
      }
      if (bad & 2) {
        free(sel);
        continue;
      }
    } else {
      cnt = p + 1;
      sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)cnt);
      for (long j = 0; j < cnt; ++j) sel[j] = (int32_t)j;
    }
    double* logit = (double*)malloc(sizeof(double) * (size_t)(cnt > 0 ? cnt : 1));
    for (int h = 0; h < H; ++h) {
      const uint16_t* qh = q + (r * H + h) * (long)Dqk;
      double* oh = out + (r * H + h) * (long)Dv;
      for (int c = 0; c < Dv; ++c) oh[c] = 0.0;
      if (cnt == 0) {
        if (lse) lse[r * H + h] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (long j = 0; j < cnt; ++j) {
        const uint16_t* row = kv + ((long)b * S_max + sel[j]) * Dqk;
        double dot = 0.0;
        for (int d = 0; d < Dqk; ++d) dot += bf16_value(qh[d]) * bf16_value(row[d]);
        logit[j] = scale * dot;
        if (logit[j] > m) m = logit[j];
      }
      double z = 0.0;
      for (long j = 0; j < cnt; ++j) {
        double e = exp(logit[j] - m);
        z += e;
        const uint16_t* row = kv + ((long)b * S_max + sel[j]) * Dqk;
        for (int c = 0; c < Dv; ++c) oh[c] += e * bf16_value(row[c]);
      }
      for (int c = 0; c < Dv; ++c) oh[c] /= z;
      if (lse) lse[r * H + h] = m + log(z);
    }
    free(logit);
    free(sel);
  }
  if (bad & 1) return -1;
  if (bad & 2) return -3;
  return 0;
}

/*
 * Indexer front end (page 1, "LSA": the index query is the q-LoRA representation projected by
 * wq_b to index_n_heads x index_head_dim; the index key is the hidden state projected by wk and
 * RMS-normalised; weights_proj gives one weight per index head; index queries and keys use the
 * attention's rotary settings, qk_rope_head_dim and rope_theta from "架构总览").  Per token
 * (b, i) at position p = seqlens[b] - Lq + i, in fp64:
 *   q[h][d] = sum_j cq[j] * wq_b[h*Di + d][j]
 *   k[d]    = g[d] * x[d] / sqrt(mean_e x[e]^2 + eps),  x[d] = sum_j hid[j] * wk[d][j]
 *   w[h]    = sum_j hid[j] * w_proj[h][j]
 * then the rotary embedding on the last R dims of every q head and of k: pair (2m, 2m+1) of
 * that part turns by the angle p * theta^(-2m/R):
 *   (u, v) -> (u cos a - v sin a, u sin a + v cos a).
 * Readings: the rotated part is the last R dims (the latent rows put rope last), pairs are
 * adjacent, RMSNorm carries a per-dim gain and eps, no extra scale on w.  Which dims rotate and
 * how they pair is parity unpinned against the pages (they do not say); the pins fix this
 * function to the readings.
 * cq: bf16 [B, Lq, q_lora]; hid: bf16 [B, Lq, hidden]; wq_b: bf16 [Hi*Di, q_lora];
 * wk: bf16 [Di, hidden]; gain: fp32 [Di]; w_proj: bf16 [Hi, hidden]; outputs fp64:
 * q_out [B, Lq, Hi, Di], w_out [B, Lq, Hi], k_out [B, Lq, Di].
 * Returns 0, -1 on a negative position, -2 on a bad rotary size.
 */
static void rotate_tail(double* v, int Di, int R, long p, double theta) {
  for (int m = 0; m < R / 2; ++m) {
    double a = (double)p * pow(theta, -2.0 * m / R);
    double c = cos(a), s = sin(a);
    double* u = v + (Di - R) + 2 * m;
    double x = u[0], y = u[1];
    u[0] = x * c - y * s;
    u[1] = x * s + y * c;
  }
}

int lsa_oracle_index_frontend(const uint16_t* cq, const uint16_t* hid, const uint16_t* wq_b,
                              const uint16_t* wk, const float* gain, const uint16_t* w_proj,
                              const int32_t* seqlens, int B, int Lq, int q_lora, int hidden,
                              int Hi, int Di, int R, double theta, double eps, double* q_out,
                              double* w_out, double* k_out) {
  if (R < 0 || R > Di || (R & 1)) return -2;
  int bad = 0;
  long rows = (long)B * Lq;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long r = 0; r < rows; ++r) {
    int b = (int)(r / Lq), i = (int)(r % Lq);
    long p = query_position(seqlens[b], Lq, i);
    if (p < 0) {
      bad |= 1;
      continue;
    }
    const uint16_t* c = cq + r * (long)q_lora;
    const uint16_t* x = hid + r * (long)hidden;
    for (int h = 0; h < Hi; ++h) {
      double* qh = q_out + (r * Hi + h) * (long)Di;
      for (int d = 0; d < Di; ++d) {
        const uint16_t* wrow = wq_b + ((long)h * Di + d) * q_lora;
        double s = 0.0;
        for (int j = 0; j < q_lora; ++j) s += bf16_value(c[j]) * bf16_value(wrow[j]);
        qh[d] = s;
      }
      rotate_tail(qh, Di, R, p, theta);
    }
    double* kr = k_out + r * (long)Di;
    double ms = 0.0;
    for (int d = 0; d < Di; ++d) {
      const uint16_t* wrow = wk + (long)d * hidden;
      double s = 0.0;
      for (int j = 0; j < hidden; ++j) s += bf16_value(x[j]) * bf16_value(wrow[j]);
      kr[d] = s;
      ms += s * s;
    }
    double inv = 1.0 / sqrt(ms / Di + eps);
    for (int d = 0; d < Di; ++d) kr[d] = (double)gain[d] * (kr[d] * inv);
    rotate_tail(kr, Di, R, p, theta);
    for (int h = 0; h < Hi; ++h) {
      const uint16_t* wrow = w_proj + (long)h * hidden;
      double s = 0.0;
      for (int j = 0; j < hidden; ++j) s += bf16_value(x[j]) * bf16_value(wrow[j]);
      w_out[r * Hi + h] = s;
    }
  }
  return (bad & 1) ? -1 : 0;
}

/*
 * Hierarchical indexing (page "LongCat Sparse Attention技术深度解析", section on LSA's three
 * strategies, "分层索引": a coarse block-level score first, then the token selection inside the
 * chosen blocks, which shrinks the candidates the indexer scores).  The page gives no block size
 * and no block score; the readings taken here:
 *  - block j of sequence b is tokens [j*Bk, (j+1)*Bk); its key is the mean of their index keys,
 *    rounded once to bf16 (round to nearest even);
 *  - a block is scored like a token, I_j = sum_h w[h] * max(0, q[h] . key_j) (fp64, rounded
 *    once to fp32);
 *  - the blocks scored are the nb = w0 / Bk complete blocks before the sliding window, which
 *    starts at w0 = max(p - local + 1, 0); the M best are kept (larger score first, then the
 *    lower block), all of them when nb <= M;
 *  - candidates: the sink (s < init), every position from nb*Bk on (the partial block before the
 *    window and the window), and the tokens of the kept blocks; the other tokens get the score
 *    -inf; then the selection of lsa_oracle_topk (dense fallback when n <= topk, sink and window
 *    forced, larger key first, then the lower position).
 * Decode rows only (one query per sequence, at p = seqlens[b] - 1).
 * q_idx: bf16 [B, Hi, Di]; w: fp32 [B, Hi]; k_idx: bf16 [B, S_max, Di]; indices: int32
 * [B, topk] ascending, padded with -1; n_sel: int32 [B].
 * Returns 0, -1 on a bad position, -2 on bad sizes.
 */
static uint16_t bf16_round(double x) {
  /* round x to 8 significant bits, nearest even (the default rounding mode), then take the
     top half of the fp32 pattern (exact: the value has at most 8 significant bits) */
  if (x == 0.0) return 0;
  int e;
  double m = frexp(x, &e); /* x = m * 2^e, 0.5 <= |m| < 1 */
  float f = (float)ldexp(nearbyint(ldexp(m, 8)), e - 8);
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static double weighted_relu_score(const uint16_t* q, const float* w, const uint16_t* k, int Hi, int Di) {
  double total = 0.0;
  for (int h = 0; h < Hi; ++h) {
    double g = 0.0;
    for (int d = 0; d < Di; ++d) g += bf16_value(q[(long)h * Di + d]) * bf16_value(k[d]);
    total += (double)w[h] * (g > 0.0 ? g : 0.0);
  }
  return (double)(float)total;
}

int lsa_oracle_hier_topk(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                         const int32_t* seqlens, int B, int Hi, int Di, int S_max, int topk,
                         int init_tokens, int local_tokens, int Bk, int M, int32_t* indices,
                         int32_t* n_sel) {
  if (Bk <= 0 || M < 0 || init_tokens < 0 || local_tokens < 0 || init_tokens + local_tokens > topk)
    return -2;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int b = 0; b < B; ++b) {
    long p = (long)seqlens[b] - 1, n = p + 1;
    int32_t* out = indices + (long)b * topk;
    if (p < 0 || p >= S_max) {
      bad |= 1;
      continue;
    }
    for (int j = 0; j < topk; ++j) out[j] = -1;
    if (n <= topk) {
      for (long s = 0; s < n; ++s) out[s] = (int32_t)s;
      n_sel[b] = (int32_t)n;
      continue;
    }
    const uint16_t* qr = q_idx + (long)b * Hi * Di;
    const float* wr = w + (long)b * Hi;
    const uint16_t* kb = k_idx + (long)b * S_max * Di;
    long w0 = p - local_tokens + 1;
    if (w0 < 0) w0 = 0;
    long nb = w0 / Bk;
    /* stage 1: block keys and block scores, the M best blocks kept */
    ranked_t* blocks = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(nb > 0 ? nb : 1));
    uint16_t* key = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)Di);
    for (long j = 0; j < nb; ++j) {
      for (int d = 0; d < Di; ++d) {
        double s = 0.0;
        for (int t = 0; t < Bk; ++t) s += bf16_value(kb[(j * Bk + t) * (long)Di + d]);
        key[d] = bf16_round(s / Bk);
      }
      blocks[j].key = weighted_relu_score(qr, wr, key, Hi, Di);
      blocks[j].pos = (int32_t)j;
    }
    qsort(blocks, (size_t)nb, sizeof(ranked_t), cmp_rank);
    char* kept = (char*)calloc((size_t)(nb > 0 ? nb : 1), 1);
    for (long j = 0; j < nb && j < M; ++j) kept[blocks[j].pos] = 1;
    /* stage 2: token keys over the candidates, -inf elsewhere; sink and window forced */
    ranked_t* all = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)n);
    for (long s = 0; s < n; ++s) {
      int forced = (s < init_tokens) || (s > p - local_tokens);
      int cand = s < init_tokens || s >= nb * Bk || kept[s / Bk];
      all[s].key = forced ? INFINITY
                   : cand ? weighted_relu_score(qr, wr, kb + s * (long)Di, Hi, Di)
                          : -INFINITY;
      all[s].pos = (int32_t)s;
    }
    qsort(all, (size_t)n, sizeof(ranked_t), cmp_rank);
    for (int j = 0; j < topk; ++j) out[j] = all[j].pos;
    qsort(out, (size_t)topk, sizeof(int32_t), cmp_int);
    n_sel[b] = topk;
    free(all);
    free(kept);
    free(key);
    free(blocks);
  }
  return bad ? -1 : 0;
}
