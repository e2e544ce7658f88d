/* Runs the C oracle on small inputs (dense and sparse rows, ties, all-zero scores, prefill rows,
 * dense attention) and through its error returns, so that an address or undefined-behaviour
 * sanitizer build sees every path.  Exit status 0 when every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int lsa_oracle_index_scores(const uint16_t*, const float*, const uint16_t*, const int32_t*, int, int,
                            int, int, int, float*);
int lsa_oracle_topk(const float*, const int32_t*, int, int, int, int, int, int, int32_t*, int32_t*);
int lsa_oracle_sparse_mla(const uint16_t*, const uint16_t*, const int32_t*, const int32_t*,
                          const int32_t*, int, int, int, int, int, int, int, double, double*, double*);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next(void) {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)(state >> 32);
}
/* bf16 bits of a small dyadic value in {-3/4 .. 3/4}, or zero */
static uint16_t dyadic(int zero) {
  if (zero) return 0;
  const float v = ((int)(next() % 7) - 3) * 0.25f;
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}

#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main(void) {
  enum { B = 3, Lq = 4, Hi = 4, Di = 32, S = 150, TOPK = 64, I = 4, W = 16, H = 3, DQK = 80, DV = 64 };
  const int32_t seqlens[B] = {150, 60, 4}; /* sparse rows, dense rows (n <= topk), tiny */
  uint16_t* q = malloc(sizeof(uint16_t) * B * Lq * Hi * Di);
  float* w = malloc(sizeof(float) * B * Lq * Hi);
  uint16_t* k = malloc(sizeof(uint16_t) * B * S * Di);
  float* sc = malloc(sizeof(float) * B * Lq * S);
  int32_t* idx = malloc(sizeof(int32_t) * B * Lq * TOPK);
  int32_t nsel[B * Lq];
  uint16_t* qm = malloc(sizeof(uint16_t) * B * Lq * H * DQK);
  uint16_t* kv = malloc(sizeof(uint16_t) * B * S * DQK);
  double* out = malloc(sizeof(double) * B * Lq * H * DV);
  double* lse = malloc(sizeof(double) * B * Lq * H);
  for (int pass = 0; pass < 2; ++pass) { /* pass 1: zero queries -> all scores 0 (ties everywhere) */
    for (int i = 0; i < B * Lq * Hi * Di; ++i) q[i] = dyadic(pass == 1);
    for (int i = 0; i < B * Lq * Hi; ++i) w[i] = (float)((int)(next() % 7) - 3) * 0.125f;
    for (int i = 0; i < B * S * Di; ++i) k[i] = dyadic(0);
    for (int i = 0; i < B * Lq * S; ++i) sc[i] = NAN;
    CHECK(lsa_oracle_index_scores(q, w, k, seqlens, B, Lq, Hi, Di, S, sc) == 0);
    for (int i = 0; i < B * Lq * S; ++i)
      if (isnan(sc[i])) sc[i] = 0.0f; /* positions past p are never read */
    CHECK(lsa_oracle_topk(sc, seqlens, B, Lq, S, TOPK, I, W, idx, nsel) == 0);
    CHECK(lsa_oracle_topk(sc, seqlens, B, Lq, S, TOPK, 40, 30, idx, nsel) == -2); /* I + W > topk */
    CHECK(lsa_oracle_topk(sc, seqlens, B, Lq, S, TOPK, TOPK - W, W, idx, nsel) == 0); /* no free slot */
    CHECK(lsa_oracle_topk(sc, seqlens, B, Lq, S, TOPK, I, W, idx, nsel) == 0);
    for (int r = 0; r < B * Lq; ++r) {
      const int n = seqlens[r / Lq] - Lq + r % Lq + 1;
      if (n <= 0) continue;
      CHECK(nsel[r] == (n < TOPK ? n : TOPK));
    }
  }
  for (int i = 0; i < B * Lq * H * DQK; ++i) qm[i] = dyadic(0);
  for (int i = 0; i < B * S * DQK; ++i) kv[i] = dyadic(0);
  /* the tiny sequence (seqlen 4 == Lq) has rows with p = 0..3: every row sees at least itself */
  CHECK(lsa_oracle_sparse_mla(qm, kv, idx, nsel, seqlens, B, Lq, H, DQK, DV, S, TOPK, 0.1, out, lse) == 0);
  CHECK(lsa_oracle_sparse_mla(qm, kv, NULL, NULL, seqlens, B, Lq, H, DQK, DV, S, TOPK, 0.1, out, NULL) == 0);
  for (int i = 0; i < B * Lq * H * DV; ++i) CHECK(isfinite(out[i]));
  idx[0] = S + 5; /* a selected index outside [0, p] is refused */
  CHECK(lsa_oracle_sparse_mla(qm, kv, idx, nsel, seqlens, B, Lq, H, DQK, DV, S, TOPK, 0.1, out, lse) == -3);
  const int32_t bad_len[B] = {S + 1, 60, 4}; /* a query position past S_max is refused */
  CHECK(lsa_oracle_index_scores(q, w, k, bad_len, B, Lq, Hi, Di, S, sc) == -1);
  free(q); free(w); free(k); free(sc); free(idx); free(qm); free(kv); free(out); free(lse);
  puts("oracle driver: ok");
  return 0;
}
