/* oracle_driver.c -- runs every function of the CPU oracle (oracle/dsa_oracle.c) on small inputs
 * held in exactly sized heap buffers, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Any read or write past a buffer, any
 * use of freed memory and any undefined arithmetic aborts the run. The cases walk the oracle's
 * edge paths: permuted and invalid pages, rows at position 0 and at the last position, index
 * lists with holes, repeats and invisible entries, empty sets, k above and below the prefix
 * length, FP8 saturation and skipped tokens in the cache writes. Results are not checked here
 * (the pins in test_oracle.py do that); a zero exit status means no sanitizer report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsa_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64*: input bits only, no method arithmetic */
  g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float uniform(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f; }
static void* xmalloc(size_t n) { void* p = malloc(n ? n : 1); if (!p) { perror("malloc"); exit(2); } return p; }
static uint16_t bf16_of(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }

#define CHECK(call) do { int rc_ = (call); if (rc_ != 0) { fprintf(stderr, "%s -> %d\n", #call, rc_); return 1; } } while (0)

int main(void) {
  enum { PAGE = 64, NSEQ = 2, QPS = 3, ROWS = NSEQ * QPS, LDPT = 4, NPAGES = 9, HI = 4, DI = 32, K = 40,
         H = 2, DQK = 24, DV = 8, KVD = 32, V0 = 16 };
  const int ntok = NPAGES * PAGE;
  int32_t* pt = xmalloc(sizeof(int32_t) * NSEQ * LDPT);
  const int32_t pages[NSEQ * LDPT] = {7, 2, 5, 0, 1, 8, 3, 6};
  memcpy(pt, pages, sizeof pages);
  int32_t* q_pos = xmalloc(sizeof(int32_t) * ROWS);
  const int32_t qp[ROWS] = {0, 200, 17, 63, 64, 255};
  memcpy(q_pos, qp, sizeof qp);
  const int max_ctx = LDPT * PAGE;

  /* indexer, both element formats */
  uint8_t* q8 = xmalloc((size_t)ROWS * HI * DI);
  float* qf = xmalloc(sizeof(float) * ROWS * HI * DI);
  uint8_t* k8 = xmalloc((size_t)ntok * DI);
  float* kf = xmalloc(sizeof(float) * ntok * DI);
  float* ks = xmalloc(sizeof(float) * ntok);
  float* w = xmalloc(sizeof(float) * ROWS * HI);
  for (int i = 0; i < ROWS * HI * DI; ++i) { qf[i] = uniform(); q8[i] = (uint8_t)(next_u32() & 0x7E); }
  for (int i = 0; i < ntok * DI; ++i) { kf[i] = uniform(); k8[i] = (uint8_t)(next_u32() & 0xFE); if ((k8[i] & 0x7F) == 0x7F) k8[i] = 0; }
  for (int i = 0; i < ntok; ++i) ks[i] = 0.01f + 0.001f * (float)(i % 7);
  for (int i = 0; i < ROWS * HI; ++i) w[i] = uniform();
  float* scores = xmalloc(sizeof(float) * ROWS * max_ctx);
  for (int i = 0; i < ROWS * max_ctx; ++i) scores[i] = -INFINITY;
  int32_t* q_seq = xmalloc(sizeof(int32_t) * ROWS);            /* a ragged mix: 1 row, then 5 rows */
  const int32_t qs[ROWS] = {1, 0, 0, 0, 0, 0};
  memcpy(q_seq, qs, sizeof qs);
  CHECK(oracle_indexer_scores(q8, w, k8, ks, pt, LDPT, PAGE, NPAGES, NULL, q_pos, ROWS, NSEQ, QPS, HI, DI, ORACLE_E4M3,
                              scores, max_ctx, 0, ROWS));
  CHECK(oracle_indexer_scores(qf, w, kf, NULL, pt, LDPT, PAGE, NPAGES, q_seq, q_pos, ROWS, NSEQ, 1, HI, DI, ORACLE_F32,
                              scores, max_ctx, 1, ROWS - 1));

  /* top-k: k above and below the prefix lengths, k = 1, ties */
  int32_t* idx = xmalloc(sizeof(int32_t) * ROWS * K);
  scores[1 * max_ctx + 3] = scores[1 * max_ctx + 4] = -0.0f;
  CHECK(oracle_topk(scores, max_ctx, q_pos, ROWS, K, idx, K, 0, ROWS));
  int32_t* idx1 = xmalloc(sizeof(int32_t) * ROWS);
  CHECK(oracle_topk(scores, max_ctx, q_pos, ROWS, 1, idx1, 1, 0, ROWS));

  /* attention over index sets: holes, repeats, invisible entries, an empty set */
  uint16_t* q = xmalloc(sizeof(uint16_t) * ROWS * H * DQK);
  uint16_t* kv = xmalloc(sizeof(uint16_t) * ntok * KVD);
  for (int i = 0; i < ROWS * H * DQK; ++i) q[i] = bf16_of(uniform());
  for (int i = 0; i < ntok * KVD; ++i) kv[i] = bf16_of(uniform());
  idx[2 * K + 5] = -1;
  idx[2 * K + 6] = idx[2 * K + 7];
  idx[3 * K + 0] = 64 + 9;             /* beyond q_pos = 63: invisible */
  for (int e = 0; e < K; ++e) idx[5 * K + e] = -1;
  float* out = xmalloc(sizeof(float) * ROWS * H * DV);
  float* lse = xmalloc(sizeof(float) * ROWS * H);
  CHECK(oracle_sparse_mla(q, kv, pt, LDPT, PAGE, NPAGES, NULL, q_pos, ROWS, NSEQ, QPS, idx, K, K, H, DQK, DV, KVD, V0,
                          0.3, out, lse, 0, ROWS));
  CHECK(oracle_sparse_mla(q, kv, pt, LDPT, PAGE, NPAGES, q_seq, q_pos, ROWS, NSEQ, 1, idx, K, K, H, DQK, DV, KVD, V0,
                          0.3, out, NULL, 2, 4));
  CHECK(oracle_dense_mla(q, kv, pt, LDPT, PAGE, NPAGES, NULL, q_pos, ROWS, NSEQ, QPS, H, DQK, DV, KVD, V0, 0.3, out,
                         lse, 0, ROWS));
  CHECK(oracle_dense_mla(q, kv, pt, LDPT, PAGE, NPAGES, q_seq, q_pos, ROWS, NSEQ, 1, H, DQK, DV, KVD, V0, 0.3, out,
                         lse, 0, ROWS));

  /* expanded attention, dense and masked */
  enum { DN = 16, DR = 8, DVX = 8 };
  const int ldkv = max_ctx;
  uint16_t* xq = xmalloc(sizeof(uint16_t) * ROWS * H * (DN + DR));
  uint16_t* xkn = xmalloc(sizeof(uint16_t) * NSEQ * H * ldkv * DN);
  uint16_t* xkr = xmalloc(sizeof(uint16_t) * NSEQ * ldkv * DR);
  uint16_t* xv = xmalloc(sizeof(uint16_t) * NSEQ * H * ldkv * DVX);
  for (int i = 0; i < ROWS * H * (DN + DR); ++i) xq[i] = bf16_of(uniform());
  for (int i = 0; i < NSEQ * H * ldkv * DN; ++i) xkn[i] = bf16_of(uniform());
  for (int i = 0; i < NSEQ * ldkv * DR; ++i) xkr[i] = bf16_of(uniform());
  for (int i = 0; i < NSEQ * H * ldkv * DVX; ++i) xv[i] = bf16_of(uniform());
  float* xo = xmalloc(sizeof(float) * ROWS * H * DVX);
  CHECK(oracle_mha(xq, xkn, xkr, xv, ldkv, q_pos, NSEQ, QPS, NULL, 0, 0, H, DN, DR, DVX, 0.2, xo, lse, 0, ROWS));
  CHECK(oracle_mha(xq, xkn, xkr, xv, ldkv, q_pos, NSEQ, QPS, idx, K, K, H, DN, DR, DVX, 0.2, xo, NULL, 0, ROWS));

  /* the step before the indexer: quantisation and both paged cache writes, with skipped tokens */
  enum { NT = 7 };
  float* src = xmalloc(sizeof(float) * NT * 128);
  for (int i = 0; i < NT * 128; ++i) src[i] = uniform() * 1000.0f;
  for (int c = 0; c < 128; ++c) src[2 * 128 + c] = 0.0f;          /* a zero key: scale 0 */
  uint8_t* codes = xmalloc((size_t)NT * 128);
  CHECK(oracle_e4m3_quantize(src, NT * 128, codes));
  int32_t* seq = xmalloc(sizeof(int32_t) * NT);
  int32_t* pos = xmalloc(sizeof(int32_t) * NT);
  const int32_t sq[NT] = {0, 1, 1, 2, -1, 0, 1}, ps[NT] = {0, 255, 100, 5, 3, 256, -4};
  memcpy(seq, sq, sizeof sq);
  memcpy(pos, ps, sizeof ps);
  uint8_t* kc = xmalloc((size_t)ntok * 128);
  float* ksc = xmalloc(sizeof(float) * ntok);
  int skipped = 0;
  CHECK(oracle_indexer_cache_write(src, ORACLE_F32, 128, seq, pos, NT, NSEQ, pt, LDPT, PAGE, NPAGES, kc, ksc, &skipped));
  uint16_t* lat = xmalloc(sizeof(uint16_t) * NT * KVD);
  for (int i = 0; i < NT * KVD; ++i) lat[i] = bf16_of(uniform());
  CHECK(oracle_latent_cache_write(lat, KVD, seq, pos, NT, NSEQ, pt, LDPT, PAGE, NPAGES, kv, &skipped));
  (void)oracle_e4m3_from_float(1e9f);
  (void)oracle_e4m3_from_float(-1e-9f);
  (void)oracle_e4m3_to_double(0x7F);
  (void)oracle_bf16_to_double(0xFFFF);

  free(pt); free(q_pos); free(q_seq); free(q8); free(qf); free(k8); free(kf); free(ks); free(w); free(scores); free(idx);
  free(idx1); free(q); free(kv); free(out); free(lse); free(xq); free(xkn); free(xkr); free(xv); free(xo);
  free(src); free(codes); free(seq); free(pos); free(kc); free(ksc); free(lat);
  printf("oracle driver: ok\n");
  return 0;
}
