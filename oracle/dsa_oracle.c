/* dsa_oracle.c -- plain, slow, double-precision CPU statement of the DeepSeek Sparse
 * Attention (DSA) hot path: Lightning Indexer scores, exact top-k, sparse attention on
 * the selected latent rows, and dense causal attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the benchmark's CPU
 * baseline, never by the GPU library. No code here is shared with the GPU path.
 *
 * Page references:
 *   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org)
 *   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io, ai-infra-handbooks)
 *
 * The method is exact (no approximation, no iteration), so each function is the plain
 * definition written out with double accumulation and one final rounding to float.
 * Readings taken where the pages leave a step open are listed beside the code.
 *
 * Pins: every function here is checked against values fixed independently of this file
 * (the worked example, closed forms, library routines, brute force); see tests/test_oracle.py.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoders ------------------------------------------------------------- */

/* OCP 8-bit floating point, E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities. */
double oracle_e4m3_to_double(uint8_t code) {
  int sign = code >> 7;
  int expo = (code >> 3) & 0xF;
  int mant = code & 0x7;
  double mag;
  if (expo == 0xF && mant == 0x7) return NAN;
  if (expo == 0)
    mag = ldexp((double)mant / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);
  return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int64_t i, int fmt) {
  if (fmt == ORACLE_E4M3) return oracle_e4m3_to_double(((const uint8_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* Physical row of position p of sequence s in a paged cache; -1 if p lies outside the sequence's
 * page-table row or the page id is invalid. */
static int64_t phys_row(const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                        int s, int64_t p) {
  if (p < 0 || p / page_size >= ld_pt) return -1; /* outside the sequence's page table row */
  int32_t page = page_table[(int64_t)s * ld_pt + p / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + p % page_size;
}

/* The query-row descriptor: `rows` rows; row r belongs to sequence q_seq[r] when q_seq is given
 * (then q_per_seq must be 1), else to sequence r / q_per_seq with rows = n_seq * q_per_seq. */
static int bad_common(const int32_t* q_seq, int rows, int n_seq, int q_per_seq, int row_begin, int row_end) {
  if (rows < 0 || n_seq < 0 || q_per_seq < 1) return 1;
  if (q_seq ? q_per_seq != 1 : (int64_t)n_seq * q_per_seq != rows) return 1;
  if (row_begin < 0 || row_end > rows || row_begin > row_end) return 1;
  return 0;
}

/* Sequence of row r, or -1 when its id lies outside [0, n_seq). */
static int seq_of(const int32_t* q_seq, int q_per_seq, int n_seq, int r) {
  int s = q_seq ? q_seq[r] : r / q_per_seq;
  return (s >= 0 && s < n_seq) ? s : -1;
}

/* ---- Lightning Indexer ------------------------------------------------------------ */

/* [DSA-blog] "Lightning Indexer": I_tj = sum over indexer heads r of
 * w_tr * ReLU(q_tr . k_j), for every visible j <= t, one key k_j shared by all heads.
 * Reading (key scale): the cached key is k_j = k_scale_j * k8_j, dequantised before the
 * dot product exactly as written here. */
int oracle_indexer_scores(const void* q, const float* w, const void* k_cache, const float* k_scale,
                          const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                          const int32_t* q_seq, const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                          int Hi, int Di, int fmt, float* scores, int64_t ld_scores, int row_begin, int row_end) {
  if (bad_common(q_seq, rows, n_seq, q_per_seq, row_begin, row_end)) return 1;
  if (Hi < 1 || Di < 1 || page_size < 1 || (fmt != ORACLE_E4M3 && fmt != ORACLE_F32)) return 1;
  double* key = (double*)malloc(sizeof(double) * (size_t)Di);
  if (!key) return 2;
  for (int r = row_begin; r < row_end; ++r) {
    int s = seq_of(q_seq, q_per_seq, n_seq, r);
    int64_t t = q_pos[r];
    if (s < 0) { free(key); return 3; }
    for (int64_t j = 0; j <= t; ++j) {
      int64_t row = phys_row(page_table, ld_pt, page_size, num_pages, s, j);
      if (row < 0) { free(key); return 3; }
      double scale = k_scale ? (double)k_scale[row] : 1.0;
      for (int c = 0; c < Di; ++c) key[c] = scale * elem(k_cache, row * Di + c, fmt);
      double score = 0.0;
      for (int h = 0; h < Hi; ++h) {
        double dot = 0.0;
        for (int c = 0; c < Di; ++c) dot += elem(q, ((int64_t)r * Hi + h) * Di + c, fmt) * key[c];
        double relu = dot > 0.0 ? dot : 0.0;
        score += (double)w[(int64_t)r * Hi + h] * relu;
      }
      scores[(int64_t)r * ld_scores + j] = (float)score;
    }
  }
  free(key);
  return 0;
}

/* ---- top-k ------------------------------------------------------------------------ */

typedef struct {
  float v;
  int32_t j;
} cand_t;

/* Larger score first; equal scores (by value, so -0 == +0) by smaller position first. */
static int cmp_rank(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int cmp_i32(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* [DSA-blog] "Lightning Indexer": S_t = TopK over j <= t of I_tj with k positions;
 * [Handbook] cost model: k = min(L, 2048), i.e. a prefix shorter than k keeps every
 * position. Reading (ties): equal scores rank the smaller position first. */
int oracle_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows, int k,
                int32_t* idx, int64_t ld_idx, int row_begin, int row_end) {
  if (k < 1 || rows < 0 || row_begin < 0 || row_end > rows || row_begin > row_end) return 1;
  for (int r = row_begin; r < row_end; ++r) {
    int64_t n = (int64_t)q_pos[r] + 1;
    if (n < 0) n = 0;
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
    if (!c) return 2;
    for (int64_t j = 0; j < n; ++j) {
      c[j].v = scores[(int64_t)r * ld_scores + j];
      c[j].j = (int32_t)j;
    }
    qsort(c, (size_t)n, sizeof(cand_t), cmp_rank);
    int64_t m = n < k ? n : k;
    int32_t* out = idx + (int64_t)r * ld_idx;
    for (int64_t i = 0; i < m; ++i) out[i] = c[i].j;
    qsort(out, (size_t)m, sizeof(int32_t), cmp_i32);
    for (int64_t i = m; i < k; ++i) out[i] = -1;
    free(c);
  }
  return 0;
}

/* ---- attention over a position set -------------------------------------------------- */

/* Softmax attention of one query row over the listed positions ([DSA-blog] "Sparse
 * Attention": softmax(q K^T / sqrt(d_h) + M) V with M = 0 on S_t and -inf elsewhere, which
 * on S_t alone is an ordinary softmax). Two passes: logits and their maximum, then the
 * normalised weighted sum of value rows. */
static int attend_row(const uint16_t* q_row /* [H, Dqk] */, const uint16_t* kv_cache,
                      const int64_t* rows_of_set, int64_t n_set, int H, int Dqk, int Dv,
                      int kv_dim, int v_col0, double sm_scale, float* out /* [H, Dv] */,
                      float* lse /* [H] or NULL */) {
  double* logit = (double*)malloc(sizeof(double) * (size_t)(n_set > 0 ? n_set : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)Dv);
  if (!logit || !acc) { free(logit); free(acc); return 2; }
  for (int h = 0; h < H; ++h) {
    const uint16_t* qh = q_row + (int64_t)h * Dqk;
    double mx = -INFINITY;
    for (int64_t i = 0; i < n_set; ++i) {
      const uint16_t* kr = kv_cache + rows_of_set[i] * kv_dim;
      double dot = 0.0;
      for (int c = 0; c < Dqk; ++c) dot += oracle_bf16_to_double(qh[c]) * oracle_bf16_to_double(kr[c]);
      logit[i] = sm_scale * dot;
      if (logit[i] > mx) mx = logit[i];
    }
    for (int c = 0; c < Dv; ++c) acc[c] = 0.0;
    double denom = 0.0;
    for (int64_t i = 0; i < n_set; ++i) {
      double p = exp(logit[i] - mx);
      const uint16_t* vr = kv_cache + rows_of_set[i] * kv_dim + v_col0;
      denom += p;
      for (int c = 0; c < Dv; ++c) acc[c] += p * oracle_bf16_to_double(vr[c]);
    }
    for (int c = 0; c < Dv; ++c) out[(int64_t)h * Dv + c] = n_set > 0 ? (float)(acc[c] / denom) : 0.0f;
    if (lse) lse[h] = n_set > 0 ? (float)(mx + log(denom)) : -INFINITY;
  }
  free(logit);
  free(acc);
  return 0;
}

static int bad_attn(int H, int Dqk, int Dv, int kv_dim, int v_col0, int page_size) {
  if (H < 1 || Dqk < 1 || Dv < 1 || page_size < 1) return 1;
  if (Dqk > kv_dim || v_col0 < 0 || v_col0 + Dv > kv_dim) return 1;
  return 0;
}

int oracle_sparse_mla(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                      int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                      int rows, int n_seq, int q_per_seq, const int32_t* idx, int64_t ld_idx, int k, int H,
                      int Dqk, int Dv, int kv_dim, int v_col0, double sm_scale, float* out, float* lse,
                      int row_begin, int row_end) {
  if (bad_common(q_seq, rows, n_seq, q_per_seq, row_begin, row_end) || k < 0) return 1;
  if (bad_attn(H, Dqk, Dv, kv_dim, v_col0, page_size)) return 1;
  int64_t* set = (int64_t*)malloc(sizeof(int64_t) * (size_t)(k > 0 ? k : 1));
  if (!set) return 2;
  for (int r = row_begin; r < row_end; ++r) {
    int s = seq_of(q_seq, q_per_seq, n_seq, r);
    int64_t t = q_pos[r], n_set = 0;
    if (s < 0) { free(set); return 3; }
    /* S_t is a set ([DSA-blog] "Sparse Attention": the mask is 0 exactly on S_t): mark every
     * listed visible position once, then visit the marked positions in ascending order */
    unsigned char* in_set = (unsigned char*)calloc((size_t)(t >= 0 ? t + 1 : 1), 1);
    if (!in_set) { free(set); return 2; }
    for (int i = 0; i < k; ++i) {
      int64_t j = idx[(int64_t)r * ld_idx + i];
      if (j < 0 || j > t) continue; /* not a visible position, so not in S_t */
      in_set[j] = 1;
    }
    for (int64_t j = 0; j <= t; ++j) {
      if (!in_set[j]) continue;
      int64_t row = phys_row(page_table, ld_pt, page_size, num_pages, s, j);
      if (row < 0) { free(in_set); free(set); return 3; }
      set[n_set++] = row;
    }
    free(in_set);
    int rc = attend_row(q + (int64_t)r * H * Dqk, kv_cache, set, n_set, H, Dqk, Dv, kv_dim, v_col0,
                        sm_scale, out + (int64_t)r * H * Dv, lse ? lse + (int64_t)r * H : NULL);
    if (rc) { free(set); return rc; }
  }
  free(set);
  return 0;
}

int oracle_dense_mla(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                     int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                     int rows, int n_seq, int q_per_seq, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                     double sm_scale, float* out, float* lse, int row_begin, int row_end) {
  if (bad_common(q_seq, rows, n_seq, q_per_seq, row_begin, row_end)) return 1;
  if (bad_attn(H, Dqk, Dv, kv_dim, v_col0, page_size)) return 1;
  for (int r = row_begin; r < row_end; ++r) {
    int s = seq_of(q_seq, q_per_seq, n_seq, r);
    if (s < 0) return 3;
    int64_t n_set = (int64_t)q_pos[r] + 1;
    if (n_set < 0) n_set = 0;
    int64_t* set = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_set > 0 ? n_set : 1));
    if (!set) return 2;
    for (int64_t j = 0; j < n_set; ++j) {
      set[j] = phys_row(page_table, ld_pt, page_size, num_pages, s, j);
      if (set[j] < 0) { free(set); return 3; }
    }
    int rc = attend_row(q + (int64_t)r * H * Dqk, kv_cache, set, n_set, H, Dqk, Dv, kv_dim, v_col0,
                        sm_scale, out + (int64_t)r * H * Dv, lse ? lse + (int64_t)r * H : NULL);
    free(set);
    if (rc) return rc;
  }
  return 0;
}

/* ---- expanded multi-head attention (the short-prefill fallback) ----------------------- */

/* [Handbook] "稀疏注意力：NSA 与 DSA", the cost model's expanded pair and the note on short
 * prefill: the dense fallback runs multi-head attention with per-head keys of 128 + 64 (rope)
 * dims and 128-dim values, and V3.2 emulates the DSA mask in that mode. For row r (sequence
 * s = r / q_per_seq, position t = q_pos[r]) and head h, with
 *   K_hj = [k_nope[s, h, j, 0:Dn] | k_rope[s, j, 0:Dr]]   (the rope part is shared by all heads)
 *   V_hj = v[s, h, j, 0:Dv]
 * the set S is {0..t} when idx is NULL, else the positions j in [0, t] listed in idx[r, 0:k]
 * (as a set: a repeated entry counts once, [DSA-blog] "Sparse Attention", M = 0 on S_t);
 * positions are taken in ascending order, and the softmax is attend_row's two passes. */
int oracle_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
               int64_t ld_kv, const int32_t* q_pos, int n_seq, int q_per_seq, const int32_t* idx,
               int64_t ld_idx, int k, int H, int Dn, int Dr, int Dv, double sm_scale, float* out,
               float* lse, int row_begin, int row_end) {
  if (bad_common(NULL, n_seq * q_per_seq, n_seq, q_per_seq, row_begin, row_end) || k < 0) return 1;
  if (H < 1 || Dn < 1 || Dr < 0 || Dv < 1 || ld_kv < 1) return 1;
  const int Dq = Dn + Dr;
  unsigned char* in_set = (unsigned char*)malloc((size_t)ld_kv);
  double* logit = (double*)malloc(sizeof(double) * (size_t)ld_kv);
  double* acc = (double*)malloc(sizeof(double) * (size_t)Dv);
  if (!in_set || !logit || !acc) { free(in_set); free(logit); free(acc); return 2; }
  for (int r = row_begin; r < row_end; ++r) {
    const int s = r / q_per_seq;
    const int64_t t = q_pos[r];
    if (t >= ld_kv) { free(in_set); free(logit); free(acc); return 3; }
    for (int64_t j = 0; j < ld_kv; ++j) in_set[j] = (unsigned char)(idx == NULL && j <= t);
    if (idx)
      for (int i = 0; i < k; ++i) {
        const int64_t j = idx[(int64_t)r * ld_idx + i];
        if (j >= 0 && j <= t) in_set[j] = 1;
      }
    for (int h = 0; h < H; ++h) {
      const uint16_t* qh = q + ((int64_t)r * H + h) * Dq;
      double mx = -INFINITY;
      int64_t n = 0;
      for (int64_t j = 0; j <= t; ++j) {
        if (!in_set[j]) continue;
        const uint16_t* kn = k_nope + (((int64_t)s * H + h) * ld_kv + j) * Dn;
        const uint16_t* kr = k_rope + ((int64_t)s * ld_kv + j) * Dr;
        double dot = 0.0;
        for (int c = 0; c < Dn; ++c) dot += oracle_bf16_to_double(qh[c]) * oracle_bf16_to_double(kn[c]);
        for (int c = 0; c < Dr; ++c) dot += oracle_bf16_to_double(qh[Dn + c]) * oracle_bf16_to_double(kr[c]);
        logit[j] = sm_scale * dot;
        if (logit[j] > mx) mx = logit[j];
        ++n;
      }
      for (int c = 0; c < Dv; ++c) acc[c] = 0.0;
      double denom = 0.0;
      for (int64_t j = 0; j <= t; ++j) {
        if (!in_set[j]) continue;
        const double p = exp(logit[j] - mx);
        const uint16_t* vr = v + (((int64_t)s * H + h) * ld_kv + j) * Dv;
        denom += p;
        for (int c = 0; c < Dv; ++c) acc[c] += p * oracle_bf16_to_double(vr[c]);
      }
      for (int c = 0; c < Dv; ++c) out[((int64_t)r * H + h) * Dv + c] = n > 0 ? (float)(acc[c] / denom) : 0.0f;
      if (lse) lse[(int64_t)r * H + h] = n > 0 ? (float)(mx + log(denom)) : -INFINITY;
    }
  }
  free(in_set);
  free(logit);
  free(acc);
  return 0;
}

/* ---- upstream: FP8 quantisation and the paged cache writes ---------------------------- */

/* OCP 8-bit floating point, E4M3FN, from a float: round to nearest, ties to even, saturating
 * to +-448 (the largest finite value; the format has no infinity). Finite input only. Worked
 * from the format's definition: subnormals are multiples of 2^-9 below 2^-6; a normal value
 * 2^e * (1 + m/8) has exponent field e + 7 and mantissa field m. */
uint8_t oracle_e4m3_from_float(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: the code is the count of 2^-9 quanta (8 quanta = the smallest normal,
     * whose code is also 8) */
    return (uint8_t)(sign | (uint8_t)rint(a * 512.0));
  }
  int e2;
  frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1): the binade is 2^(e2-1) */
  const int e = e2 - 1;   /* -6 .. 8 */
  double n = rint(ldexp(a, 3 - e));  /* a / 2^(e-3), in [8, 16] after rounding */
  int ee = e;
  if (n >= 16.0) { n = 8.0; ++ee; }
  const int field = ee + 7;
  if (field > 15 || (field == 15 && n - 8.0 > 6.0)) return (uint8_t)(sign | 0x7E);
  return (uint8_t)(sign | (uint8_t)(field << 3) | (uint8_t)(n - 8.0));
}

/* The indexer query in FP8 without a scale (no query scale is given on the pages; the query
 * is quantised as is). */
int oracle_e4m3_quantize(const float* x, int64_t n, uint8_t* out) {
  if (n < 0) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_float(x[i]);
  return 0;
}

/* The Indexer Key Cache write ([DSA-blog] "Lightning Indexer": each position's indexer key comes
 * from its own hidden state and is cached; [Handbook] "对推理引擎的新要求": the indexer keys are
 * paged like the latent cache, IDX_D + 4 bytes per token). Per token: the scale
 * s = max_c |k_c| / 448 in float, the codes E4M3(k_c / s) with the quotient in float (all zero
 * when s = 0), written at the token's physical row. Tokens whose sequence is not in [0, n_seq) or
 * whose position has no valid page are skipped (their count is put in *skipped). fmt: ORACLE_F32 or
 * ORACLE_BF16 input rows [n_tok, Di]. */
int oracle_indexer_cache_write(const void* k, int fmt, int Di, const int32_t* seq, const int32_t* pos,
                               int n_tok, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                               int num_pages, uint8_t* k_cache, float* k_scale, int* skipped) {
  if (Di < 1 || n_tok < 0 || page_size < 1 || (fmt != ORACLE_F32 && fmt != ORACLE_BF16)) return 1;
  int skip = 0;
  float* row = (float*)malloc(sizeof(float) * (size_t)Di);
  if (!row) return 2;
  for (int t = 0; t < n_tok; ++t) {
    const int64_t r = seq[t] >= 0 && seq[t] < n_seq ? phys_row(page_table, ld_pt, page_size, num_pages, seq[t], pos[t]) : -1;
    if (r < 0) { ++skip; continue; }
    float mx = 0.0f;
    for (int c = 0; c < Di; ++c) {
      row[c] = fmt == ORACLE_F32 ? ((const float*)k)[(int64_t)t * Di + c]
                                 : (float)oracle_bf16_to_double(((const uint16_t*)k)[(int64_t)t * Di + c]);
      const float v = fabsf(row[c]);
      if (v > mx) mx = v;
    }
    const float s = mx / 448.0f;
    for (int c = 0; c < Di; ++c) k_cache[r * Di + c] = s > 0.0f ? oracle_e4m3_from_float(row[c] / s) : 0;
    k_scale[r] = s;
  }
  free(row);
  if (skipped) *skipped = skip;
  return 0;
}

/* The latent cache write: each token's row (kv_dim bf16: the 512 latent dims, then the 64 rope
 * dims) copied to its physical row; tokens without a valid page are skipped. */
int oracle_latent_cache_write(const uint16_t* rows, int kv_dim, const int32_t* seq, const int32_t* pos,
                              int n_tok, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                              int num_pages, uint16_t* kv_cache, int* skipped) {
  if (kv_dim < 1 || n_tok < 0 || page_size < 1) return 1;
  int skip = 0;
  for (int t = 0; t < n_tok; ++t) {
    const int64_t r = seq[t] >= 0 && seq[t] < n_seq ? phys_row(page_table, ld_pt, page_size, num_pages, seq[t], pos[t]) : -1;
    if (r < 0) { ++skip; continue; }
    for (int c = 0; c < kv_dim; ++c) kv_cache[r * kv_dim + c] = rows[(int64_t)t * kv_dim + c];
  }
  if (skipped) *skipped = skip;
  return 0;
}

/* ---- the indexer's projections --------------------------------------------------------- */

/* out[i, o] = sum_c x[i, c] * wt[o, c] over c < K in double, rounded once to float: a linear layer
 * with its weights in the [out, in] layout, on bf16 inputs. */
static void linear_bf16(const uint16_t* x, const uint16_t* wt, int rows, int K, int N, float* out) {
  for (int i = 0; i < rows; ++i)
    for (int o = 0; o < N; ++o) {
      double acc = 0.0;
      for (int c = 0; c < K; ++c)
        acc += oracle_bf16_to_double(x[(int64_t)i * K + c]) * oracle_bf16_to_double(wt[(int64_t)o * K + c]);
      out[(int64_t)i * N + o] = (float)acc;
    }
}

/* [DSA-blog] "Lightning Indexer", the first step of its figure: every position's hidden state h_j
 * gives the one indexer key k_j all heads share, kept in the Indexer Key Cache. k = h w_k^T, then
 * the key format of oracle_indexer_cache_write (per token s = max|k| / 448, codes E4M3(k / s)).
 * The keys before quantisation go to k_out [n_tok, Di] when it is not NULL. */
int oracle_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int Di, const int32_t* seq,
                               const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                               int num_pages, uint8_t* k_cache, float* k_scale, float* k_out, int* skipped) {
  if (n_tok < 0 || d < 1 || Di < 1) return 1;
  float* k = (float*)malloc(sizeof(float) * (size_t)(n_tok > 0 ? n_tok : 1) * (size_t)Di);
  if (!k) return 2;
  linear_bf16(h, w_k, n_tok, d, Di, k);
  int rc = oracle_indexer_cache_write(k, ORACLE_F32, Di, seq, pos, n_tok, n_seq, page_table, ld_pt, page_size,
                                      num_pages, k_cache, k_scale, skipped);
  if (k_out) memcpy(k_out, k, sizeof(float) * (size_t)n_tok * (size_t)Di);
  free(k);
  return rc;
}

/* [DSA-blog] "Lightning Indexer", the first step of its figure: the query path takes the MLA query
 * latent c_q and applies the indexer projection to get the n_h^I query heads, and the current
 * token's hidden state h gives the head weights. q = c_q w_q^T coded E4M3 without a scale (the pages
 * give the indexer query none), w = h w_w^T in float. q_out [rows, Hi * Di] receives q before its
 * coding when not NULL. */
int oracle_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h, const uint16_t* w_w,
                                 int rows, int d_cq, int d, int Hi, int Di, uint8_t* q8, float* w, float* q_out) {
  if (rows < 0 || d_cq < 1 || d < 1 || Hi < 1 || Di < 1) return 1;
  const int64_t n = (int64_t)rows * Hi * Di;
  float* q = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  if (!q) return 2;
  linear_bf16(c_q, w_q, rows, d_cq, Hi * Di, q);
  int rc = oracle_e4m3_quantize(q, n, q8);
  if (q_out) memcpy(q_out, q, sizeof(float) * (size_t)n);
  free(q);
  if (rc) return rc;
  linear_bf16(h, w_w, rows, d, Hi, w);
  return 0;
}
