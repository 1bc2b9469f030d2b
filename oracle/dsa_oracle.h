/* dsa_oracle.h -- host-pointer interface of the CPU oracle for the DeepSeek Sparse
 * Attention (DSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this library. It shares no source, header, table or helper with
 * the GPU library; the GPU library never calls it.
 *
 * Page references used in this file:
 *   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org)
 *   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io, ai-infra-handbooks)
 *
 * Conventions (shared by every function below):
 *   - Positions are 0-based; a query row at position t sees keys j in [0, t]
 *     ([DSA-blog] section "Lightning Indexer", notation j <= t; the worked example
 *     includes the query's own position).
 *   - Rows: `rows` query rows; row r sits at position q_pos[r] of sequence q_seq[r] when the
 *     per-row array q_seq is given (q_per_seq must then be 1), else of sequence r / q_per_seq
 *     with rows = n_seq * q_per_seq. A sequence id outside [0, n_seq) is an error (code 3).
 *   - Paged caches: position p of sequence s lives in physical row
 *       page_table[s * ld_pt + p / page_size] * page_size + p % page_size.
 *   - Every function processes rows [row_begin, row_end) only, so callers may split
 *     rows across threads. Return value: 0 on success, nonzero on a bad argument.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element formats of the indexer operands. */
#define ORACLE_E4M3 0 /* OCP FP8 E4M3FN bytes */
#define ORACLE_F32 1  /* IEEE binary32 */
#define ORACLE_BF16 2 /* bfloat16 bits (the cache-write inputs only) */

/* Exact decoders (OCP 8-bit floating point spec, E4M3FN; bfloat16 = top half of binary32). */
double oracle_e4m3_to_double(uint8_t code);
double oracle_bf16_to_double(uint16_t bits);

/* Lightning Indexer score ([DSA-blog] "Lightning Indexer", equation for I_tj;
 * [Handbook] "稀疏注意力：NSA 与 DSA", the index-score formula):
 *   I[r, j] = sum_h w[r, h] * ReLU( q[r, h, :] . k_j ),  j in [0, q_pos[r]],
 * with the dequantised key k_j = k_scale[row_j] * k8[row_j, :] (k_scale may be NULL => 1).
 * q: [rows, Hi, Di], k_cache: [num_pages*page_size, Di], both of element format `fmt`.
 * All arithmetic in double; each score is rounded once to float.
 * scores[r * ld_scores + j] is written for j <= q_pos[r] only. */
int oracle_indexer_scores(const void* q, const float* w, const void* k_cache, const float* k_scale,
                          const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                          const int32_t* q_seq, const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                          int Hi, int Di, int fmt, float* scores, int64_t ld_scores, int row_begin, int row_end);

/* Top-k ([DSA-blog] "Lightning Indexer", S_t = TopK_{j<=t}(I_tj, k)): for row r the
 * m = min(k, q_pos[r] + 1) positions with the largest score; equal scores are ordered by
 * the smaller position first; -0 and +0 compare equal. The chosen positions are written in
 * ascending order to idx[r * ld_idx + 0 .. m-1]; slots m .. k-1 get -1. */
int oracle_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows, int k,
                int32_t* idx, int64_t ld_idx, int row_begin, int row_end);

/* Sparse attention on the selected rows ([DSA-blog] "Sparse Attention", the masked-softmax
 * equation, evaluated only on S_t; [Handbook] absorbed MLA: one latent row per position
 * serves as key for all heads, its first Dv columns after v_col0 as value):
 *   for head h:  l_j = sm_scale * q[r,h,:Dqk] . row_j[0:Dqk]          for j in S
 *                o[r,h,:] = sum_j softmax(l)_j * row_j[v_col0 : v_col0+Dv]
 *                lse[r,h] = log sum_j exp(l_j)
 * S = the set of positions that idx[r * ld_idx + 0 .. k-1] lists within [0, q_pos[r]]: a
 * position listed several times is in S once ([DSA-blog] "Sparse Attention": M_tj = 0 exactly
 * when j is in S_t, so S_t is a set), and S is visited in ascending position order. Entries
 * outside that range (e.g. the -1 padding) are not visible and are skipped.
 * An empty S gives o = 0 and lse = -inf. q: bf16 [rows, H, Dqk]; kv_cache: bf16
 * [num_pages*page_size, kv_dim]; out: float [rows, H, Dv]; lse: float [rows, H] or NULL. */
int oracle_sparse_mla(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                      int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                      int rows, int n_seq, int q_per_seq, const int32_t* idx, int64_t ld_idx, int k, int H,
                      int Dqk, int Dv, int kv_dim, int v_col0, double sm_scale, float* out, float* lse,
                      int row_begin, int row_end);

/* Dense causal attention: the same computation with S = {0, 1, ..., q_pos[r]} visited in
 * ascending order ([DSA-blog] "SWA" section, the causal set C_t). */
int oracle_dense_mla(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                     int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                     int rows, int n_seq, int q_per_seq, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                     double sm_scale, float* out, float* lse, int row_begin, int row_end);

/* Expanded multi-head attention, the short-prefill fallback ([Handbook] "稀疏注意力：NSA 与
 * DSA": the expanded pair of the cost model, per head 128 + 64 (rope) query/key dims and 128
 * value dims, and the masked MHA mode that emulates DSA for short prefill). For row r of
 * sequence s at position t and head h: K_hj = [k_nope[s,h,j,:] | k_rope[s,j,:]],
 * V_hj = v[s,h,j,:], S = {0..t} (idx NULL) or the idx[r] entries within [0, t] taken as a set;
 * out = softmax(sm_scale q K^T over S) V in double, rounded to float; lse natural log.
 *   q [rows, H, Dn+Dr]; k_nope [n_seq, H, ld_kv, Dn]; k_rope [n_seq, ld_kv, Dr];
 *   v [n_seq, H, ld_kv, Dv] (all bf16 bits); out [rows, H, Dv]; lse [rows, H] or NULL. */
int oracle_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
               int64_t ld_kv, const int32_t* q_pos, int n_seq, int q_per_seq, const int32_t* idx,
               int64_t ld_idx, int k, int H, int Dn, int Dr, int Dv, double sm_scale, float* out,
               float* lse, int row_begin, int row_end);

/* Upstream of the indexer ([DSA-blog] "Lightning Indexer": keys from each position's hidden
 * state, cached in their own cache; [Handbook] "对推理引擎的新要求": both caches paged, the indexer
 * key cache holding FP8 codes plus a float scale per token):
 *   oracle_e4m3_from_float      float -> E4M3FN, round to nearest even, saturating to +-448
 *   oracle_e4m3_quantize        elementwise, no scale (the indexer query)
 *   oracle_indexer_cache_write  per token s = max|k| / 448 (float), codes E4M3(k / s) (float
 *                               quotient; zero when s = 0), written at the token's physical row
 *   oracle_latent_cache_write   each token's latent row copied to its physical row
 * Tokens whose sequence is not in [0, n_seq) (page_table is [n_seq, ld_pt]) or whose position has
 * no valid page are skipped and counted in *skipped. */
uint8_t oracle_e4m3_from_float(float x);
int oracle_e4m3_quantize(const float* x, int64_t n, uint8_t* out);
int oracle_indexer_cache_write(const void* k, int fmt, int Di, const int32_t* seq, const int32_t* pos,
                               int n_tok, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                               int num_pages, uint8_t* k_cache, float* k_scale, int* skipped);
int oracle_latent_cache_write(const uint16_t* rows, int kv_dim, const int32_t* seq, const int32_t* pos,
                              int n_tok, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                              int num_pages, uint16_t* kv_cache, int* skipped);

/* The indexer's projections ([DSA-blog] "Lightning Indexer", the first step of its figure), linear
 * layers with weights in the [out, in] layout on bf16 inputs, each output summed in double and
 * rounded once to float:
 *   oracle_indexer_key_project    k = h w_k^T (h [n_tok, d], w_k [Di, d]), then the key format and
 *                                 placement of oracle_indexer_cache_write; k_out (or NULL) gets k
 *   oracle_indexer_query_project  q8 = E4M3(c_q w_q^T) (c_q [rows, d_cq], w_q [Hi*Di, d_cq]; no
 *                                 scale) and w = h w_w^T (h [rows, d], w_w [Hi, d]) in float; q_out
 *                                 (or NULL) gets q before its coding */
int oracle_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int Di, const int32_t* seq,
                               const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                               int num_pages, uint8_t* k_cache, float* k_scale, float* k_out, int* skipped);
int oracle_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h, const uint16_t* w_w,
                                 int rows, int d_cq, int d, int Hi, int Di, uint8_t* q8, float* w, float* q_out);

#ifdef __cplusplus
}
#endif
#endif
