/* dsa.h -- C ABI of libdsa.so: the DeepSeek Sparse Attention (DSA) hot path on gfx950.
 *
 * Page references:
 *   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org)
 *   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io, ai-infra-handbooks)
 *
 * The path, per query row: the Lightning Indexer scores every visible position
 * (dsa_indexer_scores), an exact top-k picks the index set S_t (dsa_topk), and attention runs
 * over the latent rows in S_t only (dsa_sparse_mla_decode / dsa_sparse_mla_prefill). A dense
 * causal attention (dsa_dense_mla_prefill) serves short prefill, where it equals DSA exactly
 * whenever every prefix is no longer than k.
 *
 * Common conventions
 * ------------------
 * Pointers: every array argument is a DEVICE pointer (HIP global memory) unless stated
 *   otherwise; `stream` is a hipStream_t passed as void* (NULL = the null stream). The caller
 *   owns all memory. The library never allocates, frees or synchronises: each call validates
 *   its host-side arguments, then only enqueues kernels on `stream` and returns. Arrays must
 *   stay valid until that work completes. Calls on different streams are independent.
 * Rows: a call processes `rows` query rows. Row r sits at 0-based position q_pos[r] (device
 *   int32 [rows]) of its sequence and sees positions j in [0, q_pos[r]], itself included
 *   ([DSA-blog] "Lightning Indexer": j <= t; the worked example selects the query's own position
 *   8). Its sequence (the page-table row of its caches) is given in one of two ways:
 *     q_seq == NULL   rows = n_seq * q_per_seq, and row r belongs to sequence r / q_per_seq:
 *                     decode uses q_per_seq = 1, MTP verification q_per_seq = 2 (both rows of a
 *                     request share one scan of its keys), a prefill chunk n_seq = 1 and
 *                     q_per_seq = chunk length;
 *     q_seq != NULL   device int32 [rows]: row r belongs to sequence q_seq[r], in [0, n_seq);
 *                     q_per_seq must be 1. Any mix of rows fits (a decode batch beside a prefill
 *                     chunk, requests with different numbers of rows); the indexer then scans
 *                     each row's keys on its own. A row whose q_seq is outside [0, n_seq) has no
 *                     page-table row: no access is made for it and its results are unspecified.
 * Paging: both caches are paged. Position p of sequence s is physical row
 *   page_table[s * ld_pt + p / page_size] * page_size + p % page_size
 *   of a cache holding num_pages * page_size rows. page_table is device int32 [n_seq, ld_pt].
 *   A contiguous cache is the identity table.
 * Host bound: max_ctx (host int) must exceed every q_pos; it sizes grids so that no call has
 *   to read device memory on the host. Page ids and positions outside their ranges never cause
 *   an out-of-bounds access (kernels bound-check them); the affected results are unspecified.
 * Errors: DSA_ERR_INVALID_ARG for a bad host argument (null pointer, 16-byte misalignment of
 *   a cache or activation array, non-positive size, inconsistent dims), DSA_ERR_WORKSPACE for
 *   a missing or small workspace, DSA_ERR_UNSUPPORTED for a shape no kernel here handles (the
 *   library never substitutes a different computation), DSA_ERR_HIP when a launch fails. On
 *   any error nothing is enqueued (a DSA_ERR_HIP may follow partial work of the same call).
 *   dsa_last_error() gives a message for the calling thread's last failed call.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE = 3,
  DSA_ERR_HIP = 4
} dsa_status_t;

/* Element format of the indexer operands. */
typedef enum {
  DSA_E4M3 = 0, /* OCP FP8 E4M3FN bytes (gfx950's native FP8) */
  DSA_F32 = 1,  /* IEEE binary32 */
  DSA_BF16 = 2  /* bfloat16 (dsa_indexer_cache_write input only) */
} dsa_dtype_t;

/* Kernel variants reported by dsa_last_path() (observability only, never a control). */
enum {
  DSA_PATH_NONE = 0,
  DSA_PATH_INDEXER_GENERIC = 1,       /* any Hi, Di, dtype: one thread per (row, key), VALU */
  DSA_PATH_INDEXER_SCAN_MFMA = 2,     /* Hi=64, Di=128, E4M3, 64-token pages: key scan, 2 rows/wave */
  DSA_PATH_INDEXER_PREFILL_MFMA = 3,  /* Hi=64, Di=128, E4M3, other page sizes: query x key tiles */
  DSA_PATH_INDEXER_TOPK_FUSED = 4,    /* dsa_indexer_topk: scan counting the first radix digit, then
                                         the register top-k starting from those counts */
  DSA_PATH_TOPK_COPY = 10,            /* every row no longer than k: all positions kept */
  DSA_PATH_TOPK_RADIX = 11,           /* radix select, one workgroup per row */
  DSA_PATH_TOPK_RADIX_REG = 12,       /* as 11 for max_ctx <= 16384, the row held in registers */
  DSA_PATH_TOPK_RADIX_STAGED = 13,    /* longer rows: per-chunk candidates, then a merge (workspace) */
  DSA_PATH_MLA_GENERIC = 20,          /* any shape: one wave per (row, head), VALU */
  DSA_PATH_MLA_MFMA = 21,             /* H=128, Dqk=576, Dv=512: bf16 MFMA, one pass */
  DSA_PATH_MLA_MFMA_SPLIT = 22,       /* as 21, key set split over workgroups + combine */
  DSA_PATH_MHA_MFMA = 30,             /* expanded attention, dense causal: bf16 MFMA */
  DSA_PATH_MHA_MFMA_MASKED = 31,      /* as 30, restricted to the index sets (bitmap in ws) */
  DSA_PATH_CACHE_WRITE = 40,          /* quantise / place rows into a paged cache */
  DSA_PATH_QUANTIZE = 41,             /* elementwise E4M3 quantisation */
  DSA_PATH_PROJECT = 42               /* indexer projections: bf16 MFMA GEMM + quantise / place */
};

const char* dsa_status_string(dsa_status_t status);
/* Message of the calling thread's most recent failed call ("" if none). */
const char* dsa_last_error(void);
/* DSA_PATH_* of the kernel variant used by the calling thread's most recent successful call. */
int dsa_last_path(void);

/* ---------------------------------------------------------------------------------------------
 * dsa_indexer_scores -- Lightning Indexer ([DSA-blog] "Lightning Indexer", the equation for
 * I_tj; [Handbook] "稀疏注意力：NSA 与 DSA", index score with 64 heads of 128 dims, FP8):
 *     scores[r, j] = k_scale[j] * sum_h w[r, h] * ReLU( q[r, h, :] . k8[j, :] ),  j <= q_pos[r]
 * i.e. the page's I_tj with the dequantised key k_j = k_scale_j * k8_j (k_scale > 0, so the
 * scale commutes with ReLU).
 *   q        [rows, Hi, Di]        E4M3 bytes or f32 (per dtype), 16-byte aligned
 *   w        [rows, Hi]            f32 head weights
 *   k_cache  [num_pages, page_size, Di]  E4M3 or f32, 16-byte aligned
 *   k_scale  [num_pages, page_size] f32 per-token key scale, or NULL for 1
 *   scores   [rows, ld_scores] f32, ld_scores >= max_ctx; entries j <= q_pos[r] are written,
 *            entries q_pos[r] < j < max_ctx may be written with -inf, nothing beyond.
 * Accumulation is exact up to fp32 rounding: FP8 operands are widened exactly to f16 and
 * contracted on the f16 matrix cores with fp32 accumulation.
 * ------------------------------------------------------------------------------------------- */
dsa_status_t dsa_indexer_scores(const void* q, const float* w, const void* k_cache,
                                const float* k_scale, const int32_t* page_table, int64_t ld_pt,
                                int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                                int rows, int n_seq, int q_per_seq, int max_ctx, int Hi, int Di,
                                dsa_dtype_t dtype, float* scores, int64_t ld_scores, void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_topk -- S_t = TopK_{j <= t}(I_tj, k) ([DSA-blog] "Lightning Indexer", the TopK equation);
 * a row whose prefix holds fewer than k positions keeps all of them ([Handbook] cost model,
 * k = min(L, 2048)).
 *   scores [rows, ld_scores] f32 from dsa_indexer_scores; row r uses entries 0..q_pos[r]
 *   idx    [rows, ld_idx] int32 out, ld_idx >= k: the min(k, q_pos[r]+1) selected positions in
 *          ASCENDING order, then -1 up to slot k-1.
 * Ranking: larger score first; equal scores (by value: -0 == +0) rank the smaller position
 * first, so the result is unique. NaN scores are not supported (their rank is unspecified).
 * Workspace: rows longer than 16384 positions (max_ctx > 16384, k <= 4096, and
 * ceil(max_ctx / 16384) * k <= 16384) are selected in two stages (per-chunk candidates, then a
 * merge), which needs dsa_topk_workspace_size(rows, max_ctx, k) bytes at ws (device memory owned
 * by the caller, contents not preserved; 0 for shorter rows). With ws NULL or smaller, the
 * same result comes from a single-workgroup-per-row kernel (reported as DSA_PATH_TOPK_RADIX).
 * ------------------------------------------------------------------------------------------- */
size_t dsa_topk_workspace_size(int rows, int max_ctx, int k);
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                      int max_ctx, int k, int32_t* idx, int64_t ld_idx, void* ws,
                      size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_indexer_topk -- dsa_indexer_scores followed by dsa_topk in one call, with the top-k's first
 * radix pass done while the scores are produced ([DSA-blog] "Lightning Indexer": the index
 * scores exist only to feed TopK; [Handbook] "对推理引擎的新要求": the indexer and the top-k are
 * the new kernels the method asks of an engine). The scan counts, per row, its valid scores by
 * the first digit (the top 11 bits of the order key the top-k ranks by) in LDS, adds the counts
 * into a per-row histogram in the workspace, and the top-k starts from those counts instead of
 * its own first pass over the row.
 *   Arguments as dsa_indexer_scores (scores is still written in full: the caller may keep it)
 *   and dsa_topk (k, idx, ld_idx); the results equal those of the two calls bit for bit.
 *   ws  dsa_indexer_topk_workspace_size(rows, max_ctx, k) bytes of device memory, owned by the
 *       caller and reused across calls: it must be ZERO-FILLED before its first use, and every
 *       call that returns DSA_OK leaves its histogram part zero again (after a failed call,
 *       zero it again). Calls sharing one workspace must not overlap in time.
 * The shared counts are used for the MFMA scan shapes (Hi=64, Di=128, E4M3, 64-token pages) with
 * max_ctx <= 16384 and k <= 4096, or rows the two-stage top-k takes (counts per 16384-position
 * chunk; the chunk stage also counts the merge's candidates) (DSA_PATH_INDEXER_TOPK_FUSED). Other shapes run the two calls one after the other (the
 * path is then the top-k's).
 * ------------------------------------------------------------------------------------------- */
size_t dsa_indexer_topk_workspace_size(int rows, int max_ctx, int k);
dsa_status_t dsa_indexer_topk(const void* q, const float* w, const void* k_cache, const float* k_scale,
                              const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                              const int32_t* q_seq, const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                              int max_ctx, int Hi, int Di, dsa_dtype_t dtype, float* scores, int64_t ld_scores, int k,
                              int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_sparse_mla_decode / dsa_sparse_mla_prefill -- attention over the selected rows only
 * ([DSA-blog] "Sparse Attention": softmax(QK^T/sqrt(d_h) + M^DSA)V with M = 0 on S_t and -inf
 * elsewhere, computed by reading only the indexed rows; [Handbook] absorbed MLA: one latent row
 * of 512+64 bf16 per position is the key of all 128 heads, its first 512 columns the value).
 * For row r and head h, with S = the SET of positions that idx[r, 0..k-1] lists within
 * [0, q_pos[r]] (the -1 padding and any invisible position are skipped, and a position listed
 * several times is in S once: [DSA-blog] "Sparse Attention", M_tj = 0 exactly when j is in S_t):
 *     l_j    = sm_scale * q[r, h, 0:Dqk] . kv[j, 0:Dqk]
 *     out[r, h, :] = sum_{j in S} softmax(l)_j * kv[j, v_col0 : v_col0 + Dv]
 *     lse[r, h]    = log sum_{j in S} exp(l_j)         (natural log; -inf for an empty S)
 * An empty S gives out = 0.
 *   q        [rows, H, Dqk] bf16 bits, 16-byte aligned
 *   kv_cache [num_pages, page_size, kv_dim] bf16 bits, 16-byte aligned; kv_dim >= Dqk and
 *            kv_dim >= v_col0 + Dv (absorbed MLA: kv_dim = Dqk = 576, Dv = 512, v_col0 = 0)
 *   idx      [rows, ld_idx] int32, k entries per row (e.g. from dsa_topk)
 *   out      [rows, H, Dv] bf16 bits out (fp32 accumulation, one rounding)
 *   lse      [rows, H] f32 out, or NULL
 *   ws       device workspace of at least dsa_sparse_mla_workspace_size(...) bytes (may be
 *            NULL when that size is 0); its contents on entry do not matter
 * Softmax runs in fp32 with the probabilities rounded to bf16 for the value product.
 * List order: any. A row whose visible entries run strictly ascending from entry 0 (what
 * dsa_topk writes) cannot repeat a position and is attended directly; any other row is first
 * checked for repeats (a bitmap of the row's positions in LDS), which costs extra time.
 * Tuned shape: H=128, Dqk=576, Dv=512, kv_dim=576, v_col0=0 (bf16 MFMA). Other shapes with
 * Dqk <= 1024 and Dv <= 512 run a generic VALU kernel (reported by dsa_last_path()).
 * The decode entry point may split each row's index set over several workgroups and merge
 * their partial results, kept in the workspace as fp16 outputs normalised per split plus an
 * fp32 (max, sum) pair per head; the prefill entry point does one pass per row.
 * ------------------------------------------------------------------------------------------- */
size_t dsa_sparse_mla_workspace_size(int rows, int H, int Dv, int k);
dsa_status_t dsa_sparse_mla_decode(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                   int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                   const int32_t* q_pos, int rows, int n_seq, int q_per_seq, const int32_t* idx,
                                   int64_t ld_idx, int k, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                                   float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream);
dsa_status_t dsa_sparse_mla_prefill(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                    int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                    const int32_t* q_pos, int rows, int n_seq, int q_per_seq, const int32_t* idx,
                                    int64_t ld_idx, int k, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                                    float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_sparse_mla_decode_noalloc -- dsa_sparse_mla_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without ws / ws_bytes, the same kernels and the same results
 * bit for bit. Its split-merge workspace is a 65 MiB array the library holds on each device it
 * runs on (from the first call on that device until the process ends), which covers every shape
 * the decode entry point splits (at most 510 (row, split) units of 128 x 512 fp16 partials plus
 * their (max, sum) pairs); a call needing more returns DSA_ERR_WORKSPACE. It allocates nothing.
 * The stream must belong to the calling thread's current device. All calls on one device share
 * that array: calls that overlap in time on one device (different streams, or host threads)
 * race and give undefined results; calls ordered on one stream are safe.
 * ------------------------------------------------------------------------------------------- */
dsa_status_t dsa_sparse_mla_decode_noalloc(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                           int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                           const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                                           const int32_t* idx, int64_t ld_idx, int k, int H, int Dqk, int Dv,
                                           int kv_dim, int v_col0, float sm_scale, uint16_t* out, float* lse,
                                           void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_dense_mla_prefill -- dense causal attention: the computation above with S = {0..q_pos[r]}
 * ([DSA-blog] "SWA" section, the causal set C_t). It equals DSA exactly when q_pos[r] + 1 <= k
 * for every row ([Handbook]: short prefill falls back to dense). Arguments as above, without
 * idx; max_ctx (> every q_pos) sizes the key loop. Workspace: dsa_dense_mla_workspace_size.
 * ------------------------------------------------------------------------------------------- */
size_t dsa_dense_mla_workspace_size(int rows, int H, int Dv, int max_ctx);
dsa_status_t dsa_dense_mla_prefill(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                   int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                   const int32_t* q_pos, int rows, int n_seq, int q_per_seq, int max_ctx, int H,
                                   int Dqk, int Dv, int kv_dim, int v_col0, float sm_scale, uint16_t* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * dsa_expanded_mha_prefill -- expanded multi-head attention, the dense fallback for short prefill
 * ([Handbook] "稀疏注意力：NSA 与 DSA": the cost model's expanded pair, per head a query/key of
 * 128 + 64 (rope) dims and a 128-dim value, about 3.4x cheaper per (query, key) pair than the
 * absorbed form; short prefill runs it, and V3.2 emulates DSA in a masked MHA mode). With the
 * per-head up-projections of the latent row c_j applied beforehand (k_nope = c W_UK, v = c W_UV),
 * it computes the same attention as the absorbed MLA above, output projected by W_UV.
 * Rows take the uniform layout only (rows = n_seq * q_per_seq, no q_seq): a workgroup shares one
 * sequence's key and value tiles among up to 256 consecutive rows of that sequence.
 * For row r (sequence s = r / q_per_seq, position t = q_pos[r]) and head h:
 *     K_hj = [k_nope[s, h, j, :] | k_rope[s, j, :]]      (the rope key is shared by all heads)
 *     l_j  = sm_scale * q[r, h, :] . K_hj,   j in S
 *     out[r, h, :] = sum_{j in S} softmax(l)_j v[s, h, j, :];  lse[r, h] = log sum exp(l_j)
 * with S = {0..t} when idx is NULL (dense causal), else the positions in [0, t] that idx[r, 0..k-1]
 * lists ([DSA-blog] "Sparse Attention": M = 0 on S_t), as a set (the masked MHA mode: every
 * pair is computed, then masked). An empty S gives out = 0, lse = -inf.
 *   q      [rows, H, 192] bf16 bits (128 nope dims, then 64 rope dims), 16-byte aligned
 *   k_nope [n_seq, H, max_ctx, 128] bf16 bits (head-major per sequence), 16-byte aligned
 *   k_rope [n_seq, max_ctx, 64] bf16 bits, 16-byte aligned
 *   v      [n_seq, H, max_ctx, 128] bf16 bits, 16-byte aligned
 *   q_pos  [rows] int32, each in [0, max_ctx) (larger values see only the first max_ctx positions)
 *   idx    [rows, ld_idx] int32 or NULL; k entries per row
 *   out    [rows, H, 128] bf16 bits out (fp32 accumulation, one rounding); lse [rows, H] f32 or NULL
 *   ws     with idx: at least dsa_expanded_mha_workspace_size(rows, max_ctx, k) bytes, 4-byte
 *          aligned (one bit per (row, position), rebuilt by every call); else unused
 * Softmax in fp32 with the probabilities rounded to bf16 for the value product. Shapes other than
 * (128, 64, 128) or sm_scale <= 0 return DSA_ERR_UNSUPPORTED; max_ctx is limited to 524288.
 * ------------------------------------------------------------------------------------------- */
size_t dsa_expanded_mha_workspace_size(int rows, int max_ctx, int k);
dsa_status_t dsa_expanded_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope,
                                      const uint16_t* v, int max_ctx, const int32_t* q_pos, int n_seq,
                                      int q_per_seq, const int32_t* idx, int64_t ld_idx, int k, int H,
                                      int Dn, int Dr, int Dv, float sm_scale, uint16_t* out, float* lse,
                                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * The step before the indexer ([DSA-blog] "Lightning Indexer": every position's indexer key is
 * produced from its own hidden state and cached in an Indexer Key Cache of its own; [Handbook]
 * "对推理引擎的新要求": both caches are paged, and the cost model stores 128 + 4 bytes per token for
 * the indexer key, FP8 codes plus a float scale). The projections that produce k, q and w from
 * the hidden state are plain GEMMs the caller runs; these entry points quantise and place.
 *
 * dsa_indexer_cache_write -- for each of n_tok tokens (sequence seq[t] in [0, n_seq), position
 * pos[t]; device int32 arrays; page_table [n_seq, ld_pt]): s = max_c |k[t, c]| / 448 and codes E4M3(k[t, c] / s), both rounded as float
 * operations (round to nearest even, saturating to +-448; all codes 0 when s = 0), written to the
 * token's physical row of k_cache [num_pages, page_size, Di] (E4M3 bytes) and k_scale
 * [num_pages, page_size] (f32). This is the key format dsa_indexer_scores reads. A token whose
 * sequence is out of range or whose position has no valid page is not written.
 *   k  [n_tok, Di] f32 (dtype DSA_F32) or bf16 bits (DSA_BF16); Di = 128; k and k_cache 16-byte
 *   aligned.
 * dsa_latent_cache_write -- each token's latent row rows[t, 0:kv_dim] (bf16 bits) copied to its
 * physical row of kv_cache [num_pages, page_size, kv_dim]; kv_dim a multiple of 8; 16-byte aligned.
 * dsa_e4m3_quantize -- out[i] = E4M3(x[i]) for i < n (round to nearest even, saturating), the
 * indexer query's format (the pages give the query no scale).
 * Errors: DSA_ERR_INVALID_ARG for NULL or misaligned pointers and bad sizes, DSA_ERR_UNSUPPORTED
 * for Di != 128 or another dtype. Out-of-range seq / pos values are not checked on the host (they
 * are device data); such tokens are skipped by the kernels.
 * ------------------------------------------------------------------------------------------- */
dsa_status_t dsa_indexer_cache_write(const void* k, dsa_dtype_t dtype, int n_tok, int Di, const int32_t* seq,
                                     const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                                     int num_pages, uint8_t* k_cache, float* k_scale, void* stream);
dsa_status_t dsa_latent_cache_write(const uint16_t* rows, int n_tok, int kv_dim, const int32_t* seq,
                                    const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                                    int num_pages, uint16_t* kv_cache, void* stream);
dsa_status_t dsa_e4m3_quantize(const float* x, int64_t n, uint8_t* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * The indexer's projections ([DSA-blog] "Lightning Indexer", the first step of its figure: the
 * current token's hidden state h_t gives the head weights w_t; the query path takes the MLA query
 * latent and applies an indexer projection to get the n_h^I query heads; every position's hidden
 * state h_j gives the one key k_j all heads share, stored in the Indexer Key Cache), as bf16
 * matrix-core GEMMs with fp32 accumulation, their results quantised and placed in the same kernel.
 * Weights are in the [out, in] layout of a linear layer (each output's weights contiguous). The
 * pages give no normalisation, rotary part or extra scale in these projections, and none is applied.
 *
 * dsa_indexer_key_project -- k[t, :] = h[t, :] . w_k^T for n_tok tokens, then per token the key
 * format of dsa_indexer_cache_write (s = max_c |k| / 448, codes E4M3(k / s), float operations,
 * round to nearest even, saturating; all codes 0 when s = 0) written to the token's physical row
 * (sequence seq[t], position pos[t]) of k_cache / k_scale; tokens without a valid page are skipped.
 *   h   [n_tok, d] bf16 bits;  w_k [Di, d] bf16 bits;  Di = 128, d a multiple of 64.
 * dsa_indexer_query_project -- q8[r, :] = E4M3(c_q[r, :] . w_q^T) (Hi * Di codes, no scale: the
 * pages give the indexer query none) and w[r, :] = h[r, :] . w_w^T in fp32, for `rows` rows.
 *   c_q [rows, d_cq] bf16 bits (the MLA query latent); w_q [Hi * Di, d_cq]; h [rows, d];
 *   w_w [Hi, d]; q8 [rows, Hi, Di] bytes out; w [rows, Hi] f32 out. d_cq and d multiples of 64
 *   up to 65536 (both calls), Hi * Di a multiple of 16.
 * Workspace (both calls): with at least dsa_indexer_projection_workspace_size(rows, d) bytes at ws
 * (16-byte aligned, contents not preserved; rows = n_tok for the keys), a small batch whose output
 * tiles would leave most of the GPU idle splits K over workgroups (fp32 partial sums, then an
 * in-order reduction that applies the coding); with ws NULL or smaller the same results come from
 * one unsplit launch.
 * Errors as for the cache writes; other shapes return DSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------------------------- */
size_t dsa_indexer_projection_workspace_size(int rows, int d);
dsa_status_t dsa_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int Di,
                                     const int32_t* seq, const int32_t* pos, int n_seq, const int32_t* page_table,
                                     int64_t ld_pt, int page_size, int num_pages, uint8_t* k_cache, float* k_scale,
                                     void* ws, size_t ws_bytes, void* stream);
dsa_status_t dsa_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h,
                                       const uint16_t* w_w, int rows, int d_cq, int d, int Hi, int Di, uint8_t* q8,
                                       float* w, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
