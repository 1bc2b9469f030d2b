// dsa_abi.hip -- the extern "C" entry points of libdsa.so: host-side argument checks, kernel
// choice and launch. No allocation, no synchronisation: every call only enqueues on `stream`.
#include <limits.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "dsa_internal.h"

// Scratch memory of dsa_sparse_mla_decode_noalloc: the split-merge workspace of the decode
// attention, held by the library itself. A decode call splits rows * splits < 512 units (the
// split count doubles only while rows * splits < 256), each needing one fp16 partial row block and
// one (max, sum) block, so 510 units always fit. Every GPU the library runs on holds its own copy
// until the process ends.
constexpr size_t kNoallocScratchBytes = 65u << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

thread_local char g_err[512] = "";
thread_local int g_path = DSA_PATH_NONE;

dsa_status_t fail(dsa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

dsa_status_t ok(int path) {
  g_path = path;
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

#define REQUIRE(cond, ...) \
  do {                     \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

dsa_status_t check_paging(const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                          int max_ctx) {
  REQUIRE(page_table != nullptr, "page_table is NULL");
  REQUIRE(page_size >= 1, "page_size must be >= 1 (got %d)", page_size);
  REQUIRE(num_pages >= 1, "num_pages must be >= 1 (got %d)", num_pages);
  REQUIRE(max_ctx >= 1, "max_ctx must be >= 1 (got %d)", max_ctx);
  REQUIRE(ld_pt >= ((int64_t)max_ctx + page_size - 1) / page_size,
          "ld_pt (%lld) must cover max_ctx / page_size pages", (long long)ld_pt);
  REQUIRE((int64_t)num_pages * page_size < ((int64_t)1 << 31), "cache larger than 2^31 rows");
  return DSA_OK;
}

// The query-row descriptor of the indexer and attention calls: `rows` rows, either in groups of
// q_per_seq consecutive rows per sequence (q_seq NULL; rows == n_seq * q_per_seq), or row r of
// sequence q_seq[r] (device array; q_per_seq must then be 1).
dsa_status_t check_rows(const int32_t* q_seq, int rows, int n_seq, int q_per_seq, dsa::RowSeq* rs) {
  REQUIRE(rows >= 0 && n_seq >= 0 && q_per_seq >= 1, "need rows >= 0, n_seq >= 0 and q_per_seq >= 1 (got %d, %d, %d)",
          rows, n_seq, q_per_seq);
  if (q_seq)
    REQUIRE(q_per_seq == 1, "with per-row sequence ids (q_seq) q_per_seq must be 1 (got %d)", q_per_seq);
  else
    REQUIRE((int64_t)n_seq * q_per_seq == rows, "without q_seq, rows (%d) must equal n_seq * q_per_seq (%d * %d)",
            rows, n_seq, q_per_seq);
  REQUIRE(rows == 0 || n_seq >= 1, "%d rows but no sequence", rows);
  *rs = dsa::RowSeq{q_seq, q_per_seq, n_seq};
  return DSA_OK;
}

// The MFMA kernels take the absorbed-MLA shape with a positive softmax scale (they track the
// running maximum on the unscaled scores).
bool mla_tuned(int H, int Dqk, int Dv, int kv_dim, int v_col0, float sm_scale = 1.f) {
  return H == 128 && Dqk == 576 && Dv == 512 && kv_dim == 576 && v_col0 == 0 && sm_scale > 0.f;
}

dsa_status_t check_attn(const uint16_t* q, const uint16_t* kv_cache, const int32_t* q_seq, const int32_t* q_pos,
                        int rows, int n_seq, int q_per_seq, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                        uint16_t* out, dsa::RowSeq* rs) {
  dsa_status_t s = check_rows(q_seq, rows, n_seq, q_per_seq, rs);
  if (s != DSA_OK) return s;
  if (rows == 0) return DSA_OK;  // nothing to do; the caller returns before any launch
  REQUIRE(q && kv_cache && q_pos && out, "q, kv_cache, q_pos and out must be non-NULL");
  REQUIRE(H >= 1 && Dqk >= 1 && Dv >= 1, "H, Dqk and Dv must be >= 1");
  REQUIRE(kv_dim >= Dqk && v_col0 >= 0 && v_col0 + Dv <= kv_dim,
          "need Dqk <= kv_dim and v_col0 + Dv <= kv_dim");
  REQUIRE(!misaligned(q) && !misaligned(kv_cache) && !misaligned(out),
          "q, kv_cache and out must be 16-byte aligned");
  if (!mla_tuned(H, Dqk, Dv, kv_dim, v_col0) && (Dqk > 1024 || Dv > 512))
    return fail(DSA_ERR_UNSUPPORTED, "attention shape Dqk=%d Dv=%d not supported (Dqk<=1024, Dv<=512)", Dqk, Dv);
  return DSA_OK;
}

dsa_status_t run_sparse(bool decode, const uint16_t* q, const uint16_t* kv_cache,
                        const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                        const int32_t* q_seq, const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                        const int32_t* idx, int64_t ld_idx, int k, int H, int Dqk, int Dv, int kv_dim,
                        int v_col0, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                        void* stream) {
  dsa::RowSeq rs;
  dsa_status_t s = check_attn(q, kv_cache, q_seq, q_pos, rows, n_seq, q_per_seq, H, Dqk, Dv, kv_dim, v_col0, out, &rs);
  if (s != DSA_OK) return s;
  REQUIRE(k >= 1 && ld_idx >= k, "need k >= 1 and ld_idx >= k");
  if (rows == 0) return ok(DSA_PATH_NONE);
  REQUIRE(idx != nullptr, "idx is NULL");
  s = check_paging(page_table, ld_pt, page_size, num_pages, 1);
  if (s != DSA_OK) return s;
  dsa::AttnArgs a{q, {kv_cache, page_table, ld_pt, page_size, num_pages}, rs, q_pos, rows,
                  idx, ld_idx, k, H, Dqk, Dv, kv_dim, v_col0, sm_scale, out, lse};
  hipStream_t st = (hipStream_t)stream;
  if (!mla_tuned(H, Dqk, Dv, kv_dim, v_col0, sm_scale)) {
    s = hip_status(dsa::launch_mla_generic(a, st), "mla_generic launch");
    return s == DSA_OK ? ok(DSA_PATH_MLA_GENERIC) : s;
  }
  const int splits = decode ? dsa::mla_mfma_pick_splits(rows, k) : 1;
  const size_t need = dsa::mla_mfma_ws_bytes(rows, splits);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (need > 0 && misaligned(ws)) return fail(DSA_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  s = hip_status(dsa::launch_mla_mfma(a, splits, ws, st), "mla_mfma launch");
  return s == DSA_OK ? ok(splits > 1 ? DSA_PATH_MLA_MFMA_SPLIT : DSA_PATH_MLA_MFMA) : s;
}

// Device address of `scratch` on the calling thread's current device, looked up once per device
// with that device current (in host code the array's name is only a stand-in, never an address).
constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

dsa_status_t scratch_on_current_device(void** ptr) {
  int dev = -1;
  dsa_status_t s = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (s != DSA_OK) return s;
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess) return hip_status(slot.err, "hipGetSymbolAddress(scratch)");
  *ptr = slot.ptr;
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "unknown dsa_status_t";
}

const char* dsa_last_error(void) { return g_err; }
int dsa_last_path(void) { return g_path; }

dsa_status_t dsa_indexer_scores(const void* q, const float* w, const void* k_cache,
                                const float* k_scale, const int32_t* page_table, int64_t ld_pt,
                                int page_size, int num_pages, const int32_t* q_seq, const int32_t* q_pos,
                                int rows, int n_seq, int q_per_seq, int max_ctx, int Hi, int Di,
                                dsa_dtype_t dtype, float* scores, int64_t ld_scores, void* stream) {
  dsa::RowSeq rs;
  dsa_status_t s = check_rows(q_seq, rows, n_seq, q_per_seq, &rs);
  if (s != DSA_OK) return s;
  if (rows == 0) return ok(DSA_PATH_NONE);  // nothing to do; pointers may be NULL
  REQUIRE(q && w && k_cache && q_pos && scores, "q, w, k_cache, q_pos and scores must be non-NULL");
  REQUIRE(Hi >= 1 && Di >= 1, "Hi and Di must be >= 1");
  REQUIRE(dtype == DSA_E4M3 || dtype == DSA_F32, "dtype must be DSA_E4M3 or DSA_F32");
  REQUIRE(!misaligned(q) && !misaligned(k_cache), "q and k_cache must be 16-byte aligned");
  s = check_paging(page_table, ld_pt, page_size, num_pages, max_ctx);
  if (s != DSA_OK) return s;
  REQUIRE(ld_scores >= max_ctx, "ld_scores (%lld) must be >= max_ctx (%d)", (long long)ld_scores, max_ctx);
  dsa::PagedCache kc{k_cache, page_table, ld_pt, page_size, num_pages};
  hipStream_t st = (hipStream_t)stream;
  if (Hi == 64 && Di == 128 && dtype == DSA_E4M3) {
    // the scan is built for 64-token pages; it takes the rows of a sequence two at a time (one
    // at a time for an odd count or per-row sequence ids), one block row per unit
    const int64_t units = rows / dsa::indexer_scan_rows_per_wave(rs);
    if (page_size == 64 && units <= 65535) {
      s = hip_status(dsa::launch_indexer_scan((const uint8_t*)q, w, kc, k_scale, rs, q_pos, rows, max_ctx, scores,
                                              ld_scores, nullptr, st), "indexer_scan launch");
      return s == DSA_OK ? ok(DSA_PATH_INDEXER_SCAN_MFMA) : s;
    }
    s = hip_status(dsa::launch_indexer_prefill((const uint8_t*)q, w, kc, k_scale, rs, q_pos, rows, max_ctx, scores,
                                               ld_scores, st), "indexer_prefill launch");
    return s == DSA_OK ? ok(DSA_PATH_INDEXER_PREFILL_MFMA) : s;
  }
  s = hip_status(dsa::launch_indexer_generic(q, w, kc, k_scale, rs, q_pos, rows, max_ctx, Hi, Di, dtype == DSA_F32,
                                             scores, ld_scores, st), "indexer_generic launch");
  return s == DSA_OK ? ok(DSA_PATH_INDEXER_GENERIC) : s;
}

size_t dsa_topk_workspace_size(int rows, int max_ctx, int k) {
  if (rows <= 0 || max_ctx < 1 || k < 1) return 0;
  return dsa::topk_staged_ws_bytes(rows, max_ctx, k);
}

dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                      int max_ctx, int k, int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes,
                      void* stream) {
  REQUIRE(rows >= 0 && k >= 1 && max_ctx >= 1, "need rows >= 0, k >= 1, max_ctx >= 1");
  if (rows == 0) return ok(DSA_PATH_NONE);  // nothing to do; pointers may be NULL
  REQUIRE(scores && q_pos && idx, "scores, q_pos and idx must be non-NULL");
  REQUIRE(ld_scores >= max_ctx, "ld_scores (%lld) must be >= max_ctx (%d)", (long long)ld_scores, max_ctx);
  REQUIRE(ld_idx >= k, "ld_idx (%lld) must be >= k (%d)", (long long)ld_idx, k);
  if (rows == 0) return ok(DSA_PATH_NONE);
  int path = DSA_PATH_NONE;
  dsa_status_t s = hip_status(dsa::launch_topk(scores, ld_scores, q_pos, rows, max_ctx, k, idx, ld_idx, ws,
                                               ws_bytes, nullptr, (hipStream_t)stream, &path), "topk launch");
  return s == DSA_OK ? ok(path) : s;
}

size_t dsa_indexer_topk_workspace_size(int rows, int max_ctx, int k) {
  if (rows <= 0 || max_ctx < 1 || k < 1) return 0;
  // per-chunk counts, then (rows over one chunk) the merge's candidate counts, then the two-stage
  // top-k's own workspace
  const int C = dsa::topk_chunks(max_ctx);
  return 256 + (size_t)rows * (C + (C > 1 ? 1 : 0)) * dsa::kTopkDigit0Bins * 4 +
         dsa::topk_staged_ws_bytes(rows, max_ctx, k);
}

dsa_status_t dsa_indexer_topk(const void* q, const float* w, const void* k_cache, const float* k_scale,
                              const int32_t* page_table, int64_t ld_pt, int page_size, int num_pages,
                              const int32_t* q_seq, const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                              int max_ctx, int Hi, int Di, dsa_dtype_t dtype, float* scores, int64_t ld_scores, int k,
                              int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes, void* stream) {
  dsa::RowSeq rs;
  dsa_status_t s = check_rows(q_seq, rows, n_seq, q_per_seq, &rs);
  if (s != DSA_OK) return s;
  REQUIRE(k >= 1 && max_ctx >= 1, "need k >= 1 and max_ctx >= 1");
  if (rows == 0) return ok(DSA_PATH_NONE);  // nothing to do; pointers may be NULL
  REQUIRE(idx && ld_idx >= k, "idx must be non-NULL with ld_idx >= k");
  const size_t need = dsa_indexer_topk_workspace_size(rows, max_ctx, k);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws ? ws_bytes : (size_t)0);
  uint32_t* hist0 = (uint32_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  const int nchunks = dsa::topk_chunks(max_ctx);
  uint8_t* topk_ws = (uint8_t*)(hist0 + (size_t)rows * (nchunks + (nchunks > 1 ? 1 : 0)) * dsa::kTopkDigit0Bins);
  const size_t topk_ws_bytes = (size_t)((uint8_t*)ws + ws_bytes - topk_ws);
  const bool fused = Hi == 64 && Di == 128 && dtype == DSA_E4M3 && page_size == 64 &&
                     (int64_t)rows / dsa::indexer_scan_rows_per_wave(rs) <= 65535 &&
                     (max_ctx <= dsa::topk_reg_max_ctx() ? k <= dsa::topk_reg_max_k()
                                                        : dsa::topk_staged_ok(max_ctx, k));
  if (!fused) {
    // the same two steps without the shared histogram
    s = dsa_indexer_scores(q, w, k_cache, k_scale, page_table, ld_pt, page_size, num_pages, q_seq, q_pos, rows, n_seq,
                           q_per_seq, max_ctx, Hi, Di, dtype, scores, ld_scores, stream);
    if (s != DSA_OK) return s;
    return dsa_topk(scores, ld_scores, q_pos, rows, max_ctx, k, idx, ld_idx, topk_ws, topk_ws_bytes, stream);
  }
  REQUIRE(q && w && k_cache && q_pos && scores, "q, w, k_cache, q_pos and scores must be non-NULL");
  REQUIRE(!misaligned(q) && !misaligned(k_cache), "q and k_cache must be 16-byte aligned");
  s = check_paging(page_table, ld_pt, page_size, num_pages, max_ctx);
  if (s != DSA_OK) return s;
  REQUIRE(ld_scores >= max_ctx, "ld_scores (%lld) must be >= max_ctx (%d)", (long long)ld_scores, max_ctx);
  dsa::PagedCache kc{k_cache, page_table, ld_pt, page_size, num_pages};
  hipStream_t st = (hipStream_t)stream;
  s = hip_status(dsa::launch_indexer_scan((const uint8_t*)q, w, kc, k_scale, rs, q_pos, rows, max_ctx, scores,
                                          ld_scores, hist0, st), "indexer_scan launch");
  if (s != DSA_OK) return s;
  int path = DSA_PATH_NONE;
  s = hip_status(dsa::launch_topk(scores, ld_scores, q_pos, rows, max_ctx, k, idx, ld_idx, topk_ws, topk_ws_bytes,
                                  hist0, st, &path), "topk launch");
  return s == DSA_OK ? ok(DSA_PATH_INDEXER_TOPK_FUSED) : s;
}

size_t dsa_sparse_mla_workspace_size(int rows, int H, int Dv, int k) {
  if (rows <= 0 || H != 128 || Dv != 512 || k < 1) return 0;
  return dsa::mla_mfma_ws_bytes(rows, dsa::mla_mfma_pick_splits(rows, k));
}

dsa_status_t dsa_sparse_mla_decode(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                   int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                   const int32_t* q_pos, int rows, int n_seq, int q_per_seq, const int32_t* idx,
                                   int64_t ld_idx, int k, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                                   float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  return run_sparse(true, q, kv_cache, page_table, ld_pt, page_size, num_pages, q_seq, q_pos, rows, n_seq, q_per_seq,
                    idx, ld_idx, k, H, Dqk, Dv, kv_dim, v_col0, sm_scale, out, lse, ws, ws_bytes, stream);
}

dsa_status_t dsa_sparse_mla_decode_noalloc(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                           int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                           const int32_t* q_pos, int rows, int n_seq, int q_per_seq,
                                           const int32_t* idx, int64_t ld_idx, int k, int H, int Dqk, int Dv,
                                           int kv_dim, int v_col0, float sm_scale, uint16_t* out, float* lse,
                                           void* stream) {
  const size_t need = dsa_sparse_mla_workspace_size(rows, H, Dv, k);
  if (need > kNoallocScratchBytes)
    return fail(DSA_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu",
                need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    dsa_status_t s = scratch_on_current_device(&ws);
    if (s != DSA_OK) return s;
  }
  return run_sparse(true, q, kv_cache, page_table, ld_pt, page_size, num_pages, q_seq, q_pos, rows, n_seq, q_per_seq,
                    idx, ld_idx, k, H, Dqk, Dv, kv_dim, v_col0, sm_scale, out, lse, ws,
                    need > 0 ? kNoallocScratchBytes : 0, stream);
}

dsa_status_t dsa_sparse_mla_prefill(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                    int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                    const int32_t* q_pos, int rows, int n_seq, int q_per_seq, const int32_t* idx,
                                    int64_t ld_idx, int k, int H, int Dqk, int Dv, int kv_dim, int v_col0,
                                    float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                                    void* stream) {
  return run_sparse(false, q, kv_cache, page_table, ld_pt, page_size, num_pages, q_seq, q_pos, rows, n_seq, q_per_seq,
                    idx, ld_idx, k, H, Dqk, Dv, kv_dim, v_col0, sm_scale, out, lse, ws, ws_bytes, stream);
}

size_t dsa_dense_mla_workspace_size(int rows, int H, int Dv, int max_ctx) {
  (void)rows; (void)H; (void)Dv; (void)max_ctx;
  return 0;
}

dsa_status_t dsa_dense_mla_prefill(const uint16_t* q, const uint16_t* kv_cache, const int32_t* page_table,
                                   int64_t ld_pt, int page_size, int num_pages, const int32_t* q_seq,
                                   const int32_t* q_pos, int rows, int n_seq, int q_per_seq, int max_ctx, int H,
                                   int Dqk, int Dv, int kv_dim, int v_col0, float sm_scale, uint16_t* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  (void)ws; (void)ws_bytes;
  dsa::RowSeq rs;
  dsa_status_t s = check_attn(q, kv_cache, q_seq, q_pos, rows, n_seq, q_per_seq, H, Dqk, Dv, kv_dim, v_col0, out, &rs);
  if (s != DSA_OK) return s;
  if (rows == 0) return ok(DSA_PATH_NONE);
  s = check_paging(page_table, ld_pt, page_size, num_pages, max_ctx);
  if (s != DSA_OK) return s;
  dsa::AttnArgs a{q, {kv_cache, page_table, ld_pt, page_size, num_pages}, rs, q_pos, rows,
                  nullptr, 0, max_ctx, H, Dqk, Dv, kv_dim, v_col0, sm_scale, out, lse};
  hipStream_t st = (hipStream_t)stream;
  if (!mla_tuned(H, Dqk, Dv, kv_dim, v_col0, sm_scale)) {
    s = hip_status(dsa::launch_mla_generic(a, st), "mla_generic launch");
    return s == DSA_OK ? ok(DSA_PATH_MLA_GENERIC) : s;
  }
  s = hip_status(dsa::launch_mla_mfma(a, 1, nullptr, st), "mla_mfma launch");
  return s == DSA_OK ? ok(DSA_PATH_MLA_MFMA) : s;
}

size_t dsa_expanded_mha_workspace_size(int rows, int max_ctx, int k) {
  return k > 0 ? dsa::mha_ws_bytes(rows, max_ctx, true) : 0;
}

dsa_status_t dsa_expanded_mha_prefill(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope,
                                      const uint16_t* v, int max_ctx, const int32_t* q_pos, int n_seq,
                                      int q_per_seq, const int32_t* idx, int64_t ld_idx, int k, int H, int Dn,
                                      int Dr, int Dv, float sm_scale, uint16_t* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream) {
  REQUIRE(n_seq >= 0 && q_per_seq >= 1, "need n_seq >= 0 and q_per_seq >= 1");
  if (n_seq == 0) return ok(DSA_PATH_NONE);
  REQUIRE(H >= 1, "H must be >= 1 (got %d)", H);
  REQUIRE(max_ctx >= 1 && max_ctx <= (1 << 19), "max_ctx must be in [1, 524288] (got %d)", max_ctx);
  REQUIRE((int64_t)n_seq * q_per_seq < ((int64_t)1 << 31), "too many rows");
  REQUIRE(q && k_nope && k_rope && v && q_pos && out, "a required pointer is NULL");
  REQUIRE(!misaligned(q) && !misaligned(k_nope) && !misaligned(k_rope) && !misaligned(v) && !misaligned(out),
          "q, k_nope, k_rope, v and out must be 16-byte aligned");
  if (Dn != 128 || Dr != 64 || Dv != 128 || !(sm_scale > 0.f))
    return fail(DSA_ERR_UNSUPPORTED, "expanded attention runs Dn=128, Dr=64, Dv=128 with sm_scale > 0 "
                                     "(got %d, %d, %d, %g)", Dn, Dr, Dv, (double)sm_scale);
  const int rows = n_seq * q_per_seq;
  if (idx) {
    REQUIRE(k >= 1 && ld_idx >= k, "need k >= 1 and ld_idx >= k with an index set (got %d, %lld)", k,
            (long long)ld_idx);
    const size_t need = dsa::mha_ws_bytes(rows, max_ctx, true);
    if (!ws || ws_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    REQUIRE(((uintptr_t)ws & 3u) == 0, "ws must be 4-byte aligned");
  }
  dsa_status_t s = hip_status(dsa::launch_mha(q, k_nope, k_rope, v, max_ctx, q_pos, n_seq, q_per_seq, idx, ld_idx, k,
                                              H, max_ctx, sm_scale, out, lse, ws, (hipStream_t)stream),
                              "mha launch");
  return s == DSA_OK ? ok(idx ? DSA_PATH_MHA_MFMA_MASKED : DSA_PATH_MHA_MFMA) : s;
}

dsa_status_t dsa_indexer_cache_write(const void* k, dsa_dtype_t dtype, int n_tok, int Di, const int32_t* seq,
                                     const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                                     int num_pages, uint8_t* k_cache, float* k_scale, void* stream) {
  REQUIRE(n_tok >= 0, "n_tok must be >= 0 (got %d)", n_tok);
  if (n_tok == 0) return ok(DSA_PATH_NONE);
  REQUIRE(k && seq && pos && page_table && k_cache && k_scale, "a required pointer is NULL");
  REQUIRE(!misaligned(k) && !misaligned(k_cache) && ((uintptr_t)k_scale & 3u) == 0,
          "k and k_cache must be 16-byte aligned, k_scale 4-byte aligned");
  REQUIRE(n_seq >= 1, "n_seq must be >= 1 (got %d)", n_seq);
  REQUIRE(page_size >= 1 && num_pages >= 1 && ld_pt >= 1, "bad paging (page_size %d, num_pages %d, ld_pt %lld)",
          page_size, num_pages, (long long)ld_pt);
  REQUIRE((int64_t)num_pages * page_size < ((int64_t)1 << 31), "cache larger than 2^31 rows");
  if (Di != 128 || (dtype != DSA_F32 && dtype != DSA_BF16))
    return fail(DSA_ERR_UNSUPPORTED, "the indexer cache write takes Di = 128 keys in f32 or bf16 (got Di %d, dtype %d)",
                Di, (int)dtype);
  dsa::PagedCache kc{k_cache, page_table, ld_pt, page_size, num_pages};
  dsa_status_t s = hip_status(dsa::launch_indexer_cache_write(k, dtype == DSA_F32, n_tok, n_seq, seq, pos, kc, k_cache, k_scale,
                                                               (hipStream_t)stream),
                              "indexer cache write launch");
  return s == DSA_OK ? ok(DSA_PATH_CACHE_WRITE) : s;
}

dsa_status_t dsa_latent_cache_write(const uint16_t* rows, int n_tok, int kv_dim, const int32_t* seq,
                                    const int32_t* pos, int n_seq, const int32_t* page_table, int64_t ld_pt, int page_size,
                                    int num_pages, uint16_t* kv_cache, void* stream) {
  REQUIRE(n_tok >= 0, "n_tok must be >= 0 (got %d)", n_tok);
  if (n_tok == 0) return ok(DSA_PATH_NONE);
  REQUIRE(rows && seq && pos && page_table && kv_cache, "a required pointer is NULL");
  REQUIRE(!misaligned(rows) && !misaligned(kv_cache), "rows and kv_cache must be 16-byte aligned");
  REQUIRE(kv_dim >= 8 && kv_dim % 8 == 0, "kv_dim must be a positive multiple of 8 (got %d)", kv_dim);
  REQUIRE(n_seq >= 1, "n_seq must be >= 1 (got %d)", n_seq);
  REQUIRE(page_size >= 1 && num_pages >= 1 && ld_pt >= 1, "bad paging (page_size %d, num_pages %d, ld_pt %lld)",
          page_size, num_pages, (long long)ld_pt);
  REQUIRE((int64_t)num_pages * page_size < ((int64_t)1 << 31), "cache larger than 2^31 rows");
  dsa::PagedCache kc{kv_cache, page_table, ld_pt, page_size, num_pages};
  dsa_status_t s = hip_status(dsa::launch_latent_cache_write(rows, n_tok, n_seq, kv_dim, seq, pos, kc, kv_cache,
                                                              (hipStream_t)stream),
                              "latent cache write launch");
  return s == DSA_OK ? ok(DSA_PATH_CACHE_WRITE) : s;
}

// The projections' widest K: a 256-row tile's per-lane byte offsets (row x 2K) stay in 32 bits.
constexpr int kProjMaxK = 65536;

size_t dsa_indexer_projection_workspace_size(int rows, int d) {
  if (rows <= 0 || d < 64) return 0;
  const size_t k = dsa::proj_ws_bytes(rows, 128, d), w = dsa::proj_ws_bytes(rows, 64, d);
  return k > w ? k : w;
}

dsa_status_t dsa_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int Di,
                                     const int32_t* seq, const int32_t* pos, int n_seq, const int32_t* page_table,
                                     int64_t ld_pt, int page_size, int num_pages, uint8_t* k_cache, float* k_scale,
                                     void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(n_tok >= 0 && d >= 1, "need n_tok >= 0 and d >= 1 (got %d, %d)", n_tok, d);
  if (n_tok == 0) return ok(DSA_PATH_NONE);
  REQUIRE(h && w_k && seq && pos && page_table && k_cache && k_scale, "a required pointer is NULL");
  REQUIRE(!misaligned(h) && !misaligned(w_k) && !misaligned(k_cache) && ((uintptr_t)k_scale & 3u) == 0,
          "h, w_k and k_cache must be 16-byte aligned, k_scale 4-byte aligned");
  REQUIRE(n_seq >= 1, "n_seq must be >= 1 (got %d)", n_seq);
  REQUIRE(page_size >= 1 && num_pages >= 1 && ld_pt >= 1, "bad paging (page_size %d, num_pages %d, ld_pt %lld)",
          page_size, num_pages, (long long)ld_pt);
  REQUIRE((int64_t)num_pages * page_size < ((int64_t)1 << 31), "cache larger than 2^31 rows");
  if (Di != 128 || d % 64 != 0 || d > kProjMaxK)
    return fail(DSA_ERR_UNSUPPORTED, "the key projection takes Di = 128 and d a multiple of 64 up to %d (got Di %d, d %d)",
                kProjMaxK, Di, d);
  dsa::PagedCache kc{k_cache, page_table, ld_pt, page_size, num_pages};
  REQUIRE(!ws || ((uintptr_t)ws & 15u) == 0, "ws must be 16-byte aligned");
  dsa_status_t s = hip_status(dsa::launch_indexer_key_project(h, w_k, n_tok, d, n_seq, seq, pos, kc, k_cache, k_scale,
                                                               ws, ws_bytes, (hipStream_t)stream),
                              "key projection launch");
  return s == DSA_OK ? ok(DSA_PATH_PROJECT) : s;
}

dsa_status_t dsa_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h,
                                       const uint16_t* w_w, int rows, int d_cq, int d, int Hi, int Di, uint8_t* q8,
                                       float* w, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(rows >= 0 && d_cq >= 1 && d >= 1 && Hi >= 1 && Di >= 1, "need rows >= 0 and positive dims");
  if (rows == 0) return ok(DSA_PATH_NONE);
  REQUIRE(c_q && w_q && h && w_w && q8 && w, "a required pointer is NULL");
  REQUIRE(!misaligned(c_q) && !misaligned(w_q) && !misaligned(h) && !misaligned(w_w) && !misaligned(q8) &&
              ((uintptr_t)w & 3u) == 0,
          "c_q, w_q, h, w_w and q8 must be 16-byte aligned, w 4-byte aligned");
  REQUIRE((int64_t)Hi * Di < (1 << 30), "Hi * Di too large");
  if (d_cq % 64 != 0 || d % 64 != 0 || d_cq > kProjMaxK || d > kProjMaxK || (Hi * Di) % 16 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "the query projection takes d_cq and d multiples of 64 up to %d and Hi * Di a "
                                     "multiple of 16 (got %d, %d, %d)", kProjMaxK, d_cq, d, Hi * Di);
  REQUIRE(!ws || ((uintptr_t)ws & 15u) == 0, "ws must be 16-byte aligned");
  dsa_status_t s = hip_status(dsa::launch_indexer_query_project(c_q, w_q, h, w_w, rows, d_cq, d, Hi * Di, Hi, q8, w,
                                                                 ws, ws_bytes, (hipStream_t)stream),
                              "query projection launch");
  return s == DSA_OK ? ok(DSA_PATH_PROJECT) : s;
}

dsa_status_t dsa_e4m3_quantize(const float* x, int64_t n, uint8_t* out, void* stream) {
  REQUIRE(n >= 0, "n must be >= 0");
  if (n == 0) return ok(DSA_PATH_NONE);
  REQUIRE(x && out, "a required pointer is NULL");
  REQUIRE(!misaligned(x) && ((uintptr_t)out & 3u) == 0, "x must be 16-byte and out 4-byte aligned");
  REQUIRE(n < ((int64_t)1 << 40), "n too large");
  dsa_status_t s = hip_status(dsa::launch_e4m3_quantize(x, n, out, (hipStream_t)stream), "e4m3 quantize launch");
  return s == DSA_OK ? ok(DSA_PATH_QUANTIZE) : s;
}

}  // extern "C"
