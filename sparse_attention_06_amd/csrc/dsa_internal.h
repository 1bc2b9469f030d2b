// dsa_internal.h -- device helpers and kernel launchers shared by the gfx950 kernels of libdsa.
// Internal to the library; the public interface is include/dsa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// ---------------------------------------------------------------- vector types
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- numeric helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even float -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two OCP E4M3 bytes (the low or high 16-bit half of `word`) -> two f16, exact (hardware convert).
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t word, bool high) {
  return high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)word, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)word, 1.0f, false);
}

// 16 E4M3 bytes (4 dwords) -> 16 f16 (two MFMA operands of 8).
__device__ __forceinline__ void e4m3x16_to_f16(i32x4 raw, f16x8& lo, f16x8& hi) {
  f16x2 a = e4m3x2_to_f16((uint32_t)raw[0], false), b = e4m3x2_to_f16((uint32_t)raw[0], true);
  f16x2 c = e4m3x2_to_f16((uint32_t)raw[1], false), d = e4m3x2_to_f16((uint32_t)raw[1], true);
  f16x2 e = e4m3x2_to_f16((uint32_t)raw[2], false), f = e4m3x2_to_f16((uint32_t)raw[2], true);
  f16x2 g = e4m3x2_to_f16((uint32_t)raw[3], false), h = e4m3x2_to_f16((uint32_t)raw[3], true);
  lo = f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  hi = f16x8{e[0], e[1], f[0], f[1], g[0], g[1], h[0], h[1]};
}

// float -> OCP E4M3FN, round to nearest even, saturating to +-448 (finite input). Normal values:
// round the 23-bit mantissa to 3 bits by adding half an output ulp minus one plus the kept LSB
// (a carry moves into the exponent); below 2^-6 the value is a count of 2^-9 quanta.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |f| >= 448
  if (a < 0x3C800000u) {                      // |f| < 2^-6: subnormal codes 0..8 (8 = 2^-6)
    const float q = __uint_as_float(a) * 512.0f;  // exact
    return sign | (uint32_t)__builtin_rintf(q);
  }
  const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t e = (r >> 23) - 127u + 7u;  // 1 .. 15
  const uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Which sequence (page-table row) a query row belongs to: with q_seq NULL the rows come in
// groups of q_per_seq consecutive rows per sequence, otherwise row r belongs to sequence q_seq[r].
// A sequence id outside [0, n_seq) has no page-table row: -1, whose positions resolve to no
// physical row.
struct RowSeq {
  const int32_t* q_seq;
  int q_per_seq, n_seq;
  __device__ __forceinline__ int of(int r) const {
    const int s = q_seq ? q_seq[r] : r / q_per_seq;
    return (s >= 0 && s < n_seq) ? s : -1;
  }
};

// Physical row of position p of sequence s, or -1 if s is -1, p lies outside the page table's
// [0, ld_pt * page_size) or the page id outside [0, num_pages).
__device__ __forceinline__ int64_t phys_row(const int32_t* __restrict__ page_table, int64_t ld_pt,
                                            int page_size, int num_pages, int s, int p) {
  if (s < 0 || p < 0 || p / page_size >= ld_pt) return -1;
  int32_t page = page_table[(int64_t)s * ld_pt + p / page_size];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_size + p % page_size;
}

// ---------------------------------------------------------------- launchers (one per kernel family)
// Order-preserving 32-bit key of a score: larger score -> larger key; -0 ranks with +0. The
// top-k's radix digits are taken from these keys (its first digit is bits 31..21).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr int kTopkDigit0Bins = 2048;  // first radix digit: key bits 31..21
constexpr int kTopkChunkKeys = 16384;  // positions per top-k chunk (a row's first-digit counts are per chunk)

struct PagedCache {
  const void* base;
  const int32_t* page_table;
  int64_t ld_pt;
  int page_size;
  int num_pages;
};

hipError_t launch_indexer_generic(const void* q, const float* w, PagedCache kc, const float* k_scale,
                                  RowSeq rs, const int32_t* q_pos, int rows, int max_ctx, int Hi,
                                  int Di, int is_f32, float* scores, int64_t ld_scores,
                                  hipStream_t stream);
// query rows per scan unit: 2 when the uniform layout pairs rows of one sequence, else 1
int indexer_scan_rows_per_wave(RowSeq rs);
// hist0 (optional, zero on entry): per row and kTopkChunkKeys-position chunk (row-major), a
// kTopkDigit0Bins-bin count of the scores at positions 0..q_pos[r] by their key's first digit,
// added with device-scope atomics
hipError_t launch_indexer_scan(const uint8_t* q, const float* w, PagedCache kc, const float* k_scale,
                               RowSeq rs, const int32_t* q_pos, int rows, int max_ctx,
                               float* scores, int64_t ld_scores, uint32_t* hist0, hipStream_t stream);
hipError_t launch_indexer_prefill(const uint8_t* q, const float* w, PagedCache kc,
                                  const float* k_scale, RowSeq rs, const int32_t* q_pos, int rows,
                                  int max_ctx, float* scores, int64_t ld_scores, hipStream_t stream);

// hist0 (optional; rows of at most topk_reg_max_ctx() positions with k <= topk_reg_max_k(), or
// the two-stage path): per row and chunk, the first-digit histogram of the valid scores, as
// launch_indexer_scan counts it; read in place of the first radix pass and left zeroed
hipError_t launch_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                       int max_ctx, int k, int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes,
                       uint32_t* hist0, hipStream_t stream, int* path);
int topk_reg_max_ctx();
int topk_reg_max_k();
int topk_chunks(int max_ctx);
bool topk_staged_ok(int max_ctx, int k);
size_t topk_staged_ws_bytes(int rows, int max_ctx, int k);

struct AttnArgs {
  const uint16_t* q;
  PagedCache kv;
  RowSeq rs;
  const int32_t* q_pos;
  int rows;
  const int32_t* idx;  // NULL => dense causal set {0..q_pos}
  int64_t ld_idx;
  int k;               // entries per idx row (dense: max_ctx)
  int H, Dqk, Dv, kv_dim, v_col0;
  float sm_scale;
  uint16_t* out;
  float* lse;
};

hipError_t launch_mla_generic(const AttnArgs& a, hipStream_t stream);
// splits: number of workgroups sharing one row's set (1 = single pass). ws: splits > 1 partials.
hipError_t launch_mla_mfma(const AttnArgs& a, int splits, void* ws, hipStream_t stream);
size_t mla_mfma_ws_bytes(int rows, int splits);
int mla_mfma_pick_splits(int rows, int k);

// Expanded multi-head attention (Dn=128, Dr=64, Dv=128). idx NULL: dense causal; else the index
// sets as a bitmap in ws (mha_ws_bytes).
size_t mha_ws_bytes(int rows, int max_ctx, bool has_idx);
hipError_t launch_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
                      int64_t ld_kv, const int32_t* q_pos, int n_seq, int q_per_seq, const int32_t* idx,
                      int64_t ld_idx, int k, int H, int max_ctx, float sm_scale, uint16_t* out, float* lse,
                      void* ws, hipStream_t stream);
// The step before the indexer: per-token FP8 key quantisation and the paged cache writes.
hipError_t launch_indexer_cache_write(const void* k, bool f32, int n_tok, int n_seq, const int32_t* seq,
                                      const int32_t* pos, PagedCache kc, uint8_t* k_cache, float* k_scale,
                                      hipStream_t stream);
hipError_t launch_latent_cache_write(const uint16_t* rows, int n_tok, int n_seq, int kv_dim, const int32_t* seq,
                                     const int32_t* pos, PagedCache kc, uint16_t* kv_cache, hipStream_t stream);
hipError_t launch_e4m3_quantize(const float* x, int64_t n, uint8_t* out, hipStream_t stream);
// The indexer's projections (bf16 MFMA GEMMs, operands K-contiguous, K a multiple of 64): keys
// k = h w_k^T quantised per token into the paged cache (128 output columns); queries q = c_q w_q^T
// as unscaled E4M3 codes (n_q columns, a multiple of 16) and head weights w = h w_w^T in fp32.
// Small batches split K over workgroups when a workspace of proj_ws_bytes(M, N, K) is given (fp32
// partial sums, then an in-order reduction with the epilogue); without one they run unsplit.
size_t proj_ws_bytes(int M, int N, int K);
hipError_t launch_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int n_seq,
                                      const int32_t* seq, const int32_t* pos, PagedCache kc, uint8_t* k_cache,
                                      float* k_scale, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h,
                                        const uint16_t* w_w, int rows, int d_cq, int d, int n_q, int n_w, uint8_t* q8,
                                        float* w, void* ws, size_t ws_bytes, hipStream_t stream);
}  // namespace dsa
