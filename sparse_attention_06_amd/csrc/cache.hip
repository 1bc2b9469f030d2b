// cache.hip -- the step before the indexer on gfx950: FP8 quantisation of the indexer keys with a
// per-token scale and their paged cache write, the latent cache write, and the indexer query's
// FP8 quantisation.
//
// Page references:
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org), section
//               "Lightning Indexer": each position's indexer key is produced from its own hidden
//               state and kept in a separate Indexer Key Cache shared by all indexer heads
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io), section "对推理引擎的新要求": two
//               paged caches (latent rows and indexer keys); the cost model's IDX_BYTES = 128 + 4
//               (FP8 codes plus a float scale per token)
//
// All three are plain HBM streams (bytes in, bytes out, one pass) with contiguous, coalesced
// loads and stores.
#include "dsa_internal.h"

namespace dsa {

// Sixteen lanes per token (four tokens per wave), Di = 128: lane j of a token's group holds
// elements 8j .. 8j+7. The key row is loaded first, so its latency overlaps the page lookup.
template <bool kF32>
__global__ void __launch_bounds__(256) indexer_cache_write_kernel(const void* __restrict__ k, int n_tok, int n_seq,
                                                                  const int32_t* __restrict__ seq,
                                                                  const int32_t* __restrict__ pos, PagedCache kc,
                                                                  uint8_t* __restrict__ k_cache,
                                                                  float* __restrict__ k_scale) {
  const int j = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = t < n_tok;
  const int tc = live ? t : n_tok - 1;  // idle groups reload the last token and store nothing
  float x[8];
  if (kF32) {
    const float4* src = (const float4*)k + (int64_t)tc * 32 + 2 * j;
    const float4 a = src[0], b = src[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const i32x4 v = ((const i32x4*)k)[(int64_t)tc * 16 + j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_to_f32((uint16_t)((uint32_t)v[e] & 0xFFFFu));
      x[2 * e + 1] = bf16_to_f32((uint16_t)((uint32_t)v[e] >> 16));
    }
  }
  const int sq = seq[tc];
  const int64_t row = live && sq >= 0 && sq < n_seq
                          ? phys_row(kc.page_table, kc.ld_pt, kc.page_size, kc.num_pages, sq, pos[tc]) : -1;
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));  // within the 16-lane group
  if (row < 0) return;  // past the end, or no valid (sequence, page): the token is not written
  const float s = m / 448.0f;
  uint32_t lo = 0, hi = 0;
  if (s > 0.f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= e4m3_rne_sat(x[e] / s) << (8 * e);
      hi |= e4m3_rne_sat(x[4 + e] / s) << (8 * e);
    }
  }
  ((uint2*)(k_cache + row * 128))[j] = make_uint2(lo, hi);
  if (j == 0) k_scale[row] = s;
}

// One 16-byte chunk per thread over all (token, chunk) pairs, so every lane of every wave moves
// data; the page lookup of a token is repeated by its chunks' threads (cached).
__global__ void __launch_bounds__(256) latent_cache_write_kernel(const uint16_t* __restrict__ rows, int n_tok,
                                                                 int n_seq, int chunks, const int32_t* __restrict__ seq,
                                                                 const int32_t* __restrict__ pos, PagedCache kc,
                                                                 uint16_t* __restrict__ kv_cache) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_tok * chunks) return;
  const int t = (int)(i / chunks), c = (int)(i % chunks);
  const i32x4 v = ((const i32x4*)rows)[i];
  const int sq = seq[t];
  const int64_t row = sq >= 0 && sq < n_seq ? phys_row(kc.page_table, kc.ld_pt, kc.page_size, kc.num_pages, sq, pos[t]) : -1;
  if (row < 0) return;
  ((i32x4*)kv_cache)[row * chunks + c] = v;
}

// Elementwise, four values per thread.
__global__ void __launch_bounds__(256) e4m3_quantize_kernel(const float* __restrict__ x, int64_t n,
                                                            uint8_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *(const float4*)(x + i);
    *(uint32_t*)(out + i) = e4m3_rne_sat(v.x) | (e4m3_rne_sat(v.y) << 8) | (e4m3_rne_sat(v.z) << 16) |
                            (e4m3_rne_sat(v.w) << 24);
  } else {
    for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)e4m3_rne_sat(x[j]);
  }
}

hipError_t launch_indexer_cache_write(const void* k, bool f32, int n_tok, int n_seq, const int32_t* seq,
                                      const int32_t* pos, PagedCache kc, uint8_t* k_cache, float* k_scale,
                                      hipStream_t stream) {
  const dim3 grid((n_tok + 15) / 16);
  if (f32)
    hipLaunchKernelGGL(indexer_cache_write_kernel<true>, grid, dim3(256), 0, stream, k, n_tok, n_seq, seq, pos, kc,
                       k_cache, k_scale);
  else
    hipLaunchKernelGGL(indexer_cache_write_kernel<false>, grid, dim3(256), 0, stream, k, n_tok, n_seq, seq, pos, kc,
                       k_cache, k_scale);
  return hipGetLastError();
}

hipError_t launch_latent_cache_write(const uint16_t* rows, int n_tok, int n_seq, int kv_dim, const int32_t* seq,
                                     const int32_t* pos, PagedCache kc, uint16_t* kv_cache, hipStream_t stream) {
  const int64_t threads = (int64_t)n_tok * (kv_dim / 8);
  hipLaunchKernelGGL(latent_cache_write_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, rows,
                     n_tok, n_seq, kv_dim / 8, seq, pos, kc, kv_cache);
  return hipGetLastError();
}

hipError_t launch_e4m3_quantize(const float* x, int64_t n, uint8_t* out, hipStream_t stream) {
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL(e4m3_quantize_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, x, n, out);
  return hipGetLastError();
}

}  // namespace dsa
