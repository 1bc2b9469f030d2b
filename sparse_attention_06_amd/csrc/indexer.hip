// indexer.hip -- Lightning Indexer scores on gfx950.
//
// Page references:
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org),
//               section "Lightning Indexer", the equation for I_tj
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io), section "稀疏注意力：NSA 与 DSA":
//               64 indexer heads of 128 dims, one 128-dim key per position, FP8
//
//   scores[r, j] = k_scale[j] * sum_h w[r, h] * ReLU(q[r, h, :] . k8[j, :]),  j <= q_pos[r]
//
// Tuned kernel (Hi = 64, Di = 128, E4M3): the head-by-key products are a dense contraction, so
// they run on the matrix cores: M = 16 heads, N = 16 keys, K = 32 dims per MFMA
// (v_mfma_f32_16x16x32_f16). The FP8 bytes are read from HBM as FP8 and widened to f16 in
// registers (exact: every E4M3 value is an f16 value); the f16 MFMA accumulates in fp32 at full
// fp32 accuracy, whereas the FP8 MFMA's internal accumulation was measured at ~4e-5 relative
// error, too coarse for the score tolerance. ReLU, the head weights and the head sum form the
// epilogue: each lane holds 4 heads of one key per MFMA tile, sums its 16 heads, and two
// cross-lane adds finish the 64-head sum.
//
// Query operands stay in registers for the whole kernel (the A operand), keys stream through
// (the B operand). The contraction dimension is permuted identically on both sides (lane group
// g = lane/16 owns dims [32g, 32g+32) of every key and query head, 8 per K step), which lets each
// lane fetch 32 contiguous key bytes; the dot product does not depend on the order of its terms.
#include "dsa_internal.h"

namespace dsa {

// ------------------------------------------------------------------ generic (any shape)

__device__ __forceinline__ float load_elem(const void* base, int64_t i, int is_f32) {
  if (is_f32) return ((const float*)base)[i];
  uint32_t b = ((const uint8_t*)base)[i];
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

__global__ void __launch_bounds__(256) indexer_generic_kernel(
    const void* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos, int q_per_seq,
    int max_ctx, int Hi, int Di, int is_f32, float* __restrict__ scores, int64_t ld_scores) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= max_ctx) return;
  const int t = q_pos[r];
  float* out = scores + (int64_t)r * ld_scores + j;
  if (j > t) { *out = -INFINITY; return; }
  const int64_t row = phys_row(kc.page_table, kc.ld_pt, kc.page_size, kc.num_pages, r / q_per_seq, j);
  if (row < 0) { *out = -INFINITY; return; }
  float acc = 0.f;
  for (int h = 0; h < Hi; ++h) {
    float dot = 0.f;
    const int64_t qb = ((int64_t)r * Hi + h) * Di;
    for (int c = 0; c < Di; ++c) dot = fmaf(load_elem(q, qb + c, is_f32), load_elem(kc.base, row * Di + c, is_f32), dot);
    acc = fmaf(w[(int64_t)r * Hi + h], fmaxf(dot, 0.f), acc);
  }
  *out = acc * (k_scale ? k_scale[row] : 1.f);
}

hipError_t launch_indexer_generic(const void* q, const float* w, PagedCache kc, const float* k_scale,
                                  const int32_t* q_pos, int n_seq, int q_per_seq, int max_ctx, int Hi,
                                  int Di, int is_f32, float* scores, int64_t ld_scores,
                                  hipStream_t stream) {
  const int rows = n_seq * q_per_seq;
  dim3 grid((max_ctx + 255) / 256, rows);
  hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(256), 0, stream, q, w, kc, k_scale, q_pos,
                     q_per_seq, max_ctx, Hi, Di, is_f32, scores, ld_scores);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tuned (64 heads x 128 dims, E4M3)

constexpr int kHi = 64, kDi = 128;

// One wave's operands for NQ query rows: A[qi][mt][ks] holds heads 16*mt + lane%16, dims
// 32*(lane/16) + 8*ks .. +8 as f16; W[qi][mt][i] is the weight of head 16*mt + 4*(lane/16) + i.
template <int NQ>
struct QueryOps {
  f16x8 A[NQ][4][4];
  float W[NQ][4][4];
  int tpos[NQ];
  int64_t row[NQ];
};

template <int NQ>
__device__ __forceinline__ void load_query_ops(QueryOps<NQ>& o, const uint8_t* __restrict__ q,
                                               const float* __restrict__ w,
                                               const int32_t* __restrict__ q_pos, int row0,
                                               int nrows_valid, int lane) {
  const int g = lane >> 4, m = lane & 15;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const bool valid = qi < nrows_valid;
    const int r = row0 + (valid ? qi : 0);
    o.row[qi] = r;
    o.tpos[qi] = valid ? q_pos[r] : -1;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const i32x4* p = (const i32x4*)(q + ((int64_t)r * kHi + 16 * mt + m) * kDi + 32 * g);
      i32x4 r0 = p[0], r1 = p[1];
      e4m3x16_to_f16(r0, o.A[qi][mt][0], o.A[qi][mt][1]);
      e4m3x16_to_f16(r1, o.A[qi][mt][2], o.A[qi][mt][3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) o.W[qi][mt][i] = w[(int64_t)r * kHi + 16 * mt + 4 * g + i];
    }
  }
}

struct KeyTile {
  i32x4 raw0, raw1;  // 32 key bytes of this lane's key: dims 32*(lane/16) .. +32
  float scale;
  int j;             // position of this lane's key (lane%16 within the tile)
  bool valid;
};

__device__ __forceinline__ void fetch_key_tile(KeyTile& kt, const PagedCache& kc,
                                               const float* __restrict__ k_scale, int seq, int jbase,
                                               int jend, int lane) {
  const int j = jbase + (lane & 15);
  kt.j = j;
  int64_t row = -1;
  if (j < jend) row = phys_row(kc.page_table, kc.ld_pt, kc.page_size, kc.num_pages, seq, j);
  kt.valid = row >= 0;
  if (kt.valid) {
    const i32x4* p = (const i32x4*)((const uint8_t*)kc.base + row * kDi + 32 * (lane >> 4));
    kt.raw0 = __builtin_nontemporal_load(p);
    kt.raw1 = __builtin_nontemporal_load(p + 1);
    kt.scale = k_scale ? k_scale[row] : 1.f;
  } else {
    kt.raw0 = i32x4{0, 0, 0, 0};
    kt.raw1 = i32x4{0, 0, 0, 0};
    kt.scale = 0.f;
  }
}

template <int NQ>
__device__ __forceinline__ void score_key_tile(const QueryOps<NQ>& o, const KeyTile& kt,
                                               float* __restrict__ scores, int64_t ld_scores,
                                               int jend, int lane) {
  f16x8 B[4];
  e4m3x16_to_f16(kt.raw0, B[0], B[1]);
  e4m3x16_to_f16(kt.raw1, B[2], B[3]);
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    float v = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.A[qi][mt][ks], B[ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) v = fmaf(o.W[qi][mt][i], fmaxf(acc[i], 0.f), v);
    }
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (lane < 16 && kt.j < jend && o.tpos[qi] >= 0) {
      float s = (kt.j <= o.tpos[qi] && kt.valid) ? v * kt.scale : -INFINITY;
      scores[o.row[qi] * ld_scores + kt.j] = s;
    }
  }
}

// Key scan for decode / MTP: block (chunk, seq); the seq's NQ rows share every key read.
template <int NQ>
__global__ void __launch_bounds__(256) indexer_scan_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos, int keys_per_block,
    int max_ctx, float* __restrict__ scores, int64_t ld_scores) {
  const int seq = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  QueryOps<NQ> o;
  load_query_ops<NQ>(o, q, w, q_pos, seq * NQ, NQ, lane);
  int tmax = -1;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) tmax = max(tmax, o.tpos[qi]);
  const int jbeg = blockIdx.x * keys_per_block;
  const int jend = min(min(jbeg + keys_per_block, tmax + 1), max_ctx);  // never past ld_scores
  if (jbeg >= jend) return;
  // tiles of 16 keys, interleaved over the 4 waves, one tile of look-ahead
  int jb = jbeg + 16 * wave;
  if (jb >= jend) return;
  KeyTile cur, nxt;
  fetch_key_tile(cur, kc, k_scale, seq, jb, jend, lane);
  for (; jb < jend; jb += 64) {
    if (jb + 64 < jend) fetch_key_tile(nxt, kc, k_scale, seq, jb + 64, jend, lane);
    score_key_tile<NQ>(o, cur, scores, ld_scores, jend, lane);
    cur = nxt;
  }
}

// Prefill tiles: each wave owns 2 consecutive rows of one sequence and scans their causal
// prefix; the 4 waves of a block walk the same keys in step, so key reads hit the caches.
__global__ void __launch_bounds__(256) indexer_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos, int q_per_seq,
    int rows, int max_ctx, float* __restrict__ scores, int64_t ld_scores) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // heavy blocks first: in a causal chunk the last rows have the longest prefixes
  const int block = gridDim.x - 1 - blockIdx.x;
  const int row0 = block * 8 + 2 * wave;
  if (row0 >= rows) return;
  const int seq = row0 / q_per_seq;
  const int nvalid = (row0 + 1 < rows && (row0 + 1) / q_per_seq == seq) ? 2 : 1;
  QueryOps<2> o;
  load_query_ops<2>(o, q, w, q_pos, row0, nvalid, lane);
  const int jend = min(max(o.tpos[0], o.tpos[1]) + 1, max_ctx);  // never past ld_scores
  if (jend <= 0) return;
  KeyTile cur, nxt;
  int jb = 0;
  fetch_key_tile(cur, kc, k_scale, seq, jb, jend, lane);
  for (; jb < jend; jb += 16) {
    if (jb + 16 < jend) fetch_key_tile(nxt, kc, k_scale, seq, jb + 16, jend, lane);
    score_key_tile<2>(o, cur, scores, ld_scores, jend, lane);
    cur = nxt;
  }
}

hipError_t launch_indexer_scan(const uint8_t* q, const float* w, PagedCache kc, const float* k_scale,
                               const int32_t* q_pos, int n_seq, int q_per_seq, int max_ctx,
                               float* scores, int64_t ld_scores, hipStream_t stream) {
  // enough blocks to cover the chip a few times, chunks a multiple of 64 keys
  int64_t total = (int64_t)n_seq * max_ctx;
  int kpb = (int)((total / 1024 + 63) / 64 * 64);
  kpb = kpb < 256 ? 256 : (kpb > 4096 ? 4096 : kpb);
  dim3 grid((max_ctx + kpb - 1) / kpb, n_seq);
  if (q_per_seq == 1)
    hipLaunchKernelGGL(indexer_scan_kernel<1>, grid, dim3(256), 0, stream, q, w, kc, k_scale, q_pos, kpb, max_ctx, scores, ld_scores);
  else
    hipLaunchKernelGGL(indexer_scan_kernel<2>, grid, dim3(256), 0, stream, q, w, kc, k_scale, q_pos, kpb, max_ctx, scores, ld_scores);
  return hipGetLastError();
}

hipError_t launch_indexer_prefill(const uint8_t* q, const float* w, PagedCache kc,
                                  const float* k_scale, const int32_t* q_pos, int n_seq,
                                  int q_per_seq, int max_ctx, float* scores, int64_t ld_scores,
                                  hipStream_t stream) {
  const int rows = n_seq * q_per_seq;
  dim3 grid((rows + 7) / 8);
  hipLaunchKernelGGL(indexer_prefill_kernel, grid, dim3(256), 0, stream, q, w, kc, k_scale, q_pos, q_per_seq, rows, max_ctx, scores, ld_scores);
  return hipGetLastError();
}

}  // namespace dsa
