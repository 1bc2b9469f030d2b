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

// ---- decode / MTP key scan: LDS-staged, one DMA ring per wave
//
// Each wave scans a contiguous key range of one sequence for all NQ query rows of that sequence
// (the rows of a sequence share every key read). Keys stream from HBM straight into a wave-private
// ring of kRing tiles in LDS with global_load_lds (16 keys x 128 B = 2 KB per tile in two
// wave-wide loads, plus the 16 per-token scales), kRing - 1 tiles ahead of the MFMAs, so enough
// bytes are in flight to cover HBM latency without holding them in registers; no workgroup
// barrier is involved. In LDS, key k (0..7) of 1 KB block b keeps its 16-byte chunk c at granule
// 8k + (c ^ ((k & 6) | b)), so the 16 keys read together by a lane group land on 16 distinct
// bank groups.
constexpr int kRing = 8;
constexpr int kTileKeys = 16;
constexpr int kRingTileBytes = kTileKeys * kDi;         // 2048
constexpr int kRingScaleBytes = 256;                    // 64 lanes x 4 B (scale of key lane%16)
constexpr int kWaveRingBytes = kRing * (kRingTileBytes + kRingScaleBytes);
constexpr int kScanWaves = 4;
constexpr int kScanPage = 64;                           // page size the scan is built for
constexpr int kScanLdsBytes = kScanWaves * kWaveRingBytes;  // 73728

typedef __attribute__((address_space(3))) uint8_t lds8;

// Issue the loads of one tile (16 consecutive keys of one page, starting at physical row row0)
// into ring slot `slot`: two wave-wide 16-byte-per-lane key loads and one 4-byte-per-lane scale
// load, always exactly three vector-memory instructions (so the ring's wait counts are exact).
// row0 < 0 (invalid page) loads key row 0 instead: finite data, and its keys score -inf.
__device__ __forceinline__ void scan_issue_tile(lds8* ring, int slot, const uint8_t* __restrict__ kbase,
                                                const float* __restrict__ k_scale, int row0, int lane) {
  asm volatile("" : "+v"(lane));
  row0 = row0 < 0 ? 0 : row0;
  const uint8_t* kb = kbase + (int64_t)row0 * kDi;
  const int k = lane >> 3, gp = lane & 7;
  const uint32_t kdst = (uint32_t)(uintptr_t)(ring + slot * kRingTileBytes);
  const uint32_t sdst = (uint32_t)(uintptr_t)(ring + kRing * kRingTileBytes + slot * kRingScaleBytes);
  const uint8_t* src0 = kb + k * kDi + 16 * (gp ^ (k & 6));
  const uint8_t* src1 = kb + (8 + k) * kDi + 16 * (gp ^ ((k & 6) | 1));
  // without a scale array the scale slot loads key bytes and is never read
  const void* ssrc = k_scale ? (const void*)(k_scale + row0 + (lane & 15)) : (const void*)(kb + 4 * (lane & 15));
  uint32_t sv;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[d0]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[a0], off\n\t"
      "s_mov_b32 m0, %[d1]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[a1], off\n\t"
      "s_mov_b32 m0, %[d2]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %[a2], off\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(sv)
      : [d0] "s"(__builtin_amdgcn_readfirstlane(kdst)), [d1] "s"(__builtin_amdgcn_readfirstlane(kdst + 1024)),
        [d2] "s"(__builtin_amdgcn_readfirstlane(sdst)), [a0] "v"(src0), [a1] "v"(src1), [a2] "v"(ssrc)
      : "memory");
}

// Wait until at most 3*d vector-memory instructions of this wave are outstanding (d < kRing - 1).
__device__ __forceinline__ void scan_wait_tiles(int d) {
  switch (d) {
#define W(D) case D: __builtin_amdgcn_s_waitcnt(0x0F70 | ((3 * (D)) & 15) | (((3 * (D)) >> 4) << 14)); break;
    W(1) W(2) W(3) W(4) W(5) W(6)
#undef W
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Sum over the four 16-lane groups (lanes m, m+16, m+32, m+48), without an LDS round trip.
__device__ __forceinline__ float sum_lane_groups(float v, int lane) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float(lane < 32 ? a[1] : a[0]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float(((lane >> 4) & 1) == 0 ? b[1] : b[0]);
  return v;
}

// ReLU on the bit pattern: negative floats (sign bit set) are negative integers, so the integer
// maximum with 0 maps them (and -0) to +0 and keeps every non-negative value; one VALU op.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

template <int NQ>
__global__ void __launch_bounds__(256) indexer_scan_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos, int keys_per_wave,
    int max_ctx, float* __restrict__ scores, int64_t ld_scores) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kScanLdsBytes];
  const int seq = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  QueryOps<NQ> o;
  load_query_ops<NQ>(o, q, w, q_pos, seq * NQ, NQ, lane);
  int tmax = -1;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) tmax = max(tmax, o.tpos[qi]);
  // pages of kScanPage keys; a wave's range starts on a page and spans at most 64 pages
  const int jbeg = (blockIdx.x * kScanWaves + wave) * keys_per_wave;
  const int jend = min(min(jbeg + keys_per_wave, tmax + 1), max_ctx);  // never past ld_scores
  if (jbeg >= jend) return;
  const int ntiles = (jend - jbeg + kTileKeys - 1) / kTileKeys;
  // the physical ids of the range's pages, one per lane, so the tile loop reads no page table
  // from memory (such a load's wait would drain the ring)
  int vpage = -1;
  {
    const int p = jbeg / kScanPage + lane;
    if (lane * kScanPage < jend - jbeg && p < kc.ld_pt) vpage = kc.page_table[(int64_t)seq * kc.ld_pt + p];
    if (vpage >= kc.num_pages) vpage = -1;
  }
  auto tile_row0 = [&](int it) -> int {  // physical row of the tile's first key, or -1
    const int pid = __builtin_amdgcn_readlane(vpage, (kTileKeys * it) / kScanPage);
    return pid < 0 ? -1 : pid * kScanPage + (kTileKeys * it) % kScanPage;
  };
  // the query operands and page ids are complete before the ring starts, so no compiler wait
  // for them sits among the ring's loads (it would drain them)
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(o.A[qi][mt][ks]));
  asm volatile("" ::"v"(vpage));
  __builtin_amdgcn_s_waitcnt(0x0F70);
  lds8* ring = (lds8*)smem + wave * kWaveRingBytes;
  const uint8_t* kbase = (const uint8_t*)kc.base;
  const int m = lane & 15, g = lane >> 4;
  // this lane's key m within the tile: block b = m/8, key k = m%8; chunks 2g and 2g+1
  const int kb = m >> 3, kk = m & 7, x = (kk & 6) | kb;
  const int rd0 = kb * 1024 + 16 * (8 * kk + ((2 * g) ^ x));
  const int rd1 = kb * 1024 + 16 * (8 * kk + ((2 * g + 1) ^ x));
#pragma unroll
  for (int p = 0; p < kRing - 1; ++p)
    if (p < ntiles) scan_issue_tile(ring, p, kbase, k_scale, tile_row0(p), lane);

  // Wait for tile `it`'s three loads. Vector-memory instructions complete in issue order, so it
  // is enough that at most the instructions issued after them are outstanding: in steady state
  // the loads of the kRing - 2 later tiles and the NQ score stores of each of the last kRing - 2
  // iterations (a tile is waited for one iteration before it is computed). Near the ends of the
  // range the count ignores the stores (a lower count only waits longer).
  auto wait_tile = [&](int it) {
    const int later_tiles = min(kRing - 2, ntiles - 1 - it);
    if (it >= kRing - 1 && later_tiles == kRing - 2) {
      constexpr int n = 3 * (kRing - 2) + NQ * (kRing - 2);
      static_assert(n < 64, "vmcnt range");
      __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    } else {
      scan_wait_tiles(later_tiles);
    }
  };
  // the raw key bytes and scale of the tile computed next, read from LDS one iteration ahead
  auto read_tile = [&](int it, i32x4& r0, i32x4& r1, float& sc) {
    const int slot = it % kRing;
    const lds8* tk = ring + slot * kRingTileBytes;
    r0 = *(const __attribute__((address_space(3))) i32x4*)(tk + rd0);
    r1 = *(const __attribute__((address_space(3))) i32x4*)(tk + rd1);
    sc = k_scale ? *(const __attribute__((address_space(3))) float*)(ring + kRing * kRingTileBytes + slot * kRingScaleBytes + 4 * m) : 1.f;
  };
  i32x4 raw0, raw1;
  float scale;
  wait_tile(0);
  read_tile(0, raw0, raw1, scale);
  for (int it = 0; it < ntiles; ++it) {
    if (it + kRing - 1 < ntiles)
      scan_issue_tile(ring, (it + kRing - 1) % kRing, kbase, k_scale, tile_row0(it + kRing - 1), lane);
    f16x8 B[4];
    e4m3x16_to_f16(raw0, B[0], B[1]);
    e4m3x16_to_f16(raw1, B[2], B[3]);
    const float sc = scale;
    const int j = jbeg + kTileKeys * it + m;
    const bool page_ok = tile_row0(it) >= 0;
    if (it + 1 < ntiles) {
      wait_tile(it + 1);
      read_tile(it + 1, raw0, raw1, scale);
    }
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(o.A[qi][mt][ks], B[ks], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v = fmaf(o.W[qi][mt][i], relu_bits(acc[i]), v);
      }
      v = sum_lane_groups(v, lane);
      // exactly one store instruction per query per tile (lane 0 always has j < jend), so the
      // wait counts above stay exact; positions past q_pos get -inf
      if (lane < 16 && j < jend) {
        const float s = (j <= o.tpos[qi] && page_ok) ? v * sc : -INFINITY;
        scores[o.row[qi] * ld_scores + j] = s;
      }
    }
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
  // about 2048 waves (8 per CU) in all, each a whole number of pages (at most 64 of them)
  const int64_t total = (int64_t)n_seq * max_ctx;
  int kpw = (int)((total / 2048 + kScanPage - 1) / kScanPage * kScanPage);
  kpw = kpw < kScanPage ? kScanPage : (kpw > 64 * kScanPage ? 64 * kScanPage : kpw);
  const int per_block = kScanWaves * kpw;
  dim3 grid((max_ctx + per_block - 1) / per_block, n_seq);
  if (q_per_seq == 1)
    hipLaunchKernelGGL(indexer_scan_kernel<1>, grid, dim3(64 * kScanWaves), 0, stream, q, w, kc, k_scale, q_pos, kpw, max_ctx, scores, ld_scores);
  else
    hipLaunchKernelGGL(indexer_scan_kernel<2>, grid, dim3(64 * kScanWaves), 0, stream, q, w, kc, k_scale, q_pos, kpw, max_ctx, scores, ld_scores);
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
