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
    const float* __restrict__ k_scale, RowSeq rs, const int32_t* __restrict__ q_pos,
    int max_ctx, int Hi, int Di, int is_f32, float* __restrict__ scores, int64_t ld_scores) {
  const int r = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= max_ctx) return;
  const int t = q_pos[r];
  float* out = scores + (int64_t)r * ld_scores + j;
  if (j > t) { *out = -INFINITY; return; }
  const int64_t row = phys_row(kc.page_table, kc.ld_pt, kc.page_size, kc.num_pages, rs.of(r), j);
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
                                  RowSeq rs, const int32_t* q_pos, int rows, int max_ctx, int Hi,
                                  int Di, int is_f32, float* scores, int64_t ld_scores,
                                  hipStream_t stream) {
  dim3 grid((max_ctx + 255) / 256, rows);
  hipLaunchKernelGGL(indexer_generic_kernel, grid, dim3(256), 0, stream, q, w, kc, k_scale, rs, q_pos,
                     max_ctx, Hi, Di, is_f32, scores, ld_scores);
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
// Each wave scans a contiguous, page-aligned key range of one sequence for all NQ query rows of
// that sequence (the rows of a sequence share every key read). One loop iteration is one page of
// 64 keys, computed as four 16-key sub-tiles. Keys stream from HBM straight into a wave-private
// ring of eight 16-key slots (two pages) in LDS with global_load_lds: a slot is refilled with the
// same sub-tile of the page two ahead as soon as its bytes are in registers, so about six slots
// are in flight while one is computed, and no workgroup barrier is involved. Each page's 64
// per-token scales ride along in one 4-byte-per-lane load into one of four scale slots.
//
// In a slot, key k (0..7) of 1 KB block b keeps its 16-byte chunk c at granule 8k + (c ^ ((k & 6) | b)),
// so the 16 keys read together by a lane group land on 16 distinct bank groups.
//
// The head sums of a page's four sub-tiles are reduced over the four 16-lane groups together (two
// permlane32 swaps, one permlane16 swap), which leaves lane l with the score of key l of the page:
// one 256-byte store per query row per page.
constexpr int kRing = 8;
constexpr int kTileKeys = 16;
constexpr int kScanPage = 64;                           // page size the scan is built for
constexpr int kSubTiles = kScanPage / kTileKeys;        // 4
constexpr int kRingTileBytes = kTileKeys * kDi;         // 2048
constexpr int kScaleSlots = 4;
constexpr int kScaleSlotBytes = 4 * kScanPage;          // 256
constexpr int kWaveRingBytes = kRing * kRingTileBytes + kScaleSlots * kScaleSlotBytes;  // 17408
constexpr int kScanWaves = 4;
constexpr int kScanLdsBytes = kScanWaves * kWaveRingBytes;  // 69632

typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) uint32_t lds32;

// Two wave-wide 16-byte-per-lane loads of one 16-key slot (src = first key of the sub-tile);
// with_scale adds the 4-byte-per-lane load of a page's 64 scales (ssrc = first scale). Exactly
// 2 (+1) vector-memory instructions, so the ring's wait counts are exact.
template <bool with_scale>
__device__ __forceinline__ void scan_dma(uint32_t kdst, uint32_t sdst, uint64_t src, uint64_t ssrc,
                                         int voff0, int voff1, int soff) {
  uint32_t sv;
  if (with_scale) {
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[d0]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[o0], %[src]\n\t"
        "s_mov_b32 m0, %[d1]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[o1], %[src]\n\t"
        "s_mov_b32 m0, %[d2]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %[o2], %[ssrc]\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(sv)
        : [d0] "s"(kdst), [d1] "s"(kdst + 1024), [d2] "s"(sdst), [src] "s"(src), [ssrc] "s"(ssrc),
          [o0] "v"(voff0), [o1] "v"(voff1), [o2] "v"(soff)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %[sv], m0\n\t"
        "s_mov_b32 m0, %[d0]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[o0], %[src]\n\t"
        "s_mov_b32 m0, %[d1]\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %[o1], %[src]\n\t"
        "s_mov_b32 m0, %[sv]"
        : [sv] "=&s"(sv)
        : [d0] "s"(kdst), [d1] "s"(kdst + 1024), [src] "s"(src), [o0] "v"(voff0), [o1] "v"(voff1)
        : "memory");
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Reduce four per-lane values v[t] (sub-tile t of a page, this lane's 16 heads) over the four
// 16-lane groups: lane l ends with the 64-head total of sub-tile l/16 at key l%16 = key l of the page.
__device__ __forceinline__ float reduce_page(float v0, float v1, float v2, float v3) {
  // halves: lanes < 32 keep sub-tiles 0 and 1, lanes >= 32 keep 2 and 3
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float u02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float u13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  // neighbouring 16-lane groups: even groups keep sub-tile 0 / 2, odd groups 1 / 3
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u02), __float_as_uint(u13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// ReLU on the bit pattern: negative floats (sign bit set) are negative integers, so the integer
// maximum with 0 maps them (and -0) to +0 and keeps every non-negative value; one VALU op.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// Vector-memory instructions complete in issue order, so waiting for a slot means allowing only the
// instructions issued after its loads to be outstanding. Per page the wave issues 2 loads per
// sub-tile, 1 scale load and NQ score stores; the refill of a page happens two iterations before it
// is computed. For sub-tile t = 1..3 of the current page the later instructions are the page's
// remaining sub-tiles, the stores of the two previous iterations, the next page and the refills
// already issued for the page after it; t = 4 stands for sub-tile 0 of the next page, waited for
// before this iteration's stores. kTail: 0 = refills run two pages ahead, 1 = the next page is the
// last one, 2 = this is the last page.
template <int NQ, int kTail>
constexpr int scan_wait_count(int t) {
  if (t == 4) return kTail == 0 ? 16 + NQ : 7 + NQ;
  return kTail == 0 ? 16 + 2 * NQ : kTail == 1 ? 15 - 2 * t + 2 * NQ : 6 - 2 * t + 2 * NQ;
}

struct ScanCtx {
  lds8* ring;            // this wave's ring
  uint32_t ring_addr;    // its LDS address
  uint64_t kbase;        // key rows
  uint64_t sbase;        // per-token scales (key rows when there are none: loaded, never read)
  int vpage;             // physical page of this wave's page `lane`, or -1
  int voff0, voff1, soff;
  int rd0, rd1;          // this lane's LDS read offsets within a slot
};

__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | lo;
}

// refill sub-tile t of page p (into the slot its page parity and t select)
template <int t>
__device__ __forceinline__ void scan_refill(const ScanCtx& c, int p, bool has_scale) {
  int pid = __builtin_amdgcn_readlane(c.vpage, p);
  pid = pid < 0 ? 0 : pid;  // a missing page loads page 0: finite bytes whose scores are -inf
  const uint32_t kdst = c.ring_addr + ((p & 1) * kSubTiles + t) * kRingTileBytes;
  const uint64_t src = c.kbase + (uint64_t)(uint32_t)pid * (kScanPage * kDi) + t * kRingTileBytes;
  if (t == 0) {
    const uint32_t sdst = c.ring_addr + kRing * kRingTileBytes + (p & (kScaleSlots - 1)) * kScaleSlotBytes;
    const uint64_t ssrc = has_scale ? c.sbase + (uint64_t)(uint32_t)pid * (4 * kScanPage) : c.kbase;
    scan_dma<true>(__builtin_amdgcn_readfirstlane(kdst), __builtin_amdgcn_readfirstlane(sdst), uniform_u64(src),
                   uniform_u64(ssrc), c.voff0, c.voff1, c.soff);
  } else {
    scan_dma<false>(__builtin_amdgcn_readfirstlane(kdst), 0, uniform_u64(src), 0, c.voff0, c.voff1, 0);
  }
}

__device__ __forceinline__ void scan_read(const ScanCtx& c, int p, int t, i32x4& r0, i32x4& r1) {
  const lds8* tk = c.ring + ((p & 1) * kSubTiles + t) * kRingTileBytes;
  r0 = *(const __attribute__((address_space(3))) i32x4*)(tk + c.rd0);
  r1 = *(const __attribute__((address_space(3))) i32x4*)(tk + c.rd1);
}

// One query row's 16 MFMAs over a sub-tile (the four accumulation chains advance together, K step
// outermost, so consecutive MFMAs never wait on each other).
__device__ __forceinline__ void row_mfmas(const f16x8 (&A)[4][4], const f16x8 (&B)[4], f32x4 (&acc)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][ks], B[ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt],
                                                        0, 0, 0);
}

// This lane's 16-head sum of w * ReLU(s) from one row's accumulators (two partial sums break the
// FMA chain).
__device__ __forceinline__ float head_sum(const float (&W)[4][4], const f32x4 (&acc)[4]) {
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      v0 = fmaf(W[mt][i], relu_bits(acc[mt][i]), v0);
      v1 = fmaf(W[mt][i + 1], relu_bits(acc[mt][i + 1]), v1);
    }
  return v0 + v1;
}

// Ask the scheduler to alternate one MFMA with two VALU ops, sixteen times: a row's MFMAs then run
// while the VALU works through another row's head sums, within one wave.
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
  }
}

// Sub-tile t of page p: its bytes are in raw0/raw1 (read during the previous sub-tile). The rows'
// MFMAs and head sums are software-pipelined: row 0's MFMAs run alongside the head sum of the
// last row of the previous sub-tile (its accumulators carried in `carry`), row 1's alongside row
// 0's head sum; the last row's head sum of this sub-tile is left in `carry` for the next one
// (for the last sub-tile of a page, the page's epilogue does it). Leaves v[qi][t] (v[NQ-1][t-1])
// and the next sub-tile's bytes in raw0/raw1.
template <int NQ, int kTail, int t>
__device__ __forceinline__ void scan_subtile(const ScanCtx& c, const QueryOps<NQ>& o, int p, bool has_scale,
                                             i32x4& raw0, i32x4& raw1, f32x4 (&carry)[4],
                                             float (&v)[NQ][kSubTiles]) {
  f16x8 B[4];
  e4m3x16_to_f16(raw0, B[0], B[1]);
  e4m3x16_to_f16(raw1, B[2], B[3]);
  if (kTail == 0) {
    // the slot's bytes are in registers: refill it with the same sub-tile two pages ahead
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    scan_refill<t>(c, p + 2, has_scale);
  }
  // read the next sub-tile (of this page, or sub-tile 0 of the next page)
  if (t + 1 < kSubTiles) {
    wait_vm<scan_wait_count<NQ, kTail>(t + 1)>();
    scan_read(c, p, t + 1, raw0, raw1);
  } else if (kTail != 2) {
    wait_vm<scan_wait_count<NQ, kTail>(4)>();
    scan_read(c, p + 1, 0, raw0, raw1);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc0[4];
  row_mfmas(o.A[0], B, acc0);
  if (t > 0) v[NQ - 1][t - 1] = head_sum(o.W[NQ - 1], carry);
  interleave_mfma_valu();
  if (NQ == 2) {
    f32x4 acc1[4];
    row_mfmas(o.A[NQ - 1], B, acc1);
    v[0][t] = head_sum(o.W[0], acc0);
    interleave_mfma_valu();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) carry[mt] = acc1[mt];
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) carry[mt] = acc0[mt];
  }
  __builtin_amdgcn_sched_barrier(0);
  // pin the head sums here, so that their accumulators die in this sub-tile
  if (t > 0) asm volatile("" : "+v"(v[NQ - 1][t - 1]));
  if (NQ == 2) asm volatile("" : "+v"(v[0][t]));
}

// One page: four sub-tiles, then the page's reduction, scale, mask and stores.
template <int NQ, bool kHist, int kTail>
__device__ __forceinline__ void scan_page(const ScanCtx& c, const QueryOps<NQ>& o, int p, int jpage, int jend,
                                          bool has_scale, float* __restrict__ scores, int64_t ld_scores,
                                          i32x4& raw0, i32x4& raw1, lds32* hist, int lane) {
  float v[NQ][kSubTiles];
  f32x4 carry[4];
  scan_subtile<NQ, kTail, 0>(c, o, p, has_scale, raw0, raw1, carry, v);
  scan_subtile<NQ, kTail, 1>(c, o, p, has_scale, raw0, raw1, carry, v);
  scan_subtile<NQ, kTail, 2>(c, o, p, has_scale, raw0, raw1, carry, v);
  scan_subtile<NQ, kTail, 3>(c, o, p, has_scale, raw0, raw1, carry, v);
  v[NQ - 1][kSubTiles - 1] = head_sum(o.W[NQ - 1], carry);
  // lane l now scores key jpage + l
  const float sc = has_scale ? *(const __attribute__((address_space(3))) float*)(
                                   c.ring + kRing * kRingTileBytes + (p & (kScaleSlots - 1)) * kScaleSlotBytes + 4 * lane)
                             : 1.f;
  const bool page_ok = __builtin_amdgcn_readlane(c.vpage, p) >= 0;
  const int j = jpage + lane;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float tot = reduce_page(v[qi][0], v[qi][1], v[qi][2], v[qi][3]);
    // exactly one store instruction per query row per page (lane 0 always has j < jend), so the
    // wait counts stay exact; positions past the row's q_pos get -inf
    const float val = (j <= o.tpos[qi] && page_ok) ? tot * sc : -INFINITY;
    if (j < jend) scores[o.row[qi] * ld_scores + j] = val;
    if (kHist && j < jend && j <= o.tpos[qi]) {
      // the row's first-digit histogram, two 16-bit counts per word
      const uint32_t d = order_key(val) >> 21;
      __hip_atomic_fetch_add(hist + qi * (kTopkDigit0Bins / 2) + (d >> 1), 1u << ((d & 1u) << 4), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

// One wave's key range [jbeg, jend) of a unit's rows.
template <int NQ, bool kHist>
__device__ __forceinline__ void scan_range(const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
                                           const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos,
                                           int unit, int seq, int jbeg, int jend, float* __restrict__ scores,
                                           int64_t ld_scores, lds32* hist, uint8_t* smem, int lane, int wave) {
  const int np = (jend - jbeg + kScanPage - 1) / kScanPage;
  ScanCtx c;
  // the physical ids of the range's pages, one per lane, so the loop reads no page table from
  // memory (such a load's wait would drain the ring)
  c.vpage = -1;
  {
    const int pg = jbeg / kScanPage + lane;
    if (seq >= 0 && lane < np && pg < kc.ld_pt) c.vpage = kc.page_table[(int64_t)seq * kc.ld_pt + pg];
    if (c.vpage >= kc.num_pages) c.vpage = -1;
  }
  QueryOps<NQ> o;
  load_query_ops<NQ>(o, q, w, q_pos, unit * NQ, NQ, lane);
  c.ring = (lds8*)smem + wave * kWaveRingBytes;
  c.ring_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)c.ring);
  c.kbase = uniform_u64((uint64_t)(uintptr_t)kc.base);
  const bool has_scale = k_scale != nullptr;
  c.sbase = uniform_u64((uint64_t)(uintptr_t)(has_scale ? (const void*)k_scale : kc.base));
  {
    const int k = lane >> 3, gp = lane & 7;
    c.voff0 = k * kDi + 16 * (gp ^ (k & 6));
    c.voff1 = (8 + k) * kDi + 16 * (gp ^ ((k & 6) | 1));
    c.soff = 4 * lane;
    const int m = lane & 15, g = lane >> 4;
    const int kb = m >> 3, kk = m & 7, x = (kk & 6) | kb;
    c.rd0 = kb * 1024 + 16 * (8 * kk + ((2 * g) ^ x));
    c.rd1 = kb * 1024 + 16 * (8 * kk + ((2 * g + 1) ^ x));
  }
  // the first two pages, then drain everything (query operands included) before the loop
  scan_refill<0>(c, 0, has_scale); scan_refill<1>(c, 0, has_scale);
  scan_refill<2>(c, 0, has_scale); scan_refill<3>(c, 0, has_scale);
  if (np > 1) {
    scan_refill<0>(c, 1, has_scale); scan_refill<1>(c, 1, has_scale);
    scan_refill<2>(c, 1, has_scale); scan_refill<3>(c, 1, has_scale);
  }
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" ::"v"(o.A[qi][mt][ks]));
  wait_vm<0>();
  i32x4 raw0, raw1;
  scan_read(c, 0, 0, raw0, raw1);
  int p = 0;
  for (; p + 2 < np; ++p)
    scan_page<NQ, kHist, 0>(c, o, p, jbeg + kScanPage * p, jend, has_scale, scores, ld_scores, raw0, raw1, hist, lane);
  if (p + 1 < np) {
    scan_page<NQ, kHist, 1>(c, o, p, jbeg + kScanPage * p, jend, has_scale, scores, ld_scores, raw0, raw1, hist, lane);
    ++p;
  }
  scan_page<NQ, kHist, 2>(c, o, p, jbeg + kScanPage * p, jend, has_scale, scores, ld_scores, raw0, raw1, hist, lane);
}


// Adds the workgroup's histogram counts into the rows' global histograms (non-zero bins only).
template <int NQ>
__device__ __forceinline__ void flush_hist(lds32* hist, uint32_t* __restrict__ hist0, int unit, int chunks, int chunk) {
  __syncthreads();
  for (int i = threadIdx.x; i < NQ * kTopkDigit0Bins / 2; i += 64 * kScanWaves) {
    const uint32_t v = hist[i];
    if (v == 0u) continue;
    const int qi = i / (kTopkDigit0Bins / 2), b = 2 * (i % (kTopkDigit0Bins / 2));
    uint32_t* g = hist0 + ((int64_t)(unit * NQ + qi) * chunks + chunk) * kTopkDigit0Bins + b;
    if (v & 0xFFFFu) __hip_atomic_fetch_add(g, v & 0xFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >> 16) __hip_atomic_fetch_add(g + 1, v >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int NQ, bool kHist>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) indexer_scan_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, RowSeq rs, const int32_t* __restrict__ q_pos, int keys_per_wave,
    int max_ctx, float* __restrict__ scores, int64_t ld_scores, uint32_t* __restrict__ hist0) {
  // with kHist, the rows' first-digit histograms (2 x 16 bits per word) follow the rings
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kScanLdsBytes + (kHist ? NQ * kTopkDigit0Bins * 2 : 0)];
  lds32* hist = (lds32*)((lds8*)smem + kScanLdsBytes);
  if (kHist) {
    for (int i = threadIdx.x; i < NQ * kTopkDigit0Bins / 8; i += 64 * kScanWaves)
      *(__attribute__((address_space(3))) i32x4*)(hist + 4 * i) = i32x4{0, 0, 0, 0};
    __syncthreads();
  }
  // this block's NQ query rows: unit * NQ .. + NQ - 1, all of one sequence (decode: the request's
  // rows; prefill: two consecutive rows of the block; one row per unit with per-row sequence ids)
  const int unit = blockIdx.y;
  const int seq = rs.of(unit * NQ);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tmax = -1;
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) tmax = max(tmax, q_pos[unit * NQ + qi]);
  // a wave's range starts on a page and spans at most 64 pages
  const int jbeg = (blockIdx.x * kScanWaves + wave) * keys_per_wave;
  const int jend = min(min(jbeg + keys_per_wave, tmax + 1), max_ctx);  // never past ld_scores
  if (jbeg < jend) scan_range<NQ, kHist>(q, w, kc, k_scale, q_pos, unit, seq, jbeg, jend, scores, ld_scores, hist, smem, lane, wave);
  // a workgroup's keys lie in one top-k chunk (its range is a power of two of at most a chunk)
  if (kHist) flush_hist<NQ>(hist, hist0, unit, (max_ctx + kTopkChunkKeys - 1) / kTopkChunkKeys,
                         blockIdx.x * kScanWaves * keys_per_wave / kTopkChunkKeys);
}

// Prefill tiles: each wave owns 2 consecutive rows and scans their causal prefix, the two
// together when they belong to one sequence, else one after the other; the 4 waves of a block walk
// the same keys in step, so key reads hit the caches.
__global__ void __launch_bounds__(256) indexer_prefill_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, PagedCache kc,
    const float* __restrict__ k_scale, RowSeq rs, const int32_t* __restrict__ q_pos,
    int rows, int max_ctx, float* __restrict__ scores, int64_t ld_scores) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // heavy blocks first: in a causal chunk the last rows have the longest prefixes
  const int block = gridDim.x - 1 - blockIdx.x;
  const int row0 = block * 8 + 2 * wave;
  const int row_end = min(row0 + 2, rows);
  for (int r = row0; r < row_end;) {
    const int seq = rs.of(r);
    const int nvalid = (r + 1 < row_end && rs.of(r + 1) == seq) ? 2 : 1;
    QueryOps<2> o;
    load_query_ops<2>(o, q, w, q_pos, r, nvalid, lane);
    const int jend = min(max(o.tpos[0], o.tpos[1]) + 1, max_ctx);  // never past ld_scores
    KeyTile cur, nxt;
    int jb = 0;
    if (jend > 0) fetch_key_tile(cur, kc, k_scale, seq, jb, jend, lane);
    for (; jb < jend; jb += 16) {
      if (jb + 16 < jend) fetch_key_tile(nxt, kc, k_scale, seq, jb + 16, jend, lane);
      score_key_tile<2>(o, cur, scores, ld_scores, jend, lane);
      cur = nxt;
    }
    r += nvalid;
  }
}

static_assert(kTopkChunkKeys % (kScanWaves * 64 * kScanPage) == 0, "a workgroup range never straddles a chunk");
static_assert(kScanWaves * 64 * kScanPage < 65536, "a workgroup's count per bin fits the 16-bit LDS counters");

int indexer_scan_rows_per_wave(RowSeq rs) { return (!rs.q_seq && rs.q_per_seq % 2 == 0) ? 2 : 1; }

hipError_t launch_indexer_scan(const uint8_t* q, const float* w, PagedCache kc, const float* k_scale,
                               RowSeq rs, const int32_t* q_pos, int rows, int max_ctx,
                               float* scores, int64_t ld_scores, uint32_t* hist0, hipStream_t stream) {
  // units of NQ query rows of one sequence; about 2048 waves (8 per CU) per launch for a decode
  // batch of two-row units, 1024 for one-row units (half the work per key, so twice the keys per
  // wave balance its fixed query load and ring fill), each a whole number of pages (at most 64)
  const int nq = indexer_scan_rows_per_wave(rs);
  const int units = rows / nq;
  const int64_t total = (int64_t)units * max_ctx;
  int kpw = (int)((total / (nq == 1 ? 1024 : 2048) + kScanPage - 1) / kScanPage * kScanPage);
  kpw = kpw < kScanPage ? kScanPage : (kpw > 64 * kScanPage ? 64 * kScanPage : kpw);
  // at least 8 ranges per row: in a causal prefill block the rows' prefixes differ in length, and
  // ranges as long as the row leave most of a workgroup's waves without keys
  while (kpw > kScanPage && 8 * kpw > max_ctx) kpw = kpw / 2 / kScanPage * kScanPage;  // whole pages
  if (hist0) {
    // counted per top-k chunk: a workgroup's range (4 kpw) must not straddle one, so kpw is a
    // power of two (64 .. 4096 keys) and 4 kpw divides the chunk
    int p2 = kScanPage;
    while (p2 < kpw) p2 *= 2;
    kpw = p2;
  }
  const int per_block = kScanWaves * kpw;
  dim3 grid((max_ctx + per_block - 1) / per_block, units);
  const dim3 block(64 * kScanWaves);
  if (nq == 1 && !hist0)
    hipLaunchKernelGGL((indexer_scan_kernel<1, false>), grid, block, 0, stream, q, w, kc, k_scale, rs, q_pos, kpw, max_ctx, scores, ld_scores, hist0);
  else if (nq == 1)
    hipLaunchKernelGGL((indexer_scan_kernel<1, true>), grid, block, 0, stream, q, w, kc, k_scale, rs, q_pos, kpw, max_ctx, scores, ld_scores, hist0);
  else if (!hist0)
    hipLaunchKernelGGL((indexer_scan_kernel<2, false>), grid, block, 0, stream, q, w, kc, k_scale, rs, q_pos, kpw, max_ctx, scores, ld_scores, hist0);
  else
    hipLaunchKernelGGL((indexer_scan_kernel<2, true>), grid, block, 0, stream, q, w, kc, k_scale, rs, q_pos, kpw, max_ctx, scores, ld_scores, hist0);
  return hipGetLastError();
}

hipError_t launch_indexer_prefill(const uint8_t* q, const float* w, PagedCache kc,
                                  const float* k_scale, RowSeq rs, const int32_t* q_pos, int rows,
                                  int max_ctx, float* scores, int64_t ld_scores, hipStream_t stream) {
  dim3 grid((rows + 7) / 8);
  hipLaunchKernelGGL(indexer_prefill_kernel, grid, dim3(256), 0, stream, q, w, kc, k_scale, rs, q_pos, rows, max_ctx, scores, ld_scores);
  return hipGetLastError();
}

}  // namespace dsa
