// proj.hip -- the Lightning Indexer's projections on gfx950, fused with the FP8 quantisation and
// the paged key-cache write.
//
// Page references:
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org), section
//               "Lightning Indexer", its figure's first step: the current token's hidden state h_t
//               gives the head weights w_t; the query path reuses the MLA query latent and applies
//               an indexer projection to get the n_h^I query heads q_{t,r}; every position's own
//               hidden state h_j gives one key k_j shared by all heads, kept in the Indexer Key Cache
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io): 64 indexer heads of 128 dims,
//               scored in FP8; the key cache stores 128 FP8 codes plus a float scale per token
//
// GEMMs C[M x N] = A[M x K] . B[N x K]^T with bf16 operands (both K-contiguous: the activations
// row-major, the weights in the [out, in] layout of a linear layer) on v_mfma_f32_32x32x16_bf16
// with fp32 accumulation, and three epilogues:
//   key    N = 128: per row (token) s = max|c| / 448 and codes E4M3(c / s), written to the token's
//          physical row of the paged key cache (the format dsa_indexer_cache_write writes)
//   query  codes E4M3(c) without a scale, row-major [M, N] bytes
//   f32    c as fp32, row-major [M, N]
// proj_gemm_kernel: 4 waves, a 128 x 128 output tile, K in blocks of 64; each wave owns four 32 x 32
// accumulator blocks (a 64 x 64 quarter of the tile, or for keys rows 32w..32w+31 and all 128
// columns, so that a row's scale stays within a wave). Within a block of 64 the K order is
// permuted the same way for both operands (lane half h supplies elements 32h + 8j .. +8 as its
// part of MFMA j), which leaves every dot product unchanged. The K blocks go straight from global
// memory into a ring of kPStages LDS stages (global_load_lds_dwordx4, no register staging), issued
// kPStages - 1 blocks ahead, one workgroup barrier per block; an LDS row of a block is its 128
// bytes, 16-byte chunk c of row r stored at c ^ (r % 8), so the operand reads of 8 consecutive
// rows hit distinct banks. Small batches (32-row tiles, and the split-K partials) stage through
// registers instead: the next block is loaded into registers while the current one is
// multiplied, LDS rows padded to 144 bytes. proj_query_big_kernel: query codes of large batches
// on 256 x 256 tiles with 8 waves, the same ring and swizzle.
#include "dsa_internal.h"

namespace dsa {

constexpr int kPM = 128, kPN = 128, kPK = 64;
constexpr int kPRowBytes = 2 * kPK + 16;                 // 144: padded LDS row of a K block
constexpr int kPStageBytes = 32 * kPN;                   // one wave's 32 x 128 byte codes
constexpr int kPStages = 2;                              // LDS stages of the 128-row tiles' ring
constexpr int kPBlockBytes = 2 * kPM * 2 * kPK;          // 32768: one K block of A and B

// kEpiPartial: fp32 sums over one K range (blockIdx.z) to ws[z][M][N], for the split-K path
enum { kEpiKey = 0, kEpiQuery = 1, kEpiF32 = 2, kEpiPartial = 3 };

struct ProjArgs {
  const uint16_t* a;  // [M, K] bf16
  const uint16_t* b;  // [N, K] bf16
  int M, N, K;
  // key epilogue
  const int32_t* seq;
  const int32_t* pos;
  int n_seq;
  PagedCache kc;
  uint8_t* k_cache;
  float* k_scale;
  // query / f32 epilogues
  uint8_t* q8;
  float* f32;
  // split-K: K range of blockIdx.z is [z * k_split, (z + 1) * k_split); partials in ws
  int k_split;
  float* ws;
  int tiles_m, tiles;  // output tiles (tiles_m row tiles x tiles / tiles_m column tiles)
};

// Workgroups are dispatched to the 8 XCDs round robin. The padded 1-D grid gives each XCD a
// contiguous range of tiles (tile_origin orders them), so the tiles that share operand panels run
// on one XCD and read them through its L2. -1 for the padding.
__device__ __forceinline__ int tile_of(const ProjArgs& p) {
  const int per = (int)gridDim.x >> 3;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  return t < p.tiles ? t : -1;
}
static inline dim3 tile_grid(int tiles, int z = 1) { return dim3(8 * ((tiles + 7) / 8), 1, z); }

// Tile t's first row and column. Tiles come in groups of 8 row tiles by all column tiles, row
// tiles fastest within a group: the workgroups an XCD runs at once then cover about 8 row tiles x
// 8 column tiles, each operand panel shared through its L2 eight ways.
__device__ __forceinline__ void tile_origin(const ProjArgs& p, int t, int tm, int* m0, int* n0, int tn = kPN) {
  constexpr int kGroup = 8;
  const int n_tiles = p.tiles / p.tiles_m;
  const int g = t / (kGroup * n_tiles), first = kGroup * g;
  const int gs = min(p.tiles_m - first, kGroup), r = t - g * kGroup * n_tiles;
  *m0 = (first + r % gs) * tm;
  *n0 = (r / gs) * tn;
}

// The K loop of a 128 x 128 tile over the whole K, through the LDS ring. Wave w moves rows
// 32w..32w+31 of both operands: four global_load_lds_dwordx4 per operand and block, each 8 rows x
// 128 bytes, lane l taking row 8i + l/8 and the global chunk (l % 8) ^ (l / 8), which lands at LDS
// chunk l % 8 of its row (the swizzle above). Rows past M or N re-read the last row; their results
// are never stored. The loads are inline asm (LDS address in M0, saved and restored), so their
// completion is awaited with explicit vmcnt counts: at block kb the wave's own loads of block kb
// are done once at most 8 (loads of one block) times the blocks issued after it are in flight;
// the barrier after that wait makes every wave's loads of the block visible and also frees the
// stage that the next issue overwrites (its last reader is the previous block's multiply).
// kSq: wave w owns rows 64 (w / 2) .. +63 and columns 64 (w % 2) .. +63 (acc[2 mi + ci]: rows
// 64 (w / 2) + 32 mi, columns 64 (w % 2) + 32 ci), so a K step reads 2 + 2 operands for 4 MFMAs;
// otherwise rows 32w .. +31 and all 128 columns (acc[cb]: columns 32 cb), 1 + 4 operands.
template <bool kSq>
__device__ __forceinline__ void gemm_loop_lds_ring(const ProjArgs& p, int m0, int n0, int wave, int lane,
                                                   uint8_t* smem, f32x16 (&acc)[4]) {
  const int hl = lane & 31, half = lane >> 5;
  const int nkb = p.K / kPK;
  const uint32_t k_bytes = 2u * (uint32_t)p.K;
  const uint32_t chunk = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const int max_ra = p.M - 1 - m0, max_rb = p.N - 1 - n0;
  uint32_t va[4], vb[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = 32 * wave + 8 * ii + (lane >> 3);
    va[ii] = (uint32_t)min(r, max_ra) * k_bytes + chunk;
    vb[ii] = (uint32_t)min(r, max_rb) * k_bytes + chunk;
  }
  const uint8_t* ga = (const uint8_t*)(p.a + (int64_t)m0 * p.K);
  const uint8_t* gb = (const uint8_t*)(p.b + (int64_t)n0 * p.K);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto issue = [&](int kb, int st) {
    const uint64_t sa = (uint64_t)(uintptr_t)(ga + 2 * kPK * kb), sb = (uint64_t)(uintptr_t)(gb + 2 * kPK * kb);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds0 + st * kPBlockBytes + 4096 * wave);
    const uint32_t lb = la + kPBlockBytes / 2;
    uint32_t sv;
    asm volatile(
        "s_mov_b32 %[sv], m0\n"
        "s_mov_b32 m0, %[la]\n s_nop 0\n global_load_lds_dwordx4 %[a0], %[sa]\n"
        "s_add_u32 m0, %[la], 1024\n s_nop 0\n global_load_lds_dwordx4 %[a1], %[sa]\n"
        "s_add_u32 m0, %[la], 2048\n s_nop 0\n global_load_lds_dwordx4 %[a2], %[sa]\n"
        "s_add_u32 m0, %[la], 3072\n s_nop 0\n global_load_lds_dwordx4 %[a3], %[sa]\n"
        "s_mov_b32 m0, %[lb]\n s_nop 0\n global_load_lds_dwordx4 %[b0], %[sb]\n"
        "s_add_u32 m0, %[lb], 1024\n s_nop 0\n global_load_lds_dwordx4 %[b1], %[sb]\n"
        "s_add_u32 m0, %[lb], 2048\n s_nop 0\n global_load_lds_dwordx4 %[b2], %[sb]\n"
        "s_add_u32 m0, %[lb], 3072\n s_nop 0\n global_load_lds_dwordx4 %[b3], %[sb]\n"
        "s_mov_b32 m0, %[sv]\n"
        : [sv] "=&s"(sv)
        : [sa] "s"(sa), [sb] "s"(sb), [la] "s"(la), [lb] "s"(lb), [a0] "v"(va[0]), [a1] "v"(va[1]),
          [a2] "v"(va[2]), [a3] "v"(va[3]), [b0] "v"(vb[0]), [b1] "v"(vb[1]), [b2] "v"(vb[2]), [b3] "v"(vb[3])
        : "scc", "memory");
  };
  // per-lane byte offsets of the four operand chunks 4 half + j of an LDS row (row % 8 = hl % 8)
  uint32_t co[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) co[j] = 16u * (uint32_t)((4 * half + j) ^ (hl & 7));
#pragma unroll
  for (int kb = 0; kb < kPStages - 1; ++kb)
    if (kb < nkb) issue(kb, kb);
  int st = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    // the wave's loads of block kb: done once those of later blocks are all that is in flight
    const int later = min(kPStages - 2, nkb - 1 - kb);
    if (later <= 0) __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0)
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    else __builtin_amdgcn_s_waitcnt(0x4F70);                  // vmcnt(16)
    __syncthreads();
    if (kb + kPStages - 1 < nkb) issue(kb + kPStages - 1, st == 0 ? kPStages - 1 : st - 1);
    const uint8_t* sa = smem + st * kPBlockBytes;
    const uint8_t* sb = sa + kPBlockBytes / 2;
    if constexpr (kSq) {
      const int wm = wave >> 1, wn = wave & 1;
      bf16x8 a[2][4], b[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a[i][j] = *(const bf16x8*)(sa + (64 * wm + 32 * i + hl) * 128 + co[j]);
          b[i][j] = *(const bf16x8*)(sb + (64 * wn + 32 * i + hl) * 128 + co[j]);
        }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ci = 0; ci < 2; ++ci)
            acc[2 * mi + ci] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi][j], b[ci][j], acc[2 * mi + ci], 0, 0, 0);
    } else {
      bf16x8 a[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = *(const bf16x8*)(sa + (32 * wave + hl) * 128 + co[j]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        bf16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)(sb + (32 * cb + hl) * 128 + co[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[cb], 0, 0, 0);
      }
    }
    st = st == kPStages - 1 ? 0 : st + 1;
  }
}

// kTM: rows per tile. 128: wave w owns a 64 x 64 quarter of the tile (query and fp32 outputs) or
// rows 32w.. and all 128 columns (keys, whose scale needs a whole row); 32 (small batches, so the
// grid covers the GPU): the 4 waves share the 32 rows and wave w owns columns 32w..32w+31.
template <int kEpi, int kTM>
__global__ void __launch_bounds__(256) proj_gemm_kernel(ProjArgs p) {
  static_assert(kTM == 128 || kTM == 32, "row tile");
  static_assert(kTM == 32 || kEpi != kEpiPartial, "split-K partials take 32-row tiles");
  constexpr int kCB = kTM == 128 ? 4 : 1;  // 32-column accumulator blocks per wave
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kTM == 128 ? kPStages * kPBlockBytes : (kTM + kPN) * kPRowBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane & 31, half = lane >> 5;
  const int tile = tile_of(p);
  if (tile < 0) return;
  int m0, n0;
  tile_origin(p, tile, kTM, &m0, &n0);
  const int kbeg = kEpi == kEpiPartial ? blockIdx.z * p.k_split : 0;
  const int kend = kEpi == kEpiPartial ? min(p.K, kbeg + p.k_split) : p.K;
  constexpr bool kSq = kTM == 128 && kEpi != kEpiKey;
  const int wrow = kTM == 128 ? 32 * wave : 0;       // first row of the wave's stored rows
  const int wcb0 = kTM == 128 ? 0 : wave;            // the wave's first column block (not kSq)
  // accumulator block k: its first row and column within the tile
  auto blk_row = [&](int k) { return kSq ? 64 * (wave >> 1) + 32 * (k >> 1) : wrow; };
  auto blk_col = [&](int k) { return kSq ? 64 * (wave & 1) + 32 * (k & 1) : 32 * (wcb0 + k); };
  uint8_t* lds_a = smem;
  uint8_t* lds_b = smem + kTM * kPRowBytes;

  // global -> register staging: thread tid moves chunks c = tid + 256 i (i < 4) of each operand's
  // 128 rows x 128 bytes (row c / 8, 16-byte chunk c % 8); rows past M or N load zeros
  // (A: kTM rows, so kTM / 32 chunks per thread; B: 128 rows, 4 chunks per thread). The query's
  // 32-row tiles (one workgroup per CU at decode sizes) keep kDepth K blocks in flight in
  // registers: a block's multiply is a few MFMAs, far shorter than its load, so one block of
  // lookahead leaves the loop waiting on memory. The split-K partials run several workgroups per
  // CU, which hide the loads instead, and keep the registers for that occupancy.
  constexpr int kAC = kTM / 32;
  constexpr int kDepth = kTM == 32 && kEpi == kEpiQuery ? 6 : 1;
  i32x4 ra[kDepth][kAC], rb[kDepth][4];
  auto load_block = [&](int k0, int s) {
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      ra[s][i] = (m0 + row < p.M) ? *(const i32x4*)(p.a + (int64_t)(m0 + row) * p.K + k0 + 8 * ch) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      rb[s][i] = (n0 + row < p.N) ? *(const i32x4*)(p.b + (int64_t)(n0 + row) * p.K + k0 + 8 * ch) : i32x4{0, 0, 0, 0};
    }
  };
  auto store_block = [&](int s) {
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *(i32x4*)(lds_a + row * kPRowBytes + 16 * ch) = ra[s][i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
      *(i32x4*)(lds_b + row * kPRowBytes + 16 * ch) = rb[s][i];
    }
  };

  f32x16 acc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = f32x16{};
  if constexpr (kTM == 128) {
    gemm_loop_lds_ring<kSq>(p, m0, n0, wave, lane, smem, acc);
  } else {
  // block k0 + s kPK sits in register slot s (mod kDepth); each slot is refilled with the block
  // kDepth blocks later as soon as it is in LDS
#pragma unroll
  for (int s = 0; s < kDepth; ++s)
    if (kbeg + s * kPK < kend) load_block(kbeg + s * kPK, s);
  for (int k00 = kbeg; k00 < kend; k00 += kDepth * kPK) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      const int k0 = k00 + s * kPK;
      if (k0 < kend) {  // uniform
        __syncthreads();  // the previous block's operand reads are done
        store_block(s);
        __syncthreads();
        if (k0 + kDepth * kPK < kend) load_block(k0 + kDepth * kPK, s);
        bf16x8 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *(const bf16x8*)(lds_a + (wrow + hl) * kPRowBytes + 64 * half + 16 * j);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          bf16x8 b[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            b[j] = *(const bf16x8*)(lds_b + (32 * (wcb0 + cb) + hl) * kPRowBytes + 64 * half + 16 * j);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc[cb], 0, 0, 0);
        }
      }
    }
  }
  }

  // acc[cb][e]: row blk_row(cb) + 8 (e / 4) + 4 half + e % 4 of the tile, column blk_col(cb) + hl
  if (kEpi == kEpiF32 || kEpi == kEpiPartial) {
    float* dst = kEpi == kEpiF32 ? p.f32 : p.ws + (int64_t)blockIdx.z * p.M * p.N;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int n = n0 + blk_col(cb) + hl;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + blk_row(cb) + 8 * (e >> 2) + 4 * half + (e & 3);
        if (m < p.M && n < p.N) dst[(int64_t)m * p.N + n] = acc[cb][e];
      }
    }
    return;
  }
  // Coded epilogues: the tile's codes staged as [row][128] bytes in LDS (the operand tiles are
  // done), each wave writing its accumulator blocks; then wave w stores rows 32w..32w+31
  // (128-row tiles) or the block stores the 32 rows (32-row tiles, query only).
  static_assert(kEpi != kEpiKey || kTM == 128, "the key epilogue takes 128-row tiles");
  __syncthreads();
  uint8_t* stage = smem + (kTM == 128 ? wave * kPStageBytes : 0);
  float sc[16];  // key epilogue: the row's scale s (the code is E4M3(c / s), an IEEE division)
#pragma unroll
  for (int e = 0; e < 16; ++e) sc[e] = 1.f;
  if (kEpi == kEpiKey) {
    // per row: the largest |c| over its 128 columns (4 blocks in this lane, 32 lanes of its half)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float m = 0.f;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) m = fmaxf(m, fabsf(acc[cb][e]));
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      sc[e] = m / 448.0f;
    }
  }
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * half + (e & 3);
      uint32_t code;
      if (kEpi == kEpiKey) code = sc[e] > 0.f ? e4m3_rne_sat(acc[cb][e] / sc[e]) : 0u;
      else code = e4m3_rne_sat(acc[cb][e]);
      smem[(blk_row(cb) + r) * kPN + blk_col(cb) + hl] = (uint8_t)code;
    }
  __syncthreads();
  // 32 rows x 8 chunks of 16 bytes: 4 per lane of each wave (128-row tiles) or 1 per thread
  constexpr int kStores = kTM == 128 ? 4 : 1;
#pragma unroll
  for (int i = 0; i < kStores; ++i) {
    const int c = kTM == 128 ? lane + 64 * i : tid, r = c >> 3, ch = c & 7;
    const int m = m0 + wrow + r;
    if (m >= p.M) continue;
    const i32x4 v = *(const i32x4*)(stage + r * kPN + 16 * ch);
    if (kEpi == kEpiQuery) {
      if (n0 + 16 * ch < p.N) *(i32x4*)(p.q8 + (int64_t)m * p.N + n0 + 16 * ch) = v;
    } else {
      const int sq = p.seq[m];
      const int64_t row = (sq >= 0 && sq < p.n_seq)
                              ? phys_row(p.kc.page_table, p.kc.ld_pt, p.kc.page_size, p.kc.num_pages, sq, p.pos[m])
                              : -1;
      if (row >= 0) *(i32x4*)(p.k_cache + row * 128 + 16 * ch) = v;
    }
  }
  if (kEpi == kEpiKey && hl == 0) {
    // the lane of each half that holds column 0 writes its rows' scales
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wrow + 8 * (e >> 2) + 4 * half + (e & 3);
      if (m >= p.M) continue;
      const int sq = p.seq[m];
      const int64_t row = (sq >= 0 && sq < p.n_seq)
                              ? phys_row(p.kc.page_table, p.kc.ld_pt, p.kc.page_size, p.kc.num_pages, sq, p.pos[m])
                              : -1;
      if (row >= 0) p.k_scale[row] = sc[e];
    }
  }
}

// The split-K path's second step: the kz partial blocks ws[z][M][N] summed in order of z, then the
// key epilogue (N = 128: 16 lanes per token, 8 columns per lane) or fp32 stores.
template <int kEpi>
__global__ void __launch_bounds__(256) proj_reduce_kernel(ProjArgs p, int kz) {
  const int64_t MN = (int64_t)p.M * p.N;
  if (kEpi == kEpiF32) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float sum = 0.f;
    for (int z0 = 0; z0 < kz; z0 += 4) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = z0 + u < kz ? p.ws[(z0 + u) * MN + i] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u < kz) sum += v[u];
    }
    p.f32[i] = sum;
    return;
  }
  static_assert(kEpi == kEpiKey || kEpi == kEpiF32, "reduce epilogues");
  const int j = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = t < p.M;
  const int tc = live ? t : p.M - 1;  // idle groups re-read the last token and store nothing
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < kz; z0 += 4) {
    // four partial blocks' loads issued together, then added in order of z
    float4 a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int z = z0 + u < kz ? z0 + u : kz - 1;
      const float4* src = (const float4*)(p.ws + z * MN + (int64_t)tc * 128 + 8 * j);
      a[u] = src[0];
      b[u] = src[1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (z0 + u >= kz) break;
      x[0] += a[u].x; x[1] += a[u].y; x[2] += a[u].z; x[3] += a[u].w;
      x[4] += b[u].x; x[5] += b[u].y; x[6] += b[u].z; x[7] += b[u].w;
    }
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));  // within the 16-lane group
  const int sq = p.seq[tc];
  const int64_t row = live && sq >= 0 && sq < p.n_seq
                          ? phys_row(p.kc.page_table, p.kc.ld_pt, p.kc.page_size, p.kc.num_pages, sq, p.pos[tc])
                          : -1;
  if (row < 0) return;
  const float s = m / 448.0f;
  uint32_t lo = 0, hi = 0;
  if (s > 0.f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo |= e4m3_rne_sat(x[e] / s) << (8 * e);
      hi |= e4m3_rne_sat(x[4 + e] / s) << (8 * e);
    }
  }
  ((uint2*)(p.k_cache + row * 128))[j] = make_uint2(lo, hi);
  if (j == 0) p.k_scale[row] = s;
}

// Query codes of prefill-sized batches: 8 waves, a 256 x 256 output tile, K blocks of 64 in a
// two-stage LDS ring (64 KB a stage, one workgroup per CU), loaded and swizzled as in
// gemm_loop_lds_ring (wave w moves rows 32w..32w+31 of each operand). Wave w owns rows
// 64 (w / 2) .. +63 and columns 128 (w % 2) .. +127 (acc[4 mi + ci]: rows 64 (w / 2) + 32 mi,
// columns 128 (w % 2) + 32 ci), so a K step reads 2 + 4 operands for 8 MFMAs; and a K block
// loads 64 KB for 8.4 MFLOP, half the bytes per FLOP of a 128 x 128 tile, whose loop is bound by
// its loads' issue. The codes are staged as [row][256] bytes in LDS and stored 16 bytes a lane.
constexpr int kBT = 256;                       // tile edge
constexpr int kBStage = 2 * kBT * 2 * kPK;     // 65536: one K block of A and B
__global__ void __launch_bounds__(512) proj_query_big_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * kBStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane & 31, half = lane >> 5;
  const int tile = tile_of(p);
  if (tile < 0) return;
  int m0, n0;
  tile_origin(p, tile, kBT, &m0, &n0, kBT);
  const int nkb = p.K / kPK;
  const uint32_t k_bytes = 2u * (uint32_t)p.K;
  const uint32_t chunk = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const int max_ra = p.M - 1 - m0, max_rb = p.N - 1 - n0;
  uint32_t va[4], vb[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int r = 32 * wave + 8 * ii + (lane >> 3);
    va[ii] = (uint32_t)min(r, max_ra) * k_bytes + chunk;
    vb[ii] = (uint32_t)min(r, max_rb) * k_bytes + chunk;
  }
  const uint8_t* ga = (const uint8_t*)(p.a + (int64_t)m0 * p.K);
  const uint8_t* gb = (const uint8_t*)(p.b + (int64_t)n0 * p.K);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  auto issue = [&](int kb, int st) {
    const uint64_t sa = (uint64_t)(uintptr_t)(ga + 2 * kPK * kb), sb = (uint64_t)(uintptr_t)(gb + 2 * kPK * kb);
    const uint32_t la = __builtin_amdgcn_readfirstlane(lds0 + st * kBStage + 4096 * wave);
    const uint32_t lb = la + kBStage / 2;
    uint32_t sv;
    asm volatile(
        "s_mov_b32 %[sv], m0\n"
        "s_mov_b32 m0, %[la]\n s_nop 0\n global_load_lds_dwordx4 %[a0], %[sa]\n"
        "s_add_u32 m0, %[la], 1024\n s_nop 0\n global_load_lds_dwordx4 %[a1], %[sa]\n"
        "s_add_u32 m0, %[la], 2048\n s_nop 0\n global_load_lds_dwordx4 %[a2], %[sa]\n"
        "s_add_u32 m0, %[la], 3072\n s_nop 0\n global_load_lds_dwordx4 %[a3], %[sa]\n"
        "s_mov_b32 m0, %[lb]\n s_nop 0\n global_load_lds_dwordx4 %[b0], %[sb]\n"
        "s_add_u32 m0, %[lb], 1024\n s_nop 0\n global_load_lds_dwordx4 %[b1], %[sb]\n"
        "s_add_u32 m0, %[lb], 2048\n s_nop 0\n global_load_lds_dwordx4 %[b2], %[sb]\n"
        "s_add_u32 m0, %[lb], 3072\n s_nop 0\n global_load_lds_dwordx4 %[b3], %[sb]\n"
        "s_mov_b32 m0, %[sv]\n"
        : [sv] "=&s"(sv)
        : [sa] "s"(sa), [sb] "s"(sb), [la] "s"(la), [lb] "s"(lb), [a0] "v"(va[0]), [a1] "v"(va[1]),
          [a2] "v"(va[2]), [a3] "v"(va[3]), [b0] "v"(vb[0]), [b1] "v"(vb[1]), [b2] "v"(vb[2]), [b3] "v"(vb[3])
        : "scc", "memory");
  };
  uint32_t co[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) co[j] = 16u * (uint32_t)((4 * half + j) ^ (hl & 7));
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  issue(0, 0);
  int st = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    // the wave's loads of block kb are the only ones in flight; the barrier then makes every
    // wave's visible and frees the other stage (its last reader was the previous block)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    const uint8_t* sa = smem + st * kBStage;
    const uint8_t* sb = sa + kBStage / 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8*)(sa + (64 * wm + 32 * i + hl) * 128 + co[j]);
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = *(const bf16x8*)(sb + (128 * wn + 32 * c + hl) * 128 + co[j]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[4 * i + c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[c], acc[4 * i + c], 0, 0, 0);
    }
    st ^= 1;
  }
  // codes staged [row][256] in LDS (the ring is done once every wave passes the barrier)
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
        smem[r * kBT + 128 * wn + 32 * c + hl] = (uint8_t)e4m3_rne_sat(acc[4 * i + c][e]);
      }
  __syncthreads();
  // wave w stores rows 32w..32w+31: 16 chunks of 16 bytes a row, 8 a lane
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = lane + 64 * i, r = c >> 4, ch = c & 15;
    const int m = m0 + 32 * wave + r;
    if (m >= p.M || n0 + 16 * ch >= p.N) continue;
    *(i32x4*)(p.q8 + (int64_t)m * p.N + n0 + 16 * ch) = *(const i32x4*)(smem + (32 * wave + r) * kBT + 16 * ch);
  }
}

// Split-K is taken when the unsplit launch (128-row tiles) would give fewer than two workgroups
// per CU: the K blocks of 64 are dealt out over 32-row tiles so that about 1024 workgroups run
// (a projection of a few thousand rows onto 64 or 128 columns over d = 7168 otherwise runs on a
// few dozen CUs). Returns the number of K ranges and sets *k_split (a multiple of 64); 1 means
// no split.
static int proj_plan(int M, int N, int K, int* k_split) {
  const int n_tiles = (N + kPN - 1) / kPN;
  const int tiles = ((M + 31) / 32) * n_tiles;
  const int kb = K / kPK;
  *k_split = K;
  if (((M + kPM - 1) / kPM) * n_tiles >= 512 || kb < 2) return 1;
  int want = 1024 / tiles < kb ? 1024 / tiles : kb;
  want = want > 16 ? 16 : want;  // at most 16 partial blocks: their write and re-read stay small
  if (want < 2) return 1;
  const int per = (kb + want - 1) / want;  // K blocks per range
  *k_split = per * kPK;
  return (kb + per - 1) / per;
}

size_t proj_ws_bytes(int M, int N, int K) {
  int ks = 0;
  const int kz = proj_plan(M, N, K, &ks);
  return kz > 1 ? (size_t)kz * M * N * 4 : 0;
}

hipError_t launch_indexer_key_project(const uint16_t* h, const uint16_t* w_k, int n_tok, int d, int n_seq,
                                      const int32_t* seq, const int32_t* pos, PagedCache kc, uint8_t* k_cache,
                                      float* k_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  ProjArgs p{};
  p.a = h; p.b = w_k; p.M = n_tok; p.N = 128; p.K = d;
  p.seq = seq; p.pos = pos; p.n_seq = n_seq; p.kc = kc; p.k_cache = k_cache; p.k_scale = k_scale;
  int ks = 0;
  const int kz = proj_plan(n_tok, 128, d, &ks);
  if (kz > 1 && ws && ws_bytes >= proj_ws_bytes(n_tok, 128, d)) {
    p.k_split = ks; p.ws = (float*)ws;
    p.tiles_m = (n_tok + 31) / 32; p.tiles = p.tiles_m;
    hipLaunchKernelGGL((proj_gemm_kernel<kEpiPartial, 32>), tile_grid(p.tiles, kz), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(proj_reduce_kernel<kEpiKey>, dim3((n_tok + 15) / 16), dim3(256), 0, stream, p, kz);
    return hipGetLastError();
  }
  p.tiles_m = (n_tok + kPM - 1) / kPM; p.tiles = p.tiles_m;
  hipLaunchKernelGGL((proj_gemm_kernel<kEpiKey, 128>), tile_grid(p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_indexer_query_project(const uint16_t* c_q, const uint16_t* w_q, const uint16_t* h,
                                        const uint16_t* w_w, int rows, int d_cq, int d, int n_q, int n_w, uint8_t* q8,
                                        float* w, void* ws, size_t ws_bytes, hipStream_t stream) {
  ProjArgs p{};
  p.a = c_q; p.b = w_q; p.M = rows; p.N = n_q; p.K = d_cq; p.q8 = q8;
  // small batches take 32-row tiles, so that the column tiles spread over the GPU; batches that
  // give every CU a 256 x 256 tile take those
  const int big_tiles = ((rows + kBT - 1) / kBT) * ((n_q + kBT - 1) / kBT);
  const int tm = rows <= 512 ? 32 : kPM;
  p.tiles_m = (rows + tm - 1) / tm; p.tiles = p.tiles_m * ((n_q + kPN - 1) / kPN);
  if (big_tiles >= 256) {
    p.tiles_m = (rows + kBT - 1) / kBT; p.tiles = big_tiles;
    hipLaunchKernelGGL(proj_query_big_kernel, tile_grid(p.tiles), dim3(512), 0, stream, p);
  } else if (tm == 32)
    hipLaunchKernelGGL((proj_gemm_kernel<kEpiQuery, 32>), tile_grid(p.tiles), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((proj_gemm_kernel<kEpiQuery, 128>), tile_grid(p.tiles), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ProjArgs pw{};
  pw.a = h; pw.b = w_w; pw.M = rows; pw.N = n_w; pw.K = d; pw.f32 = w;
  int ks = 0;
  const int kz = proj_plan(rows, n_w, d, &ks);
  if (kz > 1 && ws && ws_bytes >= proj_ws_bytes(rows, n_w, d)) {
    pw.k_split = ks; pw.ws = (float*)ws;
    pw.tiles_m = (rows + 31) / 32; pw.tiles = pw.tiles_m * ((n_w + kPN - 1) / kPN);
    hipLaunchKernelGGL((proj_gemm_kernel<kEpiPartial, 32>), tile_grid(pw.tiles, kz), dim3(256), 0, stream, pw);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)rows * n_w;
    hipLaunchKernelGGL(proj_reduce_kernel<kEpiF32>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, pw, kz);
    return hipGetLastError();
  }
  pw.tiles_m = (rows + kPM - 1) / kPM; pw.tiles = pw.tiles_m * ((n_w + kPN - 1) / kPN);
  hipLaunchKernelGGL((proj_gemm_kernel<kEpiF32, 128>), tile_grid(pw.tiles), dim3(256), 0, stream, pw);
  return hipGetLastError();
}

}  // namespace dsa
