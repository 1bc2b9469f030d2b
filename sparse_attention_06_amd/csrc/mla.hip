// mla.hip -- attention over a position set on gfx950: sparse (S_t from top-k) and dense causal.
//
// Page references:
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org),
//               section "Sparse Attention": softmax(QK^T/sqrt(d_h) + M^DSA)V, where M is 0 on S_t
//               and -inf elsewhere, computed by reading only the indexed rows (no full logits)
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io): absorbed MLA, 128 heads share one
//               latent row of 512 + 64 bf16 per position as key; its first 512 columns are the value
//
// Tuned kernel (H=128, Dqk=576, Dv=512): one workgroup = 4 waves per (row, split); wave w owns
// heads [32w, 32w+32). Per tile of 32 selected positions:
//   gather   the 32 latent rows (1152 B each) go straight from HBM into LDS with
//            global_load_lds_dwordx4 (no VGPR staging), two tiles in flight; each latent row's
//            16-byte chunks are rotated within a 1280-byte line so both LDS read patterns below
//            are bank-conflict free
//   QK^T     S[32 keys x 32 heads] on v_mfma_f32_32x32x16_bf16: the key tile is the A operand
//            (read from LDS), the wave's 32 query heads the B operand (latent dims resident in
//            128 VGPRs, rope dims from LDS)
//   softmax  fp32, in the log2 domain, with a lazily moved reference maximum: the running
//            output is rescaled only when a head's maximum grows by more than 2^8
//   PV       O^T[512 x 32 heads] += V^T P: the probabilities stay in registers as the B operand
//            (the QK^T output layout is reused with a matching permutation of the key order);
//            V^T comes from LDS through ds_read_b64_tr_b16 transpose reads; O^T lives in 256
//            accumulator registers per lane
// A split variant spreads one row's set over several workgroups (small decode batches) and a
// combine kernel merges the partial (o, lse) pairs.
#include "dsa_internal.h"

namespace dsa {

// ------------------------------------------------------------------ index sets

// S_t is a set ([DSA-blog] "Sparse Attention": M_tj = 0 exactly when j is in S_t), so a position
// listed more than once is attended once. A list whose visible entries (0 <= j <= t) run strictly
// ascending from entry 0 -- what the top-k writes -- cannot repeat one, and needs no filtering.
// This checks entries e = e0, e0 + stride, ... below e_end (e0 >= 1) against that form: true if
// one of them is visible while the entry before it is not visible or not smaller.
__device__ __forceinline__ bool list_needs_dedupe(const int* irow, int t, int e0, int e_end, int stride) {
  bool bad = false;
  for (int e = e0; e < e_end; e += stride) {
    const int c = irow[e], p = irow[e - 1];
    const bool vc = c >= 0 && c <= t, vp = p >= 0 && p <= t;
    bad |= vc && !(vp && p < c);
  }
  return bad;
}

// ------------------------------------------------------------------ generic (any shape)

// One wave per (row, head); lanes stride the feature dims. Online softmax in fp32.
__global__ void __launch_bounds__(256) mla_generic_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= a.rows * a.H) return;
  const int r = gw / a.H, h = gw % a.H;
  const int t = a.q_pos[r], seq = a.rs.of(r);
  const uint16_t* qh = a.q + ((int64_t)r * a.H + h) * a.Dqk;
  float qv[16], o[8];
#pragma unroll
  for (int i = 0; i < 16; ++i) { int c = lane + 64 * i; qv[i] = c < a.Dqk ? bf16_to_f32(qh[c]) : 0.f; }
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int n = a.idx ? a.k : min(t + 1, a.k);  // dense: a.k = max_ctx
  const uint16_t* kv = (const uint16_t*)a.kv.base;
  // S_t is a set: a position the list repeats counts once. A list whose visible entries run
  // strictly ascending from entry 0 (the top-k's output) holds no repeat; any other list has each
  // entry checked against the entries before it.
  const int* irow = a.idx ? a.idx + (int64_t)r * a.ld_idx : nullptr;
  const bool dedupe = irow && __any(list_needs_dedupe(irow, t, 1 + lane, n, 64));
  for (int e = 0; e < n; ++e) {
    const int j = irow ? irow[e] : e;
    if (j < 0 || j > t) continue;
    if (dedupe) {
      bool seen = false;
      for (int e2 = lane; e2 < e; e2 += 64) seen |= irow[e2] == j;
      if (__any(seen)) continue;
    }
    const int64_t row = phys_row(a.kv.page_table, a.kv.ld_pt, a.kv.page_size, a.kv.num_pages, seq, j);
    if (row < 0) continue;
    const uint16_t* kr = kv + row * a.kv_dim;
    float d = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { int c = lane + 64 * i; if (c < a.Dqk) d = fmaf(qv[i], bf16_to_f32(kr[c]), d); }
    const float logit = wave_sum(d) * a.sm_scale;
    const float mn = fmaxf(m, logit);
    const float alpha = __expf(m - mn), p = __expf(logit - mn);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < 8; ++i) { int c = lane + 64 * i; o[i] = o[i] * alpha + (c < a.Dv ? p * bf16_to_f32(kr[a.v_col0 + c]) : 0.f); }
    m = mn;
  }
  uint16_t* out = a.out + ((int64_t)r * a.H + h) * a.Dv;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) { int c = lane + 64 * i; if (c < a.Dv) out[c] = f32_to_bf16(o[i] * inv); }
  if (a.lse && lane == 0) a.lse[(int64_t)r * a.H + h] = l > 0.f ? m + __logf(l) : -INFINITY;
}

hipError_t launch_mla_generic(const AttnArgs& a, hipStream_t stream) {
  const int waves = a.rows * a.H;
  hipLaunchKernelGGL(mla_generic_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tuned MFMA kernel

constexpr int kH = 128, kDqk = 576, kDv = 512;
constexpr int kNK = 32;                          // positions per tile
constexpr int kRowBytes = kDqk * 2;              // 1152 = 1024 latent + 128 rope
constexpr int kLatBytes = 1024;                  // dims 0..511: one wave-wide 16-byte load
constexpr int kLatStride = 1280;                 // LDS line of a latent row: 1 KB + rotation room
constexpr int kRopeBytes = 128;                  // dims 512..575: 8 chunks of 16 bytes
constexpr int kRopeOff = kNK * kLatStride;       // 40960: rope region of a tile
constexpr int kTileBytes = kRopeOff + kNK * kRopeBytes;  // 45056
constexpr int kRowsPerWave = kNK / 4;            // 8 rows gathered by each wave
constexpr int kInstrPerWave = kRowsPerWave + 1;  // 8 latent loads + 1 rope load
constexpr int kNBuf = 3;                         // tile buffers: kNBuf - 1 tiles in flight
static_assert(kNBuf >= 2 && kNBuf <= 4, "wait_gathers covers up to two younger tiles");
constexpr int kListCap = 2048;                   // resolved entries held in LDS at a time
constexpr int kListOff = kNBuf * kTileBytes;
constexpr int kQRopeOff = kListOff + 4 * kListCap; // rope dims of the 128 query heads (16 KB)
constexpr int kMaskOff = kQRopeOff + kH * kRopeBytes; // valid-entry mask per tile of the list
constexpr int kFlagOff = kMaskOff + 4 * (kListCap / kNK);  // one flag per wave
constexpr int kLdsBytes = kFlagOff + 16;
// Positions per pass of the repeat filter: a bitmap of 128 KB in the tile buffers, which are idle
// while a list chunk is resolved.
constexpr int kDedupWindow = 1 << 20;
// Staged prologue: an index row of at most kListCap entries and a page-table row of at most
// kStagePages pages are copied to the start of the tile buffers before any gather is issued.
constexpr int kStagePages = 2048;
static_assert(kDedupWindow / 8 <= kNBuf * kTileBytes, "repeat filter bitmap in the tile buffers");
static_assert(4 * (kListCap + kStagePages) <= kTileBytes, "staged index and page-table rows in tile buffer 0");
static_assert(kH * kDv * 2 <= kLdsBytes, "output staging");
static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
constexpr float kLog2e = 1.4426950408889634f;
// The softmax reference of a head moves only when a logit exceeds it by 2^64 (log2 units):
// fp32 and bf16 share an exponent range of 2^+-126, so probabilities up to 2^64 and sums of
// 2048 of them times |v| stay finite, and terms far below the reference are negligible anyway.
constexpr float kRescaleThreshold = 64.0f;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// LDS layout of a tile. Latent row r (1 KB) starts 16 * lat_rot(r) bytes into its 1280-byte line,
// i.e. its 16-byte chunks are rotated over the 64 banks (4 bytes each): lat_rot is a permutation
// of 0..15 over any 16 consecutive rows (the 16 rows of a QK^T operand fetch hit distinct banks)
// and steps by 4 chunks across each aligned group of 4 rows (the 4 rows x 32 bytes served
// together in a PV transpose read hit distinct banks). The lane offsets of both operand fetches
// are then one base per lane plus immediates. Rope part: 128-byte rows, row r keeps chunk c
// (0..7) at c ^ rope_swz(r).
__device__ __forceinline__ int lat_rot(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// A wave-uniform 64-bit value, placed in scalar registers. readfirstlane returns int: each half
// goes through uint32_t so that the low half is zero-extended, not sign-extended into the high.
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | lo;
}

// This wave's share of one tile gather: latent rows 4i + w (i = 0..7), each one wave-wide
// 16-byte-per-lane global -> LDS load (global_load_lds_dwordx4) of the row's 1 KB into its rotated
// line, and the rope chunks of rows 8w..8w+7 (lane l: row 8w + l/8, chunk (l%8) ^ rope_swz(row))
// in one more load. Returns the tile's valid-entry mask; loads nothing when it is 0. Otherwise
// every lane is active in every load, so each wave has exactly kInstrPerWave loads in flight per
// tile. The row ids come from the tile's entries (read from LDS an iteration ahead) through
// v_readlane. The loads are issued from inline asm so that the compiler's wait-count pass does
// not treat their LDS writes as aliasing every later LDS read; the tile loop waits for them
// explicitly. M0 is saved and restored.
struct TileEntries {
  int ent;     // entry lane%32 of the tile
  int my_ent;  // entry 8w + lane/8, whose rope chunk this lane loads
  int mask;    // valid-entry mask of the tile (same in every lane)
};
// The tile's entries after the list pass below: every entry of a tile with a nonzero mask is a
// row id (invalid ones replaced by a valid row of the same tile).
__device__ __forceinline__ TileEntries read_entries(const int* list, const int* tmask, int t, int ntiles, int wave, int lane) {
  // opaque lane id: the addresses are recomputed here (two VALU ops) rather than kept live
  // across the tile loop, where the register file is full
  asm volatile("" : "+v"(lane));
  if (t >= ntiles) return TileEntries{0, 0, 0};
  const int* tl = list + t * kNK;
  return TileEntries{tl[lane & 31], tl[kRowsPerWave * wave + (lane >> 3)], tmask[t]};
}
__device__ __forceinline__ uint32_t issue_tile(const uint8_t* __restrict__ kv_base, lds_u8* buf,
                                               TileEntries te, int wave, int lane) {
  // An opaque copy of the lane id: the per-lane values below are recomputed per tile (a few VALU
  // ops) instead of being hoisted out of the tile loop into long-lived registers.
  asm volatile("" : "+v"(lane));
  const uint32_t vmask = (uint32_t)__builtin_amdgcn_readfirstlane(te.mask);
  if (vmask == 0u) return 0u;
  // latent row 4i + w: one 64-bit per-lane address (row start + 16 * lane) per load
  const uint8_t* kvl = kv_base + 16 * lane;
  uint64_t ad[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const uint32_t rid = (uint32_t)__builtin_amdgcn_readlane(te.ent, 4 * i + wave);
    ad[i] = (uint64_t)(uintptr_t)(kvl + (uint64_t)rid * kRowBytes);
  }
  // row 4i + w starts 16 * lat_rot(4i + w) = 16 * (4w + i%4) bytes into its line (4i + w) * 1280
  const uint32_t lat_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)buf + wave * (kLatStride + 64));
  const uint32_t rope_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(buf + kRopeOff + kRowsPerWave * wave * kRopeBytes));
  const int my_slot = kRowsPerWave * wave + (lane >> 3);
  const uint64_t rope_src = (uint64_t)(uintptr_t)(kv_base + (int64_t)te.my_ent * kRowBytes + kLatBytes + 16 * ((lane & 7) ^ rope_swz(my_slot)));
  uint32_t sv;
  asm volatile(
      "s_mov_b32 %[sv], m0\n"
      "s_add_u32 m0, %[lm0], 0\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a0], off\n"
      "s_add_u32 m0, %[lm0], 5136\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a1], off\n"
      "s_add_u32 m0, %[lm0], 10272\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a2], off\n"
      "s_add_u32 m0, %[lm0], 15408\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a3], off\n"
      "s_add_u32 m0, %[lm0], 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a4], off\n"
      "s_add_u32 m0, %[lm0], 25616\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a5], off\n"
      "s_add_u32 m0, %[lm0], 30752\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a6], off\n"
      "s_add_u32 m0, %[lm0], 35888\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[a7], off\n"
      "s_mov_b32 m0, %[rm0]\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %[rsrc], off\n"
      "s_mov_b32 m0, %[sv]\n"
      : [sv] "=&s"(sv)
      : [a0] "v"(ad[0]), [a1] "v"(ad[1]), [a2] "v"(ad[2]), [a3] "v"(ad[3]), [a4] "v"(ad[4]), [a5] "v"(ad[5]), [a6] "v"(ad[6]), [a7] "v"(ad[7]), [lm0] "s"(lat_m0), [rm0] "s"(rope_m0), [rsrc] "v"(rope_src)
      : "memory");
  return vmask;
}
static_assert(kLatStride * 4 == 5120, "latent row 4i + w lies 5120*i bytes after row w");

// Wait until this wave's loads of the oldest tile in flight have landed, leaving the loads of
// `younger` later tiles in flight (each tile is kInstrPerWave loads per wave, issued in order).
__device__ __forceinline__ void wait_gathers(int younger) {
  // s_waitcnt immediate: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and lgkmcnt
  // left at their maxima (no wait)
  constexpr int kBase = 0x0F70;
  if (younger >= 2) __builtin_amdgcn_s_waitcnt(kBase | ((2 * kInstrPerWave) & 15) | (((2 * kInstrPerWave) >> 4) << 14));
  else if (younger == 1) __builtin_amdgcn_s_waitcnt(kBase | (kInstrPerWave & 15) | ((kInstrPerWave >> 4) << 14));
  else __builtin_amdgcn_s_waitcnt(kBase);
}

// list_needs_dedupe over this workgroup's entries [e0, e_end) (e0 >= 1), eight per thread at a
// time with all their loads issued together; true in every thread if any entry fails. flags:
// four ints of LDS.
__device__ __forceinline__ bool block_needs_dedupe(const int* irow, int t, int e0, int e_end, int* flags, int wave,
                                                   int lane) {
  bool bad = false;
  for (int b0 = e0 + (int)threadIdx.x; b0 < e_end; b0 += 8 * 256) {
    int c[8], p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = b0 + 256 * u;
      c[u] = e < e_end ? irow[e] : -1;
      p[u] = e < e_end ? irow[e - 1] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool vc = c[u] >= 0 && c[u] <= t, vp = p[u] >= 0 && p[u] <= t;
      bad |= vc && !(vp && p[u] < c[u]);
    }
  }
  const bool any = __any(bad);
  if (lane == 0) flags[wave] = any ? 1 : 0;
  __syncthreads();
  return (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
}

// The repeat filter: list[e - cb] = -1 for every entry e of [cb, ce) whose position an entry
// listed before it (anywhere in the row, so across splits too) also holds. One window of
// kDedupWindow positions at a time, as a bitmap in LDS (bm, idle tile buffers): the row's entries
// before cb set their bits, then each entry of the chunk that resolved to a row test-and-sets its
// own; of several equal entries the first atomic keeps its entry. Threads own the same entries as
// in the resolve (e = cb + threadIdx.x + 256 m).
__device__ void drop_repeats(const int* irow, int t, int cb, int ce, int* list, uint32_t* bm) {
  for (int64_t w0 = 0; w0 <= t; w0 += kDedupWindow) {
    const int nb = (int)min((int64_t)kDedupWindow, (int64_t)t + 1 - w0);
    for (int i = threadIdx.x; i < (nb + 31) >> 5; i += 256) bm[i] = 0u;
    __syncthreads();
    for (int e = threadIdx.x; e < cb; e += 256) {
      const int64_t j = (int64_t)irow[e] - w0;
      if (j >= 0 && j < nb) atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    for (int e = cb + threadIdx.x; e < ce; e += 256) {
      const int64_t j = (int64_t)irow[e] - w0;
      if (j >= 0 && j < nb && list[e - cb] >= 0) {
        const uint32_t bit = 1u << (j & 31);
        if (atomicOr(&bm[j >> 5], bit) & bit) list[e - cb] = -1;
      }
    }
    __syncthreads();
  }
}

// Workspace of the split path: fp16 partial outputs [unit][head][column] and (reference, sum)
// per (unit, head), each part 256-byte aligned.
struct MlaSplitWs {
  uint16_t* part;
  f32x2* ml;
};
__host__ __device__ inline size_t mla_align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t mla_split_ws_bytes(int units) {
  return mla_align256((size_t)units * kH * kDv * 2) + mla_align256((size_t)units * kH * 8);
}
__host__ __device__ inline MlaSplitWs mla_split_ws(void* ws, int units) {
  uint8_t* p = (uint8_t*)ws;
  MlaSplitWs w;
  w.part = (uint16_t*)p;
  w.ml = (f32x2*)(p + mla_align256((size_t)units * kH * kDv * 2));
  return w;
}

__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
  const f16x2 h = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t v) {
  const f16x2 h = __builtin_bit_cast(f16x2, v);
  return f32x2{(float)h[0], (float)h[1]};
}

// O^T += V^T P for one tile (the asm text of the PV step); D0..D8 are spliced in after MFMAs
// 1, 4, ..., 25: the gathers of a later tile, or nothing.
#define MLA_PV_ASM(D0, D1, D2, D3, D4, D5, D6, D7, D8) \
  "ds_read_b64_tr_b16 v[224:225], %[ta]\n" \
  "ds_read_b64_tr_b16 v[226:227], %[ta] offset:10272\n" \
  "ds_read_b64_tr_b16 v[228:229], %[ta] offset:64\n" \
  "ds_read_b64_tr_b16 v[230:231], %[ta] offset:10336\n" \
  "ds_read_b64_tr_b16 v[232:233], %[ta] offset:128\n" \
  "ds_read_b64_tr_b16 v[234:235], %[ta] offset:10400\n" \
  "ds_read_b64_tr_b16 v[236:237], %[ta] offset:192\n" \
  "ds_read_b64_tr_b16 v[238:239], %[ta] offset:10464\n" \
  "ds_read_b64_tr_b16 v[240:241], %[ta] offset:256\n" \
  "ds_read_b64_tr_b16 v[242:243], %[ta] offset:10528\n" \
  "ds_read_b64_tr_b16 v[244:245], %[ta] offset:320\n" \
  "ds_read_b64_tr_b16 v[246:247], %[ta] offset:10592\n" \
  "ds_read_b64_tr_b16 v[248:249], %[ta] offset:384\n" \
  "ds_read_b64_tr_b16 v[250:251], %[ta] offset:10656\n" \
  "ds_read_b64_tr_b16 v[252:253], %[ta] offset:448\n" \
  "ds_read_b64_tr_b16 v[254:255], %[ta] offset:10720\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o0], v[224:227], %[p0], %[o0]\n" \
  "ds_read_b64_tr_b16 v[224:225], %[ta] offset:512\n" \
  "ds_read_b64_tr_b16 v[226:227], %[ta] offset:10784\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o1], v[228:231], %[p0], %[o1]\n" \
  D0 \
  "ds_read_b64_tr_b16 v[228:229], %[ta] offset:576\n" \
  "ds_read_b64_tr_b16 v[230:231], %[ta] offset:10848\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o2], v[232:235], %[p0], %[o2]\n" \
  "ds_read_b64_tr_b16 v[232:233], %[ta] offset:640\n" \
  "ds_read_b64_tr_b16 v[234:235], %[ta] offset:10912\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o3], v[236:239], %[p0], %[o3]\n" \
  "ds_read_b64_tr_b16 v[236:237], %[ta] offset:704\n" \
  "ds_read_b64_tr_b16 v[238:239], %[ta] offset:10976\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o4], v[240:243], %[p0], %[o4]\n" \
  D1 \
  "ds_read_b64_tr_b16 v[240:241], %[ta] offset:768\n" \
  "ds_read_b64_tr_b16 v[242:243], %[ta] offset:11040\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o5], v[244:247], %[p0], %[o5]\n" \
  "ds_read_b64_tr_b16 v[244:245], %[ta] offset:832\n" \
  "ds_read_b64_tr_b16 v[246:247], %[ta] offset:11104\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o6], v[248:251], %[p0], %[o6]\n" \
  "ds_read_b64_tr_b16 v[248:249], %[ta] offset:896\n" \
  "ds_read_b64_tr_b16 v[250:251], %[ta] offset:11168\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o7], v[252:255], %[p0], %[o7]\n" \
  D2 \
  "ds_read_b64_tr_b16 v[252:253], %[ta] offset:960\n" \
  "ds_read_b64_tr_b16 v[254:255], %[ta] offset:11232\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o8], v[224:227], %[p0], %[o8]\n" \
  "ds_read_b64_tr_b16 v[224:225], %[ta] offset:20480\n" \
  "ds_read_b64_tr_b16 v[226:227], %[ta] offset:30752\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o9], v[228:231], %[p0], %[o9]\n" \
  "ds_read_b64_tr_b16 v[228:229], %[ta] offset:20544\n" \
  "ds_read_b64_tr_b16 v[230:231], %[ta] offset:30816\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o10], v[232:235], %[p0], %[o10]\n" \
  D3 \
  "ds_read_b64_tr_b16 v[232:233], %[ta] offset:20608\n" \
  "ds_read_b64_tr_b16 v[234:235], %[ta] offset:30880\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o11], v[236:239], %[p0], %[o11]\n" \
  "ds_read_b64_tr_b16 v[236:237], %[ta] offset:20672\n" \
  "ds_read_b64_tr_b16 v[238:239], %[ta] offset:30944\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o12], v[240:243], %[p0], %[o12]\n" \
  "ds_read_b64_tr_b16 v[240:241], %[ta] offset:20736\n" \
  "ds_read_b64_tr_b16 v[242:243], %[ta] offset:31008\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o13], v[244:247], %[p0], %[o13]\n" \
  D4 \
  "ds_read_b64_tr_b16 v[244:245], %[ta] offset:20800\n" \
  "ds_read_b64_tr_b16 v[246:247], %[ta] offset:31072\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o14], v[248:251], %[p0], %[o14]\n" \
  "ds_read_b64_tr_b16 v[248:249], %[ta] offset:20864\n" \
  "ds_read_b64_tr_b16 v[250:251], %[ta] offset:31136\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o15], v[252:255], %[p0], %[o15]\n" \
  "ds_read_b64_tr_b16 v[252:253], %[ta] offset:20928\n" \
  "ds_read_b64_tr_b16 v[254:255], %[ta] offset:31200\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o0], v[224:227], %[p1], %[o0]\n" \
  D5 \
  "ds_read_b64_tr_b16 v[224:225], %[ta] offset:20992\n" \
  "ds_read_b64_tr_b16 v[226:227], %[ta] offset:31264\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o1], v[228:231], %[p1], %[o1]\n" \
  "ds_read_b64_tr_b16 v[228:229], %[ta] offset:21056\n" \
  "ds_read_b64_tr_b16 v[230:231], %[ta] offset:31328\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o2], v[232:235], %[p1], %[o2]\n" \
  "ds_read_b64_tr_b16 v[232:233], %[ta] offset:21120\n" \
  "ds_read_b64_tr_b16 v[234:235], %[ta] offset:31392\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o3], v[236:239], %[p1], %[o3]\n" \
  D6 \
  "ds_read_b64_tr_b16 v[236:237], %[ta] offset:21184\n" \
  "ds_read_b64_tr_b16 v[238:239], %[ta] offset:31456\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o4], v[240:243], %[p1], %[o4]\n" \
  "ds_read_b64_tr_b16 v[240:241], %[ta] offset:21248\n" \
  "ds_read_b64_tr_b16 v[242:243], %[ta] offset:31520\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o5], v[244:247], %[p1], %[o5]\n" \
  "ds_read_b64_tr_b16 v[244:245], %[ta] offset:21312\n" \
  "ds_read_b64_tr_b16 v[246:247], %[ta] offset:31584\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o6], v[248:251], %[p1], %[o6]\n" \
  D7 \
  "ds_read_b64_tr_b16 v[248:249], %[ta] offset:21376\n" \
  "ds_read_b64_tr_b16 v[250:251], %[ta] offset:31648\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o7], v[252:255], %[p1], %[o7]\n" \
  "ds_read_b64_tr_b16 v[252:253], %[ta] offset:21440\n" \
  "ds_read_b64_tr_b16 v[254:255], %[ta] offset:31712\n" \
  "s_waitcnt lgkmcnt(14)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o8], v[224:227], %[p1], %[o8]\n" \
  "s_waitcnt lgkmcnt(12)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o9], v[228:231], %[p1], %[o9]\n" \
  D8 \
  "s_waitcnt lgkmcnt(10)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o10], v[232:235], %[p1], %[o10]\n" \
  "s_waitcnt lgkmcnt(8)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o11], v[236:239], %[p1], %[o11]\n" \
  "s_waitcnt lgkmcnt(6)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o12], v[240:243], %[p1], %[o12]\n" \
  "s_waitcnt lgkmcnt(4)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o13], v[244:247], %[p1], %[o13]\n" \
  "s_waitcnt lgkmcnt(2)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o14], v[248:251], %[p1], %[o14]\n" \
  "s_waitcnt lgkmcnt(0)\n" \
  "v_mfma_f32_32x32x16_bf16 %[o15], v[252:255], %[p1], %[o15]\n"

// One latent-row gather of a later tile, in the PV step, skipped when %[dma] is 0: the row's
// per-lane address is formed in the temporary pair (row id from an SGPR times 1152, plus the
// lane base kv + 16 * lane), M0 is the row's LDS line. SCC is tested right before each branch
// (the M0 add overwrites it).
#define MLA_DMA_LAT(i, off) \
  "s_cmp_lg_u32 %[dma], 0\n" \
  "s_cbranch_scc0 1f\n" \
  "v_mad_u64_u32 %[ga], vcc, %[rid" #i "], %[c1152], %[kvl]\n" \
  "s_add_u32 m0, %[lm0], " #off "\n" \
  "s_nop 0\n" \
  "global_load_lds_dwordx4 %[ga], off\n" \
  "1:\n"
#define MLA_DMA_ROPE \
  "s_cmp_lg_u32 %[dma], 0\n" \
  "s_cbranch_scc0 1f\n" \
  "s_mov_b32 m0, %[rm0]\n" \
  "s_nop 0\n" \
  "global_load_lds_dwordx4 %[rsrc], off\n" \
  "1:\n"

// Operands of the gathers of one tile issued by MLA_DMA_LAT / MLA_DMA_ROPE: wave w loads latent
// rows 4i + w (i = 0..7) and the rope chunks of rows 8w + lane/8, as issue_tile does. Formed
// right before the asm that uses them (a few VALU and SALU ops), so that nothing extra stays live
// across the tile loop.
struct DmaOps {
  uint64_t kvl;       // kv + 16 * lane
  uint32_t c1152;     // the row pitch in bytes, for v_mad_u64_u32
  uint32_t rid[kRowsPerWave];
  uint32_t lat_m0, rope_m0;
  uint64_t rope_src;  // this lane's rope chunk
};
__device__ __forceinline__ DmaOps dma_ops(const uint8_t* __restrict__ kv_base, const lds_u8* buf, TileEntries te,
                                          int wave, int lane) {
  asm volatile("" : "+v"(lane));  // opaque copy: the lane values are formed per tile
  DmaOps d;
  d.kvl = (uint64_t)(uintptr_t)(kv_base + 16 * lane);
  d.c1152 = kRowBytes;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) d.rid[i] = (uint32_t)__builtin_amdgcn_readlane(te.ent, 4 * i + wave);
  d.lat_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)buf + wave * (kLatStride + 64));
  d.rope_m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(buf + kRopeOff + kRowsPerWave * wave * kRopeBytes));
  const int my_slot = kRowsPerWave * wave + (lane >> 3);
  d.rope_src = (uint64_t)(uintptr_t)(kv_base + (int64_t)te.my_ent * kRowBytes + kLatBytes + 16 * ((lane & 7) ^ rope_swz(my_slot)));
  return d;
}
#define MLA_DMA_INPUTS(d, m) \
  [dma] "s"(m), [kvl] "v"(d.kvl), [c1152] "v"(d.c1152), [lm0] "s"(d.lat_m0), [rm0] "s"(d.rope_m0), \
  [rsrc] "v"(d.rope_src), [rid0] "s"(d.rid[0]), [rid1] "s"(d.rid[1]), [rid2] "s"(d.rid[2]), [rid3] "s"(d.rid[3]), \
  [rid4] "s"(d.rid[4]), [rid5] "s"(d.rid[5]), [rid6] "s"(d.rid[6]), [rid7] "s"(d.rid[7])
// How a workgroup finishes: the whole row (no split), or a partial for the merge kernel.
constexpr int kMlaNoSplit = 0, kMlaSplitCombine = 1;

// Rare path (the lane's head moved its reference maximum): scale its running output by alpha.
// Out of line, so that the hot loop keeps its accumulators in AGPRs.
__device__ __attribute__((noinline)) void rescale_acc(f32x16* o, float alpha) {
  for (int mt = 0; mt < kDv / 32; ++mt) o[mt] *= alpha;
}

// Workgroup: 4 waves, all 128 heads of one (row, split); wave w owns heads 32w..32w+31 for the
// whole computation, so the tiles are the only thing the waves share. Per tile of 32 positions
// (v_mfma_f32_32x32x16_bf16 throughout):
//   S^T = K Q^T: key tile rows as the A operand from LDS, the wave's 32 query heads as the B
//     operand (latent dims resident in 128 VGPRs, rope dims from LDS); lane l ends up with head
//     l%32 and 16 of the 32 keys
//   softmax bookkeeping per head in the log2 domain, probabilities rounded to bf16 in registers
//   O^T += V^T P: V^T from LDS through ds_read_b64_tr_b16 as the A operand, P straight from the
//     registers as the B operand (the K steps take the keys in the order the S layout holds them),
//     512 value columns x 32 heads in 256 AGPRs
template <int kMode>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_mfma_kernel(AttnArgs a, int splits, int entries_per_split, int units, int per_xcd, void* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroups are dispatched to the 8 XCDs round robin. Split rows: each XCD takes a contiguous
  // range of units, so the splits of a row and the rows of a request share that XCD's L2. Unsplit
  // rows (prefill blocks, large decode batches): rows in pairs, the pairs dealt round robin over the
  // XCDs, the two rows of a pair one after the other on one XCD (MTP rows, neighbouring prefill
  // rows), and the last rows first; a causal block's rows differ in length, so contiguous row
  // ranges per XCD would give the XCDs uneven work.
  int unit;
  if (kMode == kMlaNoSplit) {
    const int slot = blockIdx.x >> 3;
    const int fwd = 2 * ((slot >> 1) * 8 + (int)(blockIdx.x & 7)) + (slot & 1);
    if (fwd >= units) return;
    unit = units - 1 - fwd;
  } else {
    unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (unit >= units) return;
  }
  const int r = unit / splits, sp = unit % splits;
  const int seq = a.rs.of(r);  // -1: no page-table row, every entry resolves to no row
  const int t = a.q_pos[r];
  const int n_entries = a.idx ? a.k : max(0, min(t + 1, a.k));  // dense: a.k = max_ctx
  const int e_begin = sp * entries_per_split;
  const int e_end = min(n_entries, e_begin + entries_per_split);
  lds_u8* lds = (lds_u8*)smem;
  int* list = (int*)(smem + kListOff);
  int* tmask = (int*)(smem + kMaskOff);
  const int hl = lane & 31, half = lane >> 5;  // lane's head within the wave, key half

  // query heads as B operands: lane holds head 32w + lane%32, dims 16*ks + 8*(lane/32) .. +8 of
  // the latent part in registers; the rope dims of all heads go to LDS (head h keeps chunk c at
  // c ^ rope_swz(h) of its 128-byte row). Loaded once the first tile gathers are in flight.
  bf16x8 qf[kDv / 16];
  // O^T accumulators: o[mt] = value columns 32mt .. 32mt+31 of head 32w + lane%32
  f32x16 o[kDv / 32];
#pragma unroll
  for (int i = 0; i < kDv / 32; ++i) o[i] = f32x16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  const float c_scale = a.sm_scale * kLog2e;
  const uint8_t* kv_base = (const uint8_t*)a.kv.base;

  // Per-lane LDS byte offsets of the operand fetches within a tile
  int g1_base, rope_base, qr_base, tr_base[2];
  const int rope_x = rope_swz(hl) >> 1;
  {
    // QK^T A operand: key row lane%32, chunk 2*ks + lane/32
    g1_base = hl * kLatStride + 16 * lat_rot(hl) + 16 * half;
    // rope k-step k: chunk 2k + half of key row lane%32 / of query head 32w + lane%32, both at
    // position (2k + half) ^ rope_swz = 2 * (k ^ rope_x) + (half ^ (rope_swz & 1))
    rope_base = kRopeOff + hl * kRopeBytes + 16 * (half ^ (rope_swz(hl) & 1));
    qr_base = kQRopeOff + (32 * wave + hl) * kRopeBytes + 16 * (half ^ (rope_swz(hl) & 1));
    // PV transpose reads (read a of K step ks, lane group G = lane/16, lane j in the group): key
    // row 16*ks + 4*(G/2) + 8*a + j/4, value columns 32*mt + 16*(G%2) + 4*(j%4) .. +4; the
    // row's rotation is 4*(j/4) + G/2 + 2*a
    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int a8 = 0; a8 < 2; ++a8)
      tr_base[a8] = (4 * (G >> 1) + 8 * a8 + (j >> 2)) * kLatStride + 16 * (4 * (j >> 2) + (G >> 1) + 2 * a8) +
                    32 * (G & 1) + 8 * (j & 3);
  }

  // S_t is a set: only lists that are not a strictly ascending run of visible entries from entry 0
  // up to this split's end can repeat a position into this split; those go through the filter.
  const int* irow = a.idx ? a.idx + (int64_t)r * a.ld_idx : nullptr;
  const int tid = 64 * wave + lane;
  const int ps = a.kv.page_size;
  // page-table entries a visible position of this row can use
  const int np = (seq >= 0 && t >= 0) ? min(a.kv.ld_pt, t / ps + 1) : 0;
  // Staged prologue (index lists of at most kListCap entries over at most kStagePages pages):
  // the index row up to this split's end, the sequence's page-table row and the rope part of the
  // query are loaded first, then the latent part of the query; the first three are staged in
  // LDS as soon as they land (vector loads complete in issue order, so their wait leaves the
  // query's 128 KB in flight), and the repeat check and the resolve below run from LDS while the
  // query arrives. Otherwise the query is loaded first and the resolve reads the index list and
  // the page table from memory (any load issued after the query's 147 KB waits for all of it).
  const bool staged = irow && e_end <= kListCap && np <= kStagePages;
  int* st_raw = (int*)smem;                  // staged index row [0, e_end)
  int* st_pt = (int*)(smem + 4 * kListCap);  // staged page-table row [0, np)
  auto load_query_latent = [&]() {
    const uint16_t* qh = a.q + ((int64_t)r * kH + 32 * wave + hl) * kDqk + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kDv / 16; ++ks) qf[ks] = *(const bf16x8*)(qh + 16 * ks);
  };
  // the rope part of all heads into LDS: head h keeps chunk c at c ^ rope_swz(h) of its 128-byte row
  auto rope_src = [&](int j) {
    const int i = tid + 256 * j, h = i >> 3, c = i & 7;
    return (const i32x4*)(a.q + ((int64_t)r * kH + h) * kDqk + kDv + 8 * c);
  };
  auto rope_dst = [&](int j) {
    const int i = tid + 256 * j, h = i >> 3, c = i & 7;
    return (__attribute__((address_space(3))) i32x4*)(lds + kQRopeOff + h * kRopeBytes + 16 * (c ^ rope_swz(h)));
  };
  bool dedupe = false;
  if (staged) {
    int raw[kListCap / 256], ptv[kStagePages / 256];
    i32x4 qr[kH * 8 / 256];
#pragma unroll
    for (int u = 0; u < kListCap / 256; ++u) {
      const int e = tid + 256 * u;
      raw[u] = e < e_end ? irow[e] : -1;
    }
#pragma unroll
    for (int u = 0; u < kStagePages / 256; ++u) {
      const int pg = tid + 256 * u;
      ptv[u] = pg < np ? a.kv.page_table[(int64_t)seq * a.kv.ld_pt + pg] : -1;
    }
#pragma unroll
    for (int j = 0; j < kH * 8 / 256; ++j) qr[j] = *rope_src(j);
    load_query_latent();
#pragma unroll
    for (int u = 0; u < kListCap / 256; ++u)
      if (tid + 256 * u < e_end) st_raw[tid + 256 * u] = raw[u];
#pragma unroll
    for (int u = 0; u < kStagePages / 256; ++u)
      if (tid + 256 * u < np) st_pt[tid + 256 * u] = ptv[u];
#pragma unroll
    for (int j = 0; j < kH * 8 / 256; ++j) *rope_dst(j) = qr[j];
    __syncthreads();
    // the repeat check of block_needs_dedupe, over the staged row
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kListCap / 256; ++u) {
      const int e = tid + 256 * u;
      if (e >= 1 && e < e_end) {
        const int c = st_raw[e], pv = st_raw[e - 1];
        const bool vc = c >= 0 && c <= t, vp = pv >= 0 && pv <= t;
        bad |= vc && !(vp && pv < c);
      }
    }
    int* flags = (int*)(smem + kFlagOff);
    const bool any = __any(bad);
    if (lane == 0) flags[wave] = any ? 1 : 0;
    __syncthreads();
    dedupe = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  } else {
    load_query_latent();
#pragma unroll
    for (int j = 0; j < kH * 8 / 256; ++j) *rope_dst(j) = *rope_src(j);
    dedupe = irow && block_needs_dedupe(irow, t, 1, e_end, (int*)(smem + kFlagOff), wave, lane);
  }
  for (int cb = e_begin; cb < e_end; cb += kListCap) {
    const int ce = min(e_end, cb + kListCap);
    __syncthreads();  // the previous chunk is done with the list and the buffers
    if (staged) {
      // the whole list is one chunk: resolve it from the staged rows. A position j <= t with
      // j / ps < ld_pt has j / ps < np, so it lies on a staged page; np = 0 (nothing staged) for a
      // row without a page-table row.
      for (int e = cb + (int)threadIdx.x; e < ce; e += 256) {
        const int j = st_raw[e];
        const bool vis = j >= 0 && j <= t && j / ps < np;
        const int pg = vis ? st_pt[j / ps] : -1;
        list[e - cb] = (pg >= 0 && pg < a.kv.num_pages) ? pg * ps + j % ps : -1;
      }
      // the repeat filter's bitmap overwrites the staged rows
      if (dedupe) __syncthreads();
    }
    // eight entries per thread at a time: all their index loads, then all their page-table
    // loads, so the resolve costs two memory latencies rather than two per entry
    for (int e0 = cb + (int)threadIdx.x; !staged && e0 < ce; e0 += 8 * 256) {
      int jj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 256 * u;
        jj[u] = e < ce ? (a.idx ? a.idx[(int64_t)r * a.ld_idx + e] : e) : -1;
      }
      int pg[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = jj[u];
        const bool vis = seq >= 0 && j >= 0 && j <= t && j / a.kv.page_size < a.kv.ld_pt;
        pg[u] = vis ? a.kv.page_table[(int64_t)seq * a.kv.ld_pt + j / a.kv.page_size] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + 256 * u;
        if (e < ce)
          list[e - cb] = (pg[u] >= 0 && pg[u] < a.kv.num_pages) ? pg[u] * a.kv.page_size + jj[u] % a.kv.page_size : -1;
      }
    }
    if (dedupe) drop_repeats(irow, t, cb, ce, list, (uint32_t*)smem);
    if (cb == e_begin) {
      // consume the query fragments here, before any gather is issued: their wait then covers
      // the query loads only, and no wait for them lands in the tile loop (where it would also
      // drain the tile gathers in flight). The barrier below also publishes the rope part in LDS.
#pragma unroll
      for (int ks = 0; ks < kDv / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
    }
    __syncthreads();
    const int n_list = ce - cb;
    const int ntiles = (n_list + kNK - 1) / kNK;
    // Per-tile valid-entry masks; every invalid entry of a tile (and the tail of the last tile)
    // takes the tile's first valid row id, so a gather loads finite data for it (its probability
    // is 0). Lanes 0..31 take tile t0, lanes 32..63 tile t0 + 1.
    for (int t0 = 2 * wave; t0 < ntiles; t0 += 8) {
      const int tt = t0 + half, e = tt * kNK + hl;
      const int v = (tt < ntiles && e < n_list) ? list[e] : -1;
      const uint64_t bal = __ballot(v >= 0);
      const uint32_t m = half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
      const int sub = __shfl(v, 32 * half + (m ? __ffs(m) - 1 : 0));
      if (tt < ntiles) {
        if (v < 0 && m) list[e] = sub;
        if (hl == 0) tmask[tt] = (int)m;
      }
    }
    __syncthreads();
    // Only tiles with a valid key are gathered and computed (padding past a short row's end,
    // tiles of holes): bit t of `act` is set for tile t (ntiles <= 64), and `pend` holds the
    // active tiles not gathered yet, lowest first.
    static_assert(kListCap / kNK <= 64, "a chunk's tiles fit one wave-wide mask");
    const uint64_t act = __ballot(lane < ntiles && tmask[lane] != 0);
    const int nact = __builtin_popcountll(act);
    uint64_t pend = act;
    auto next_tile = [&]() {
      const int t = __builtin_ctzll(pend);
      pend &= pend - 1;
      return t;
    };
    // Settle every vector-memory operation the compiler issued so far (the query loads are
    // already consumed; register spills of the prologue may still be in flight) before the first
    // gathers: its wait-count pass then sees nothing pending, and inserts no wait inside the tile
    // loop that would also drain the gathers in flight (a store's data register rewritten in the
    // loop would otherwise take one).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left at their maxima
    // vm[d] = valid-entry mask of active tile j + d (0 past the end); only constant indices, so
    // the masks stay in scalar registers. Active tiles 0 .. kNBuf - 2 are gathered here, active
    // tile j + kNBuf - 1 during active tile j's PV step.
    uint32_t vm[kNBuf];
#pragma unroll
    for (int pt = 0; pt < kNBuf; ++pt) {
      vm[pt] = 0u;
      if (pt < kNBuf - 1 && pt < nact)
        vm[pt] = issue_tile(kv_base, lds + pt * kTileBytes, read_entries(list, tmask, next_tile(), ntiles, wave, lane), wave, lane);
    }
    // entries of the next tile to gather, read one iteration before they are needed
    TileEntries nxt = kNBuf - 1 < nact ? read_entries(list, tmask, next_tile(), ntiles, wave, lane) : TileEntries{0, 0, 0};
    int b = 0;  // buffer of active tile j (j % kNBuf, kept as a rotating counter)
    for (int j = 0; j < nact; ++j) {
      int younger = 0;  // later tiles whose gathers are in flight
#pragma unroll
      for (int d = 1; d + 1 < kNBuf; ++d) younger += vm[d] != 0u ? 1 : 0;
      wait_gathers(younger);
      // Every wave's share of tile j has landed once all waves pass this barrier, and every wave
      // has consumed its reads of tile j - 1 (into MFMAs). A bare s_barrier: the fence of
      // __syncthreads would also drain the younger tiles' loads that are meant to stay in flight.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int b_cur = b;
      b = b + 1 == kNBuf ? 0 : b + 1;
      // active tile j + kNBuf - 1 goes to the buffer tile j - 1 used (every wave is done with it);
      // its gathers are issued in this iteration's PV step
      const TileEntries te2 = nxt;
      uint32_t mask2 = 0u;
      lds_u8* buf2 = lds;
      if (j + kNBuf - 1 < nact) {
        const int nb = b_cur == 0 ? kNBuf - 1 : b_cur - 1;
        mask2 = (uint32_t)__builtin_amdgcn_readfirstlane(te2.mask);  // nonzero: an active tile
        buf2 = lds + nb * kTileBytes;
        vm[kNBuf - 1] = mask2;
        nxt = j + kNBuf < nact ? read_entries(list, tmask, next_tile(), ntiles, wave, lane) : TileEntries{0, 0, 0};
      }
      const uint32_t valid = vm[0];
#pragma unroll
      for (int q = 0; q + 1 < kNBuf; ++q) vm[q] = vm[q + 1];
      vm[kNBuf - 1] = 0u;
      const lds_u8* tile = lds + b_cur * kTileBytes;

      // ---- S^T = K Q^T: lane holds head lane%32, keys 8*(i/4) + 4*(lane/32) + i%4, i = 0..15
      // S^T for this tile: the 4 rope k-steps (both operands from LDS) and the 32 latent k-steps
      // in one accumulation chain (back-to-back MFMAs on one accumulator measured slightly faster
      // than two interleaved chains, with 16 fewer VGPRs), 8 operand fetches in flight ahead of
      // the MFMAs (into v224..v255). Written as one asm block so that S stays in VGPRs (the AGPRs
      // hold the output) and the fetches are not reordered. LDS reads complete in order, so each
      // wait counts only the younger reads of this block; the trailing s_nops cover the
      // MFMA-result to VALU-read latency of the softmax that follows.
      f32x16 s;
      {
        const uint32_t al = (uint32_t)(uintptr_t)(tile + g1_base);
        const uint32_t kb = (uint32_t)(uintptr_t)(tile + rope_base), qb = (uint32_t)(uintptr_t)(lds + qr_base);
        const uint32_t x0 = 32 * (0 ^ rope_x), x1 = 32 * (1 ^ rope_x), x2 = 32 * (2 ^ rope_x), x3 = 32 * (3 ^ rope_x);
        f32x16 s0;
        asm volatile(
          "ds_read_b128 v[224:227], %[k0]\n"
          "ds_read_b128 v[228:231], %[r0]\n"
          "ds_read_b128 v[232:235], %[k1]\n"
          "ds_read_b128 v[236:239], %[r1]\n"
          "ds_read_b128 v[240:243], %[k2]\n"
          "ds_read_b128 v[244:247], %[r2]\n"
          "ds_read_b128 v[248:251], %[k3]\n"
          "ds_read_b128 v[252:255], %[r3]\n"
          "s_waitcnt lgkmcnt(6)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[224:227], v[228:231], 0\n"
          "ds_read_b128 v[224:227], %[al]\n"
          "ds_read_b128 v[228:231], %[al] offset:32\n"
          "s_waitcnt lgkmcnt(6)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[232:235], v[236:239], %[s0]\n"
          "ds_read_b128 v[232:235], %[al] offset:64\n"
          "ds_read_b128 v[236:239], %[al] offset:96\n"
          "s_waitcnt lgkmcnt(6)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[240:243], v[244:247], %[s0]\n"
          "ds_read_b128 v[240:243], %[al] offset:128\n"
          "ds_read_b128 v[244:247], %[al] offset:160\n"
          "s_waitcnt lgkmcnt(6)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[248:251], v[252:255], %[s0]\n"
          "ds_read_b128 v[248:251], %[al] offset:192\n"
          "ds_read_b128 v[252:255], %[al] offset:224\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[224:227], %[q0], %[s0]\n"
          "ds_read_b128 v[224:227], %[al] offset:256\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[228:231], %[q1], %[s0]\n"
          "ds_read_b128 v[228:231], %[al] offset:288\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[232:235], %[q2], %[s0]\n"
          "ds_read_b128 v[232:235], %[al] offset:320\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[236:239], %[q3], %[s0]\n"
          "ds_read_b128 v[236:239], %[al] offset:352\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[240:243], %[q4], %[s0]\n"
          "ds_read_b128 v[240:243], %[al] offset:384\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[244:247], %[q5], %[s0]\n"
          "ds_read_b128 v[244:247], %[al] offset:416\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[248:251], %[q6], %[s0]\n"
          "ds_read_b128 v[248:251], %[al] offset:448\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[252:255], %[q7], %[s0]\n"
          "ds_read_b128 v[252:255], %[al] offset:480\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[224:227], %[q8], %[s0]\n"
          "ds_read_b128 v[224:227], %[al] offset:512\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[228:231], %[q9], %[s0]\n"
          "ds_read_b128 v[228:231], %[al] offset:544\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[232:235], %[q10], %[s0]\n"
          "ds_read_b128 v[232:235], %[al] offset:576\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[236:239], %[q11], %[s0]\n"
          "ds_read_b128 v[236:239], %[al] offset:608\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[240:243], %[q12], %[s0]\n"
          "ds_read_b128 v[240:243], %[al] offset:640\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[244:247], %[q13], %[s0]\n"
          "ds_read_b128 v[244:247], %[al] offset:672\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[248:251], %[q14], %[s0]\n"
          "ds_read_b128 v[248:251], %[al] offset:704\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[252:255], %[q15], %[s0]\n"
          "ds_read_b128 v[252:255], %[al] offset:736\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[224:227], %[q16], %[s0]\n"
          "ds_read_b128 v[224:227], %[al] offset:768\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[228:231], %[q17], %[s0]\n"
          "ds_read_b128 v[228:231], %[al] offset:800\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[232:235], %[q18], %[s0]\n"
          "ds_read_b128 v[232:235], %[al] offset:832\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[236:239], %[q19], %[s0]\n"
          "ds_read_b128 v[236:239], %[al] offset:864\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[240:243], %[q20], %[s0]\n"
          "ds_read_b128 v[240:243], %[al] offset:896\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[244:247], %[q21], %[s0]\n"
          "ds_read_b128 v[244:247], %[al] offset:928\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[248:251], %[q22], %[s0]\n"
          "ds_read_b128 v[248:251], %[al] offset:960\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[252:255], %[q23], %[s0]\n"
          "ds_read_b128 v[252:255], %[al] offset:992\n"
          "s_waitcnt lgkmcnt(7)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[224:227], %[q24], %[s0]\n"
          "s_waitcnt lgkmcnt(6)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[228:231], %[q25], %[s0]\n"
          "s_waitcnt lgkmcnt(5)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[232:235], %[q26], %[s0]\n"
          "s_waitcnt lgkmcnt(4)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[236:239], %[q27], %[s0]\n"
          "s_waitcnt lgkmcnt(3)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[240:243], %[q28], %[s0]\n"
          "s_waitcnt lgkmcnt(2)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[244:247], %[q29], %[s0]\n"
          "s_waitcnt lgkmcnt(1)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[248:251], %[q30], %[s0]\n"
          "s_waitcnt lgkmcnt(0)\n"
          "v_mfma_f32_32x32x16_bf16 %[s0], v[252:255], %[q31], %[s0]\n"
          "s_nop 7\n"
          "s_nop 7\n"
          "s_nop 7\n"
          : [s0] "=&v"(s0)
          : [al] "v"(al), [k0] "v"(kb + x0), [k1] "v"(kb + x1), [k2] "v"(kb + x2), [k3] "v"(kb + x3),
            [r0] "v"(qb + x0), [r1] "v"(qb + x1), [r2] "v"(qb + x2), [r3] "v"(qb + x3),
            [q0] "v"(qf[0]), [q1] "v"(qf[1]), [q2] "v"(qf[2]), [q3] "v"(qf[3]), [q4] "v"(qf[4]), [q5] "v"(qf[5]), [q6] "v"(qf[6]), [q7] "v"(qf[7]), [q8] "v"(qf[8]), [q9] "v"(qf[9]), [q10] "v"(qf[10]), [q11] "v"(qf[11]), [q12] "v"(qf[12]), [q13] "v"(qf[13]), [q14] "v"(qf[14]), [q15] "v"(qf[15]), [q16] "v"(qf[16]), [q17] "v"(qf[17]), [q18] "v"(qf[18]), [q19] "v"(qf[19]), [q20] "v"(qf[20]), [q21] "v"(qf[21]), [q22] "v"(qf[22]), [q23] "v"(qf[23]), [q24] "v"(qf[24]), [q25] "v"(qf[25]), [q26] "v"(qf[26]), [q27] "v"(qf[27]), [q28] "v"(qf[28]), [q29] "v"(qf[29]), [q30] "v"(qf[30]), [q31] "v"(qf[31])
          : "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255", "memory");
        s = s0;
      }
      // ---- softmax bookkeeping in the log2 domain; the two lanes of a head see all 32 keys.
      //      c_scale > 0, so the largest raw score gives the largest logit.
      if (valid != 0xffffffffu) {  // uniform: a partial tile, mask its invalid keys
        const uint32_t vh = valid >> (4 * half);  // bit 8*(i/4) + i%4: key of s[i] is valid
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((vh >> (8 * (i >> 2) + (i & 3))) & 1u)) s[i] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      {
        // the other lane of the head is lane ^ 32: v_permlane32_swap exchanges the wave halves
        // (one result holds the lane's own value, the other its partner's)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]))) * c_scale;
      }
      if (mx > m_ref + kRescaleThreshold) {
        // nothing accumulated yet (m_ref = -inf): the output is still zero, just adopt mx
        const float alpha = (m_ref == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
        l_sum *= alpha;
        if (__any(alpha != 1.f)) {
          f32x16 tmp[kDv / 32];
#pragma unroll
          for (int i = 0; i < kDv / 32; ++i) tmp[i] = o[i];
          rescale_acc(tmp, alpha);
#pragma unroll
          for (int i = 0; i < kDv / 32; ++i) o[i] = tmp[i];
          // settle the reloads here, so no wait for them is left on the hot path after the join
          __builtin_amdgcn_s_waitcnt(0x0F70);
        }
      }
      // probabilities, packed to bf16 pairs: pk[ks] is the B operand of K step ks
      bf16x8 pk[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // exp2(-inf) = 0 for invalid keys
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * ks + e], c_scale, -m_ref));
          l_sum += pv[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[ks][e] = (__bf16)pv[e];
      }
      // ---- O^T += V^T P, 32 MFMAs (K step ks = j / 16, column block mt = j % 16) with the two
      //      transpose reads of each A operand issued eight MFMAs ahead into v224..v255. K step
      //      ks takes keys 16*ks + 8*(e/4) + 4*h + e%4 in slot 8*h + e, the order in which lane
      //      half h holds them in pk[ks]; the read of key row 16*ks + 4*(G/2) + 8*a + j/4 sits at
      //      tr_base[a] = tr_base[0] + 10272*a, plus 64*mt + 20480*ks. The output accumulators
      //      stay in AGPRs; their readers after the tile loop are separated by s_nops.
      {
        const uint32_t ta = (uint32_t)(uintptr_t)(tile + tr_base[0]);
        {
          // the nine gathers of tile it + kNBuf - 1 (when it has a valid key) ride in the MFMA
          // stream: a wave stalled at a gather's issue would otherwise hold its MFMAs back (rows
          // 4i + w as in issue_tile; without a tile to gather the row ids are not used)
          const DmaOps d = dma_ops(kv_base, buf2, te2, wave, lane);
          uint64_t ga;
          uint32_t sv;
          asm volatile(
            "s_mov_b32 %[sv], m0\n"
            MLA_PV_ASM(MLA_DMA_LAT(0, 0), MLA_DMA_LAT(1, 5136), MLA_DMA_LAT(2, 10272), MLA_DMA_LAT(3, 15408),
                       MLA_DMA_LAT(4, 20480), MLA_DMA_LAT(5, 25616), MLA_DMA_LAT(6, 30752), MLA_DMA_LAT(7, 35888),
                       MLA_DMA_ROPE)
            "s_mov_b32 m0, %[sv]\n"
            : [o0] "+a"(o[0]), [o1] "+a"(o[1]), [o2] "+a"(o[2]), [o3] "+a"(o[3]), [o4] "+a"(o[4]), [o5] "+a"(o[5]), [o6] "+a"(o[6]), [o7] "+a"(o[7]), [o8] "+a"(o[8]), [o9] "+a"(o[9]), [o10] "+a"(o[10]), [o11] "+a"(o[11]), [o12] "+a"(o[12]), [o13] "+a"(o[13]), [o14] "+a"(o[14]), [o15] "+a"(o[15]), [ga] "=&v"(ga), [sv] "=&s"(sv)
            : [ta] "v"(ta), [p0] "v"(pk[0]), [p1] "v"(pk[1]),
              MLA_DMA_INPUTS(d, mask2)
            : "vcc", "scc", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255", "memory");
        }
      }
    }
  }

  // the accumulators were last written by MFMAs inside asm: cover the MFMA-result to VALU-read
  // latency before the epilogue reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  // per-head totals: the two lanes of a head hold the sums over their key halves
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  const int head = 32 * wave + hl;
  // Output layout: lane holds columns 32mt + 8(i/4) + 4*half + i%4 of head 32w + lane%32. Results
  // are staged [head][column] in LDS (8-byte unit u of a head's 1 KB line at u ^ 2*(head%32), i.e.
  // 16-byte chunk c at c ^ (head%32)) and stored with coalesced 16-byte writes.
  auto stage = [&](auto cvt4) {
    lds_u8* st = lds + head * (kDv * 2);
#pragma unroll
    for (int mt = 0; mt < kDv / 32; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = 8 * mt + 2 * q + half;
        *(__attribute__((address_space(3))) u32x2*)(st + 8 * (u ^ (2 * hl))) = cvt4(mt, q);
      }
  };
  auto store_staged = [&](uint16_t* dst16) {
    i32x4* dst = (i32x4*)dst16;
    for (int i = threadIdx.x; i < kH * kDv / 8; i += 256) {
      const int h = i >> 6, c = i & 63;
      dst[i] = *(const __attribute__((address_space(3))) i32x4*)(lds + h * (kDv * 2) + 16 * (c ^ (h & 31)));
    }
  };
  auto bf16x4_of = [](float x0, float x1, float x2, float x3) {
    return u32x2{(uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16),
                 (uint32_t)f32_to_bf16(x2) | ((uint32_t)f32_to_bf16(x3) << 16)};
  };
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float lse2 = l_tot > 0.f ? m_ref + __log2f(l_tot) : -INFINITY;  // log-sum-exp, log2 units
  __syncthreads();  // every wave is done with the tile buffers
  if (kMode == kMlaNoSplit) {
    if (a.lse && half == 0) a.lse[(int64_t)r * kH + head] = lse2 / kLog2e;
    stage([&](int mt, int q) {
      return bf16x4_of(o[mt][4 * q] * inv, o[mt][4 * q + 1] * inv, o[mt][4 * q + 2] * inv, o[mt][4 * q + 3] * inv);
    });
    __syncthreads();
    store_staged(a.out + (int64_t)r * kH * kDv);
    return;
  }
  // Partial result of this split: the normalised output in fp16 ([unit][head][column]) and
  // (reference, sum) per head.
  MlaSplitWs w = mla_split_ws(ws, units);
  stage([&](int mt, int q) {
    return u32x2{pack_f16x2(o[mt][4 * q] * inv, o[mt][4 * q + 1] * inv), pack_f16x2(o[mt][4 * q + 2] * inv, o[mt][4 * q + 3] * inv)};
  });
  if (half == 0) w.ml[(int64_t)unit * kH + head] = f32x2{m_ref, l_tot};
  __syncthreads();
  store_staged(w.part + (int64_t)unit * kH * kDv);
}

// Merge the splits of each row from their fp16 partials: out = sum_s w_s N_s / sum_s w_s with
// w_s = l_s 2^(m_s - M). One thread per (row, head, 8 output columns). The (m, l) pairs, then the
// partials, of up to kBatch splits at a time are loaded together, so a row split many ways costs a
// few memory latencies rather than one per split; with at most kBatch splits the pairs and the
// partials are all loaded at once (one memory latency). A split without keys (l = 0) is skipped by
// selects: whatever its partial holds never enters the sum.
// The merged 8 columns (bf16) and, for the first column group, the lse of the row's head.
__device__ __forceinline__ void combine_store(const AttnArgs& a, int r, int head, int cg, float M, float L,
                                              const float (&acc)[8]) {
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* dst = a.out + ((int64_t)r * kH + head) * kDv + 8 * cg;
  uint32_t wd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) wd[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
  *(i32x4*)dst = i32x4{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
  if (a.lse && cg == 0) a.lse[(int64_t)r * kH + head] = L > 0.f ? (M + __log2f(L)) / kLog2e : -INFINITY;
}

template <int kBatch>
__global__ void __launch_bounds__(256) mla_combine_kernel(AttnArgs a, int splits, int units, void* __restrict__ ws) {
  const int r = blockIdx.y;
  const int item = blockIdx.x * 256 + threadIdx.x;  // head * 64 + column group
  if (item >= kH * (kDv / 8)) return;
  const int head = item / (kDv / 8), cg = item % (kDv / 8);
  MlaSplitWs w = mla_split_ws(ws, units);
  const int64_t u0 = (int64_t)r * splits * kH + head;  // split s2 at u0 + s2 * kH
  float M = -INFINITY;
  if (splits <= kBatch) {
    f32x2 ml[kBatch];
    i32x4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < splits) {  // uniform
        const int64_t u = u0 + (int64_t)j * kH;
        ml[j] = w.ml[u];
        v[j] = *(const i32x4*)(w.part + u * kDv + 8 * cg);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (j < splits && ml[j][1] > 0.f) M = fmaxf(M, ml[j][0]);
    float L = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool use = j < splits && ml[j][1] > 0.f;
      const float f = use ? ml[j][1] * exp2f(ml[j][0] - M) : 0.f;
      L += f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 x = unpack_f16x2((uint32_t)v[j][e]);
        acc[2 * e] = use ? fmaf(f, x[0], acc[2 * e]) : acc[2 * e];
        acc[2 * e + 1] = use ? fmaf(f, x[1], acc[2 * e + 1]) : acc[2 * e + 1];
      }
    }
    combine_store(a, r, head, cg, M, L, acc);
    return;
  }
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    f32x2 ml[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < splits) ml[j] = w.ml[u0 + (int64_t)(s0 + j) * kH];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j < splits && ml[j][1] > 0.f) M = fmaxf(M, ml[j][0]);
  }
  float L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    f32x2 ml[kBatch];
    i32x4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < splits) {  // uniform: the loads of a batch are still issued back to back
        const int64_t u = u0 + (int64_t)(s0 + j) * kH;
        ml[j] = w.ml[u];
        v[j] = *(const i32x4*)(w.part + u * kDv + 8 * cg);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool use = s0 + j < splits && ml[j][1] > 0.f;
      const float f = use ? ml[j][1] * exp2f(ml[j][0] - M) : 0.f;
      L += f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 x = unpack_f16x2((uint32_t)v[j][e]);
        acc[2 * e] = use ? fmaf(f, x[0], acc[2 * e]) : acc[2 * e];
        acc[2 * e + 1] = use ? fmaf(f, x[1], acc[2 * e + 1]) : acc[2 * e + 1];
      }
    }
  }
  combine_store(a, r, head, cg, M, L, acc);
}

size_t mla_mfma_ws_bytes(int rows, int splits) {
  if (splits <= 1) return 0;
  return mla_split_ws_bytes(rows * splits);
}

int mla_mfma_pick_splits(int rows, int k) {
  // aim for >= 256 workgroups (one per (row, split)), at least 4 tiles per split (a split's fixed
  // cost, its query load and partial, is worth about two tiles: 4 rows of 2048 keys run as fast in
  // 16 splits as in 32, and 16 rows run slower in 8 splits than in 16)
  int s = 1;
  while (rows * s < 256 && (k / (s * 2)) >= 4 * kNK) s *= 2;
  return s;
}

hipError_t launch_mla_mfma(const AttnArgs& a, int splits, void* ws, hipStream_t stream) {
  const int rows = a.rows;
  const int units = rows * (splits > 1 ? splits : 1);
  const int per_xcd = (units + 7) / 8;
  const int blocks = 8 * per_xcd;
  if (splits <= 1) {
    const int per = a.idx ? a.k : 1 << 30;
    // pair p of rows takes slots 2 (p / 8) and 2 (p / 8) + 1 of XCD p % 8
    const int pair_blocks = 16 * (((units + 1) / 2 + 7) / 8);
    hipLaunchKernelGGL(mla_mfma_kernel<kMlaNoSplit>, dim3(pair_blocks), dim3(256), 0, stream, a, 1, per, units, per_xcd,
                       nullptr);
    return hipGetLastError();
  }
  const int per = ((a.k + splits - 1) / splits + kNK - 1) / kNK * kNK;
  hipLaunchKernelGGL(mla_mfma_kernel<kMlaSplitCombine>, dim3(blocks), dim3(256), 0, stream, a, splits, per, units, per_xcd, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid((kH * (kDv / 8) + 255) / 256, rows);
  if (splits <= 2)
    hipLaunchKernelGGL(mla_combine_kernel<2>, cgrid, dim3(256), 0, stream, a, splits, units, ws);
  else if (splits <= 16)
    hipLaunchKernelGGL(mla_combine_kernel<16>, cgrid, dim3(256), 0, stream, a, splits, units, ws);
  else
    hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, dim3(256), 0, stream, a, splits, units, ws);
  return hipGetLastError();
}

}  // namespace dsa
