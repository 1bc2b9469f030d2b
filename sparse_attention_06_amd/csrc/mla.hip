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
//            global_load_lds_dwordx4 (no VGPR staging), three tiles in flight; rows sit at a
//            1168-byte stride so both LDS read patterns below are bank-conflict free
//   QK^T     S[32 keys x 32 heads] on v_mfma_f32_32x32x16_bf16: the key tile is the A operand
//            (read from LDS), the wave's 32 query heads the B operand (resident in 144 VGPRs)
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

// ------------------------------------------------------------------ generic (any shape)

// One wave per (row, head); lanes stride the feature dims. Online softmax in fp32.
__global__ void __launch_bounds__(256) mla_generic_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows = a.n_seq * a.q_per_seq;
  if (gw >= rows * a.H) return;
  const int r = gw / a.H, h = gw % a.H;
  const int t = a.q_pos[r], seq = r / a.q_per_seq;
  const uint16_t* qh = a.q + ((int64_t)r * a.H + h) * a.Dqk;
  float qv[16], o[8];
#pragma unroll
  for (int i = 0; i < 16; ++i) { int c = lane + 64 * i; qv[i] = c < a.Dqk ? bf16_to_f32(qh[c]) : 0.f; }
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int n = a.idx ? a.k : min(t + 1, a.k);  // dense: a.k = max_ctx
  const uint16_t* kv = (const uint16_t*)a.kv.base;
  for (int e = 0; e < n; ++e) {
    const int j = a.idx ? a.idx[(int64_t)r * a.ld_idx + e] : e;
    if (j < 0 || j > t) continue;
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
  const int waves = a.n_seq * a.q_per_seq * a.H;
  hipLaunchKernelGGL(mla_generic_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tuned MFMA kernel

constexpr int kH = 128, kDqk = 576, kDv = 512;
constexpr int kHG = 64;                          // heads per workgroup (two workgroups per row)
constexpr int kNK = 32;                          // positions per tile
constexpr int kRowBytes = kDqk * 2;              // 1152 = 1024 latent + 128 rope
constexpr int kLatBytes = 1024;                  // dims 0..511: one wave-wide 16-byte load
constexpr int kRopeBytes = 128;                  // dims 512..575: 8 chunks of 16 bytes
constexpr int kRopeOff = kNK * kLatBytes;        // 32768: rope region of a tile
constexpr int kTileBytes = kRopeOff + kNK * kRopeBytes;  // 36864
constexpr int kRowsPerWave = kNK / 4;            // 8 rows gathered by each wave
constexpr int kInstrPerWave = kRowsPerWave + 1;  // 8 latent loads + 1 rope load
constexpr int kNBuf = 3;
constexpr int kListCap = 2048;                   // resolved entries held in LDS at a time
constexpr int kListOff = kNBuf * kTileBytes;     // 110592
constexpr int kLdsBytes = kListOff + 4 * kListCap;  // 118784
static_assert(kHG * kDv * 2 <= kLdsBytes, "output staging");
constexpr float kLog2e = 1.4426950408889634f;
// The softmax reference of a head moves only when a logit exceeds it by 2^64 (log2 units):
// fp32 and bf16 share an exponent range of 2^+-126, so probabilities up to 2^64 and sums of
// 2048 of them times |v| stay finite, and terms far below the reference are negligible anyway.
constexpr float kRescaleThreshold = 64.0f;

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

// LDS swizzles (64 banks of 4 bytes). Latent part: tile row r keeps 16-byte chunk c at position
// c ^ lat_swz(r) of its 1 KB line, so the 16 rows read together by a QK^T operand fetch, and the
// 4 rows x 2 chunks of a transpose read, fall on distinct banks. Rope part: row r keeps chunk
// c (0..7) at position c ^ rope_swz(r) of its 128-byte line.
__device__ __forceinline__ int lat_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }

// Physical row of entry e of row r (sparse: position idx[r, e]; dense: position e), or -1 when
// the position is not visible or its page id is invalid.
__device__ __forceinline__ int resolve_entry(const AttnArgs& a, int r, int seq, int t, int e) {
  const int j = a.idx ? a.idx[(int64_t)r * a.ld_idx + e] : e;
  if (j < 0 || j > t) return -1;
  const int64_t row = phys_row(a.kv.page_table, a.kv.ld_pt, a.kv.page_size, a.kv.num_pages, seq, j);
  return (int)row;  // caches hold < 2^31 rows
}

// One wave-wide global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes
// land at LDS byte address lds_base + 16 * l; lds_base must be wave-uniform. Issued from inline
// asm so that the compiler's wait-count pass does not treat these LDS writes as aliasing every
// later LDS read (it would drain all in-flight tiles before each one); the tile loop waits for
// them explicitly instead. The instruction writes no VGPR; M0 is saved and restored.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr)
      : "memory");
}

// This wave's share of one tile gather: tile rows 8w..8w+7, as 8 wave-wide latent loads (lane l
// fetches chunk l ^ lat_swz(row)) and one rope load (lane l: row 8w + l/8, chunk
// (l%8) ^ rope_swz(row)). Every lane is active in every load, so each wave has exactly
// kInstrPerWave loads in flight per tile. Rows of invalid entries load the tile's first valid
// row instead (finite data; their probability is 0).
__device__ __forceinline__ void gather_tile(const uint8_t* __restrict__ kv_base, lds_u8* buf,
                                            const int* list, int n_in_tile, uint32_t vmask,
                                            int wave, int lane) {
  // An opaque copy of the lane id: the per-lane offsets below are recomputed per tile (a few
  // VALU ops) instead of being hoisted out of the tile loop into long-lived registers.
  asm volatile("" : "+v"(lane));
  const int dummy = __builtin_amdgcn_readfirstlane(list[__ffs(vmask) - 1]);
  const int my_slot = kRowsPerWave * wave + (lane >> 3);
  int my_rid = my_slot < n_in_tile ? list[my_slot] : -1;
  my_rid = my_rid < 0 ? dummy : my_rid;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int row = kRowsPerWave * wave + i;
    const int rid = __builtin_amdgcn_readfirstlane(__shfl(my_rid, 8 * i));
    const uint8_t* src = kv_base + (int64_t)rid * kRowBytes + 16 * (lane ^ lat_swz(row));
    lds_dma16(src, (uint32_t)(uintptr_t)(buf + row * kLatBytes));
  }
  const uint8_t* src = kv_base + (int64_t)my_rid * kRowBytes + kLatBytes + 16 * ((lane & 7) ^ rope_swz(my_slot));
  lds_dma16(src, (uint32_t)(uintptr_t)(buf + kRopeOff + kRowsPerWave * wave * kRopeBytes));
}

__device__ __forceinline__ void wait_gathers(bool keep_one_tile) {
  // vmcnt(kInstrPerWave) leaves the younger tile's loads in flight; vmcnt(0) drains
  if (keep_one_tile) __builtin_amdgcn_s_waitcnt(0x0F70 | kInstrPerWave);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Rare path (a head's maximum grew past its reference by more than the threshold): scale the
// running output. Out of line, so that the hot loop keeps its accumulators in AGPRs.
__device__ __attribute__((noinline)) void rescale_acc(f32x4* o, float alpha) {
  for (int mt = 0; mt < kDv / 16; ++mt) o[mt] *= alpha;
}

// Block -> (unit, head half): the two halves of a unit (row, split) get block ids b and b + 8,
// which the dispatcher places on the same XCD back to back, so the second gather of each
// latent row is an L2 hit.
__device__ __forceinline__ void block_unit(int b, int units, int& unit, int& half) {
  const int grp = b >> 4, in = b & 15;
  unit = grp * 8 + (in & 7);
  half = in >> 3;
  (void)units;
}

template <bool kSplit>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_mfma_kernel(AttnArgs a, int splits, int entries_per_split, int units, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int unit, half;
  block_unit(blockIdx.x, units, unit, half);
  if (unit >= units) return;
  const int r = unit / splits, sp = unit % splits;
  const int seq = r / a.q_per_seq;
  const int t = a.q_pos[r];
  const int n_entries = a.idx ? a.k : max(0, min(t + 1, a.k));  // dense: a.k = max_ctx
  const int e_begin = sp * entries_per_split;
  const int e_end = min(n_entries, e_begin + entries_per_split);
  lds_u8* lds = (lds_u8*)smem;
  int* list = (int*)(smem + kListOff);
  const int head0 = kHG * half + 16 * wave;  // this wave's 16 heads

  // query heads as B operands: lane holds head head0 + lane%16, dims 32*ks + 8*(lane/16) .. +8
  bf16x8 qf[kDqk / 32];
  {
    const uint16_t* qh = a.q + ((int64_t)r * kH + head0 + (lane & 15)) * kDqk + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *(const bf16x8*)(qh + 32 * ks);
    // consume the fragments here, so their loads are complete before the tile loop and no wait
    // for them lands inside it (where it would also drain the in-flight tile gathers)
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  f32x4 o[kDv / 16];
#pragma unroll
  for (int mt = 0; mt < kDv / 16; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // l_part sums the bf16-rounded probabilities the PV product uses (it normalises the output);
  // l_exact sums them unrounded (it gives the log-sum-exp)
  float m_ref = -INFINITY, l_part = 0.f, l_exact = 0.f;
  const float c_scale = a.sm_scale * kLog2e;
  const uint8_t* kv_base = (const uint8_t*)a.kv.base;

  // Per-lane LDS byte offsets of the operand fetches within a tile. The swizzles only touch the
  // low bits of the K step / column block, the rest folds into immediates.
  int g1_base[4], rope_base[2], tr_base[8];
  {
    const int g = lane >> 4, j = lane & 15;
    const int S = lat_swz(j);              // rows j and 16 + j share the swizzle
    // QK^T: row 16*st + j, chunk 4*ks + g
#pragma unroll
    for (int k3 = 0; k3 < 4; ++k3) g1_base[k3] = j * kLatBytes + 16 * (4 * (k3 ^ (S >> 2)) + (g ^ (S & 3)));
    const int R = rope_swz(j);
#pragma unroll
    for (int k1 = 0; k1 < 2; ++k1) rope_base[k1] = kRopeOff + j * kRopeBytes + 16 * ((4 * k1 + g) ^ R);
    // transpose reads: row 16*a + 4*g + j/4, column chunk 2*mt + (j%4)/2, half (j%2)
    const int rr = 4 * g + (j >> 2);
    const int T = lat_swz(rr);
#pragma unroll
    for (int m7 = 0; m7 < 8; ++m7)
      tr_base[m7] = rr * kLatBytes + 16 * (2 * (m7 ^ (T >> 1)) + (((j & 3) >> 1) ^ (T & 1))) + 8 * (j & 1);
  }

  for (int cb = e_begin; cb < e_end; cb += kListCap) {
    const int ce = min(e_end, cb + kListCap);
    __syncthreads();  // the previous chunk is done with the list and the buffers
    for (int e = cb + threadIdx.x; e < ce; e += 256) list[e - cb] = resolve_entry(a, r, seq, t, e);
    __syncthreads();
    const int n_list = ce - cb;
    const int ntiles = (n_list + kNK - 1) / kNK;
    uint32_t vmask[kNBuf];
    auto tile_mask = [&](int ti) -> uint32_t {
      const int e = ti * kNK + lane;
      const bool v = lane < kNK && e < n_list && list[e] >= 0;
      return (uint32_t)__ballot(v);
    };
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      if (pt < ntiles) {
        vmask[pt] = tile_mask(pt);
        if (vmask[pt]) gather_tile(kv_base, lds + pt * kTileBytes, list + pt * kNK, n_list - pt * kNK, vmask[pt], wave, lane);
      }
    }
    for (int it = 0; it < ntiles; ++it) {
      const int b = it % kNBuf;
      const bool next_in_flight = it + 1 < ntiles && vmask[(it + 1) % kNBuf] != 0u;
      wait_gathers(next_in_flight);
      // Every wave's share of tile `it` has landed once all waves pass this barrier, and all of
      // tile it-1's LDS reads were consumed by MFMAs already. A bare s_barrier: the fence of
      // __syncthreads would also drain the younger tile's loads that are meant to stay in flight.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (it + 2 < ntiles) {
        const int nb = (it + 2) % kNBuf;
        vmask[nb] = tile_mask(it + 2);
        if (vmask[nb]) gather_tile(kv_base, lds + nb * kTileBytes, list + (it + 2) * kNK, n_list - (it + 2) * kNK, vmask[nb], wave, lane);
      }
      const uint32_t valid = vmask[b];
      if (valid == 0u) continue;
      const lds_u8* tile = lds + b * kTileBytes;

      // ---- S = K Q^T for two 16-key halves: lane holds head lane%16,
      //      keys 16*st + 4*(lane/16) + i, i = 0..3
      f32x4 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kDv / 32; ++ks) {
          const lds_u8* p = tile + g1_base[ks & 3] + 16384 * st + 64 * (ks & 12);
          const bf16x8 af = *(const __attribute__((address_space(3))) bf16x8*)p;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int ks = kDv / 32; ks < kDqk / 32; ++ks) {
          const lds_u8* p = tile + rope_base[ks - kDv / 32] + 2048 * st;
          const bf16x8 af = *(const __attribute__((address_space(3))) bf16x8*)p;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[ks], acc, 0, 0, 0);
        }
        s[st] = acc;
      }
      // ---- softmax bookkeeping (log2 domain)
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * st + 4 * (lane >> 4) + i;
          const float v = ((valid >> key) & 1u) ? s[st][i] * c_scale : -INFINITY;
          s[st][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m_ref + kRescaleThreshold;
      if (__any(need)) {
        const float nref = need ? mx : m_ref;
        const float alpha = need ? exp2f(m_ref - nref) : 1.f;  // m_ref = -inf gives 0
        if (__any(alpha != 1.f && l_part != 0.f)) {
          f32x4 tmp[kDv / 16];
#pragma unroll
          for (int mt = 0; mt < kDv / 16; ++mt) tmp[mt] = o[mt];
          rescale_acc(tmp, alpha);
#pragma unroll
          for (int mt = 0; mt < kDv / 16; ++mt) o[mt] = tmp[mt];
          // settle the reloads here, so no wait for them is left on the hot path after the join
          __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        l_part *= alpha;
        l_exact *= alpha;
        m_ref = nref;
      }
      bf16x8 pf;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = (m_ref == -INFINITY) ? 0.f : exp2f(s[st][i] - m_ref);
          const __bf16 pb = (__bf16)p;
          l_part += (float)pb;
          l_exact += p;
          pf[4 * st + i] = pb;
        }
      // ---- O^T += V^T P : A = V^T via transpose reads; lane group g reads keys 4g..4g+3
      //      and 16+4g..16+4g+3, matching the key order of the P fragment
#pragma unroll
      for (int mt = 0; mt < kDv / 16; ++mt) {
        const lds_u8* p0 = tile + tr_base[mt & 7] + 32 * (mt & 24);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0 + 16 * kLatBytes));
        // whole-vector reinterpretation (element-wise bit casts of the 16-bit lanes were
        // miscompiled into a broadcast of element 0)
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[mt], 0, 0, 0);
      }
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float l_ex = l_exact + __shfl_xor(l_exact, 16);
  l_ex += __shfl_xor(l_ex, 32);
  const int hl = 16 * wave + (lane & 15);   // head within this workgroup's 64
  const int head = kHG * half + hl;
  if (!kSplit) {
    // normalise, stage [head][vdim] bf16 in LDS (64 KB), then coalesced 16-byte stores
    __syncthreads();
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* st = (uint16_t*)smem;
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[hl * kDv + 16 * mt + 4 * (lane >> 4) + i] = f32_to_bf16(o[mt][i] * inv);
    __syncthreads();
    i32x4* dst = (i32x4*)(a.out + ((int64_t)r * kH + kHG * half) * kDv);
    for (int i = threadIdx.x; i < kHG * kDv / 8; i += 256) dst[i] = ((const i32x4*)smem)[i];
    if (a.lse && lane < 16) a.lse[(int64_t)r * kH + head] = l_ex > 0.f ? (m_ref + __log2f(l_ex)) / kLog2e : -INFINITY;
  } else {
    // partial result of this split: unnormalised O as [unit][head][vdim] fp32, plus
    // (m_ref, rounded sum, exact sum) per head
    float* po = ws + ((int64_t)unit * kH + head) * kDv;
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt)
      *(f32x4*)(po + 16 * mt + 4 * (lane >> 4)) = o[mt];
    float* pm = ws + (int64_t)units * kH * kDv + ((int64_t)unit * kH + head) * 4;
    if (lane < 16) { pm[0] = m_ref; pm[1] = l_tot; pm[2] = l_ex; }
  }
}

// Merge the splits of each row: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One thread per (row, head, 8 output columns).
__global__ void __launch_bounds__(256) mla_combine_kernel(AttnArgs a, int splits, int units, const float* __restrict__ ws) {
  const int r = blockIdx.y;
  const int item = blockIdx.x * 256 + threadIdx.x;  // head * 64 + column group
  if (item >= kH * (kDv / 8)) return;
  const int head = item / (kDv / 8), cg = item % (kDv / 8);
  const float* pm = ws + (int64_t)units * kH * kDv;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pm[((int64_t)(r * splits + s) * kH + head) * 4]);
  float den = 0.f, den_ex = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s = 0; s < splits; ++s) {
    const int64_t u = (int64_t)(r * splits + s) * kH + head;
    const float m = pm[u * 4], l = pm[u * 4 + 1];
    if (l <= 0.f) continue;
    const float f = exp2f(m - M);
    den += f * l;
    den_ex += f * pm[u * 4 + 2];
    const f32x4* po = (const f32x4*)(ws + u * kDv + 8 * cg);
    const f32x4 v0 = po[0], v1 = po[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { acc[e] = fmaf(f, v0[e], acc[e]); acc[e + 4] = fmaf(f, v1[e], acc[e + 4]); }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* dst = a.out + ((int64_t)r * kH + head) * kDv + 8 * cg;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (uint32_t)f32_to_bf16(acc[2 * e] * inv) | ((uint32_t)f32_to_bf16(acc[2 * e + 1] * inv) << 16);
  *(i32x4*)dst = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  if (a.lse && cg == 0) a.lse[(int64_t)r * kH + head] = den_ex > 0.f ? (M + __log2f(den_ex)) / kLog2e : -INFINITY;
}

size_t mla_mfma_ws_bytes(int rows, int splits) {
  if (splits <= 1) return 0;
  return (size_t)rows * splits * kH * (kDv + 4) * sizeof(float);
}

int mla_mfma_pick_splits(int rows, int k) {
  // aim for >= 256 workgroups (two per (row, split)), at least 2 tiles per split
  int s = 1;
  while (2 * rows * s < 256 && (k / (s * 2)) >= 2 * kNK) s *= 2;
  return s;
}

hipError_t launch_mla_mfma(const AttnArgs& a, int splits, void* ws, hipStream_t stream) {
  const int rows = a.n_seq * a.q_per_seq;
  const int units = rows * (splits > 1 ? splits : 1);
  const int blocks = ((units + 7) / 8) * 16;  // groups of 8 units x 2 head halves
  if (splits <= 1) {
    const int per = a.idx ? a.k : 1 << 30;
    hipLaunchKernelGGL(mla_mfma_kernel<false>, dim3(blocks), dim3(256), 0, stream, a, 1, per, units, (float*)nullptr);
    return hipGetLastError();
  }
  const int per = ((a.k + splits - 1) / splits + kNK - 1) / kNK * kNK;
  hipLaunchKernelGGL(mla_mfma_kernel<true>, dim3(blocks), dim3(256), 0, stream, a, splits, per, units, (float*)ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((kH * (kDv / 8) + 255) / 256, rows), dim3(256), 0, stream, a, splits, units, (const float*)ws);
  return hipGetLastError();
}

}  // namespace dsa
