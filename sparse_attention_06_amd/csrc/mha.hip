// mha.hip -- expanded multi-head attention for prefill blocks on gfx950: the dense fallback for
// short prefill, dense causal or restricted to an index set (the masked MHA mode).
//
// Page references:
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io), section "稀疏注意力：NSA 与 DSA":
//               the cost model's expanded pair (per head a 128-dim key plus the 64-dim rope part,
//               a 128-dim value), and the note that short prefill prefers dense expanded MHA, with
//               V3.2 emulating DSA in a masked MHA mode
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org), section
//               "Sparse Attention": softmax(QK^T/sqrt(d_h) + M^DSA)V, M = 0 on S_t, -inf elsewhere
//
// Operands (bf16): q [rows, H, 192] (128 + 64 rope per head); per sequence s the head-major
// k_nope [s][h][j][128] and v [s][h][j][128], and the rope keys k_rope [s][j][64] shared by all
// heads. The index set, when given, is first turned into one bit per (row, position).
//
// Tuned kernel: one workgroup = 8 waves per (sequence, head, block of 256 query rows), two waves
// per SIMD; wave w owns rows 32w .. 32w+31. Per tile of 32 positions (v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T   key rows as the A operand from LDS (all 12 K steps fetched before the MFMAs),
//                 the wave's 32 queries as B operands resident in registers; lane l ends up with
//                 query l%32 and 16 of the 32 keys
//   softmax      fp32 in the log2 domain with a lazily moved reference maximum (the running
//                 output is rescaled only when a row's maximum grows by more than 2^8)
//   O^T += V^T P  V^T through ds_read_b64_tr_b16 transpose reads, P from registers
// The two waves on a SIMD interleave one's softmax with the other's MFMAs. Tiles (keys, values
// and, in the masked mode, the 256 rows' mask words) are double-buffered in LDS; the next tile is
// loaded into registers while the current one is computed and written to LDS behind it.
#include "dsa_internal.h"

namespace dsa {

constexpr int kMhaDn = 128, kMhaDr = 64, kMhaDq = kMhaDn + kMhaDr, kMhaDv = 128;
constexpr int kMhaBN = 32;                  // positions per tile
constexpr int kMhaWaves = 8;
constexpr int kMhaThreads = 64 * kMhaWaves;
constexpr int kMhaBM = 32 * kMhaWaves;      // query rows per workgroup
constexpr int kMhaNopeOff = 0;              // [32 keys][256 B], 16-byte chunk c at c ^ (key % 16)
constexpr int kMhaRopeOff = kMhaBN * 256;   // [32 keys][128 B], chunk c at c ^ ((key / 2) % 8)
constexpr int kMhaVOff = kMhaRopeOff + kMhaBN * 128;  // [32 keys][256 B], chunk c at c ^ (4 * (key % 4))
constexpr int kMhaMaskOff = kMhaVOff + kMhaBN * 256;  // [256 rows] mask word of the tile
constexpr int kMhaStageBytes = kMhaMaskOff + 4 * kMhaBM;  // 21 KB
constexpr int kMhaLdsBytes = 2 * kMhaStageBytes;
constexpr float kMhaLog2e = 1.4426950408889634f;
// A row's softmax reference moves only when a logit exceeds it by 2^8 (log2 units): probabilities
// stay below 2^8 and sums of up to 2^31 of them times |v| stay far inside the fp32 range.
constexpr float kMhaRescale = 8.0f;

typedef __attribute__((address_space(3))) uint8_t mha_lds;

struct MhaArgs {
  const uint16_t* q;
  const uint16_t* k_nope;
  const uint16_t* k_rope;
  const uint16_t* v;
  int64_t ld_kv;
  const int32_t* q_pos;
  int n_seq, q_per_seq, H;
  const uint32_t* mask;  // [rows][mask_words] bits of the index sets, or NULL (dense causal)
  int mask_words;
  float sm_scale;
  uint16_t* out;
  float* lse;
};

// ---------------------------------------------------------------- index set -> bitmap

// One workgroup per row: bit j of mask[r] is set iff position j in [0, q_pos[r]] is listed in
// idx[r] (a set: repeats and entries outside the visible range change nothing). The row is built
// in LDS and written whole, so the bitmap needs no clearing beforehand.
__global__ void __launch_bounds__(256) mha_mask_kernel(const int32_t* __restrict__ idx, int64_t ld_idx, int k,
                                                       const int32_t* __restrict__ q_pos, int words,
                                                       uint32_t* __restrict__ mask) {
  extern __shared__ uint32_t bits[];
  const int r = blockIdx.x;
  for (int i = threadIdx.x; i < words; i += 256) bits[i] = 0u;
  __syncthreads();
  const int t = q_pos[r];
  const int32_t* row = idx + (int64_t)r * ld_idx;
  for (int i = threadIdx.x; i < k; i += 256) {
    const int j = row[i];
    if (j >= 0 && j <= t && (j >> 5) < words) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t* dst = mask + (int64_t)r * words;
  for (int i = threadIdx.x; i < words; i += 256) dst[i] = bits[i];
}

// ---------------------------------------------------------------- attention

// What thread `tid` (of 512) moves for one tile: one 16-byte chunk of the nope keys, one of the
// values, one of the rope keys (threads 0..255) or the mask word of one query row (threads
// 256..511, masked mode). Key rows are clamped to the cache, so the loads stay inside it; LDS
// offsets are swizzled as the layout comment above says.
struct MhaTileRegs {
  i32x4 kn, v, kr;
  uint32_t mw;
};

__device__ __forceinline__ void mha_load_tile(MhaTileRegs& tr, const uint8_t* kn, const uint8_t* kr,
                                              const uint8_t* vv, const uint32_t* mask_row0, int mask_words,
                                              int mask_rows, int j0, int64_t ld_kv, int tid) {
  {
    const int row = tid >> 4, ch = tid & 15;
    const int64_t j = min((int64_t)(j0 + row), ld_kv - 1);
    tr.kn = *(const i32x4*)(kn + j * 256 + 16 * ch);
    tr.v = *(const i32x4*)(vv + j * 256 + 16 * ch);
  }
  if (tid < 256) {
    const int row = tid >> 3, ch = tid & 7;
    const int64_t j = min((int64_t)(j0 + row), ld_kv - 1);
    tr.kr = *(const i32x4*)(kr + j * 128 + 16 * ch);
  } else if (mask_row0) {
    const int i = tid - 256;
    tr.mw = i < mask_rows ? mask_row0[(int64_t)i * mask_words + j0 / kMhaBN] : 0u;
  }
}

__device__ __forceinline__ void mha_store_tile(const MhaTileRegs& tr, mha_lds* st, bool masked, int tid) {
  {
    const int row = tid >> 4, ch = tid & 15;
    *(__attribute__((address_space(3))) i32x4*)(st + kMhaNopeOff + row * 256 + 16 * (ch ^ (row & 15))) = tr.kn;
    *(__attribute__((address_space(3))) i32x4*)(st + kMhaVOff + row * 256 + 16 * (ch ^ (4 * (row & 3)))) = tr.v;
  }
  if (tid < 256) {
    const int row = tid >> 3, ch = tid & 7;
    *(__attribute__((address_space(3))) i32x4*)(st + kMhaRopeOff + row * 128 + 16 * (ch ^ ((row >> 1) & 7))) = tr.kr;
  } else if (masked) {
    *(__attribute__((address_space(3))) uint32_t*)(st + kMhaMaskOff + 4 * (tid - 256)) = tr.mw;
  }
}

__global__ void __launch_bounds__(kMhaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mha_fwd_kernel(MhaArgs a, int qblocks, int units, int per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kMhaLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups go to the 8 XCDs round robin: give each XCD a contiguous range of units, so the
  // query blocks of one head share that XCD's L2 for the head's keys and values. Within a head the
  // longest (last) query block comes first.
  const int unit = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (unit >= units) return;
  const int qb = qblocks - 1 - unit % qblocks;
  const int sh = unit / qblocks, h = sh % a.H, s = sh / a.H;
  const int row0 = s * a.q_per_seq + qb * kMhaBM;
  const int nrows = min(kMhaBM, a.q_per_seq - qb * kMhaBM);
  const int hl = lane & 31, half = lane >> 5;
  const bool masked = a.mask != nullptr;

  // this lane's row (query hl of the wave's 32); positions past the cache see only the cache,
  // rows past the block's end see nothing and store nothing
  const int qi = 32 * wave + hl;
  const int64_t r_lane = row0 + min(qi, nrows - 1);
  const bool row_ok = qi < nrows;
  const int t_lane = row_ok ? min(a.q_pos[r_lane], (int)(a.ld_kv - 1)) : -1;
  // the workgroup's key range: [0, max t]; tiles wholly at or below min t need no causal mask
  __shared__ int red[2][kMhaWaves];
  {
    int mx = t_lane, mn = row_ok ? t_lane : INT32_MAX;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      mx = max(mx, __shfl_xor(mx, o));
      mn = min(mn, __shfl_xor(mn, o));
    }
    if (lane == 0) { red[0][wave] = mx; red[1][wave] = mn; }
  }
  __syncthreads();
  int t_max = red[0][0], t_min = red[1][0];
#pragma unroll
  for (int w = 1; w < kMhaWaves; ++w) { t_max = max(t_max, red[0][w]); t_min = min(t_min, red[1][w]); }
  const int ntiles = t_max < 0 ? 0 : t_max / kMhaBN + 1;

  // queries as B operands: qf[ks] = dims 16ks + 8*half .. +8 of this lane's row
  bf16x8 qf[kMhaDq / 16];
  {
    const uint16_t* qr = a.q + (r_lane * a.H + h) * kMhaDq + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kMhaDq / 16; ++ks) qf[ks] = *(const bf16x8*)(qr + 16 * ks);
  }
  f32x16 o[kMhaDv / 32];
#pragma unroll
  for (int mt = 0; mt < kMhaDv / 32; ++mt) o[mt] = f32x16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  const float c_scale = a.sm_scale * kMhaLog2e;

  const uint8_t* kn = (const uint8_t*)(a.k_nope + ((int64_t)s * a.H + h) * a.ld_kv * kMhaDn);
  const uint8_t* kr = (const uint8_t*)(a.k_rope + (int64_t)s * a.ld_kv * kMhaDr);
  const uint8_t* vv = (const uint8_t*)(a.v + ((int64_t)s * a.H + h) * a.ld_kv * kMhaDv);
  const uint32_t* mask_row0 = masked ? a.mask + (int64_t)row0 * a.mask_words : nullptr;
  mha_lds* lds = (mha_lds*)smem;

  // per-lane LDS offsets within a stage
  const int nope_base = kMhaNopeOff + hl * 256;  // QK^T A operand: key row lane%32, chunk 2ks + half
  const int rope_base = kMhaRopeOff + hl * 128;
  // PV transpose reads (lane group G = lane/16, lane j in it; read a8 of K step ks): key row
  // 16ks + 8a8 + 4(G/2) + j/4, value columns 32mt + 16(G%2) + 4(j%4) .. +4, i.e. chunk
  // 4mt + 2(G%2) + (j%4)/2 stored at 4(mt ^ (j/4)) + 2(G%2) + (j%4)/2 of its row
  int tr_off[kMhaDv / 32];
  {
    const int G = lane >> 4, j = lane & 15;
    const int row = 4 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int mt = 0; mt < kMhaDv / 32; ++mt)
      tr_off[mt] = kMhaVOff + row * 256 + 16 * (4 * (mt ^ (j >> 2)) + 2 * (G & 1) + ((j & 3) >> 1)) + 8 * (j & 1);
  }

  MhaTileRegs nxt;
  nxt.mw = 0u;
  if (ntiles > 0) {
    mha_load_tile(nxt, kn, kr, vv, mask_row0, a.mask_words, nrows, 0, a.ld_kv, tid);
    mha_store_tile(nxt, lds, masked, tid);
    if (ntiles > 1) mha_load_tile(nxt, kn, kr, vv, mask_row0, a.mask_words, nrows, kMhaBN, a.ld_kv, tid);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * kMhaBN;
    const mha_lds* st = lds + (it & 1) * kMhaStageBytes;
    // ---- S^T = K Q^T: the 12 key fragments first, then the MFMAs
    bf16x8 kf[kMhaDq / 16];
#pragma unroll
    for (int ks = 0; ks < kMhaDq / 16; ++ks) {
      const int c = 2 * (ks & 7) + half;
      kf[ks] = ks < 8
          ? *(const __attribute__((address_space(3))) bf16x8*)(st + nope_base + 16 * (c ^ (hl & 15)))
          : *(const __attribute__((address_space(3))) bf16x8*)(st + rope_base + 16 * (c ^ ((hl >> 1) & 7)));
    }
    f32x16 sv = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kMhaDq / 16; ++ks) sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], sv, 0, 0, 0);
    // ---- mask and softmax bookkeeping; lane holds keys j0 + 8(i/4) + 4*half + i%4
    if (masked || j0 + kMhaBN - 1 > t_min) {
      const uint32_t bits = masked ? *(const __attribute__((address_space(3))) uint32_t*)(st + kMhaMaskOff + 4 * min(qi, kMhaBM - 1))
                                   : 0xffffffffu;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + 4 * half + (i & 3);
        const bool ok = (j0 + kk <= t_lane) && ((bits >> kk) & 1u);
        sv[i] = ok ? sv[i] : -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]))) * c_scale;
    }
    if (mx > m_ref + kMhaRescale) {
      const float alpha = m_ref == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_ref - mx);
      m_ref = mx;
      l_sum *= alpha;
#pragma unroll
      for (int mt = 0; mt < kMhaDv / 32; ++mt) o[mt] *= alpha;
    }
    // a row with no key seen yet has every logit of this tile at -inf: any finite reference
    // then gives p = 0 (and -inf - (-inf) would not)
    const float ref = m_ref == -INFINITY ? 0.f : m_ref;
    bf16x8 pk[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[8 * ks + e], c_scale, -ref));  // exp2(-inf) = 0
        l_sum += pv[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[ks][e] = (__bf16)pv[e];
    }
    // ---- O^T += V^T P: K step ks takes keys 16ks + 8(e/4) + 4*half + e%4 in slot 8*half + e, the
    //      order in which pk holds them
    bf16x8 vf[2][kMhaDv / 32];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mt = 0; mt < kMhaDv / 32; ++mt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(st + tr_off[mt] + ks * 16 * 256));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(st + tr_off[mt] + ks * 16 * 256 + 8 * 256));
        vf[ks][mt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mt = 0; mt < kMhaDv / 32; ++mt)
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks][mt], pk[ks], o[mt], 0, 0, 0);
    // ---- the next tile into the other stage (last read in the previous iteration), then fetch
    //      the one after it
    if (it + 1 < ntiles) {
      mha_store_tile(nxt, lds + ((it + 1) & 1) * kMhaStageBytes, masked, tid);
      if (it + 2 < ntiles)
        mha_load_tile(nxt, kn, kr, vv, mask_row0, a.mask_words, nrows, j0 + 2 * kMhaBN, a.ld_kv, tid);
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds value columns 32mt + 8(i/4) + 4*half + i%4 of its row
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* dst = a.out + (r_lane * a.H + h) * kMhaDv + 4 * half;
#pragma unroll
  for (int mt = 0; mt < kMhaDv / 32; ++mt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16 ov = o[mt];
      const uint32_t w0 = (uint32_t)f32_to_bf16(ov[4 * g] * inv) | ((uint32_t)f32_to_bf16(ov[4 * g + 1] * inv) << 16);
      const uint32_t w1 = (uint32_t)f32_to_bf16(ov[4 * g + 2] * inv) | ((uint32_t)f32_to_bf16(ov[4 * g + 3] * inv) << 16);
      *(uint2*)(dst + 32 * mt + 8 * g) = make_uint2(w0, w1);
    }
  if (a.lse && half == 0) a.lse[r_lane * a.H + h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) / kMhaLog2e : -INFINITY;
}

size_t mha_ws_bytes(int rows, int max_ctx, bool has_idx) {
  if (!has_idx || rows <= 0) return 0;
  const size_t words = (size_t)(max_ctx + kMhaBN - 1) / kMhaBN;
  return (size_t)rows * words * 4;
}

hipError_t launch_mha(const uint16_t* q, const uint16_t* k_nope, const uint16_t* k_rope, const uint16_t* v,
                      int64_t ld_kv, const int32_t* q_pos, int n_seq, int q_per_seq, const int32_t* idx,
                      int64_t ld_idx, int k, int H, int max_ctx, float sm_scale, uint16_t* out, float* lse,
                      void* ws, hipStream_t stream) {
  MhaArgs a{};
  a.q = q; a.k_nope = k_nope; a.k_rope = k_rope; a.v = v; a.ld_kv = ld_kv; a.q_pos = q_pos;
  a.n_seq = n_seq; a.q_per_seq = q_per_seq; a.H = H; a.sm_scale = sm_scale; a.out = out; a.lse = lse;
  const int rows = n_seq * q_per_seq;
  if (idx) {
    const int words = (max_ctx + kMhaBN - 1) / kMhaBN;
    a.mask = (const uint32_t*)ws;
    a.mask_words = words;
    hipLaunchKernelGGL(mha_mask_kernel, dim3(rows), dim3(256), (size_t)words * 4, stream, idx, ld_idx, k, q_pos,
                       words, (uint32_t*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int qblocks = (q_per_seq + kMhaBM - 1) / kMhaBM;
  const int units = n_seq * H * qblocks;
  const int per_xcd = (units + 7) / 8;
  hipLaunchKernelGGL(mha_fwd_kernel, dim3(8 * per_xcd), dim3(kMhaThreads), 0, stream, a, qblocks, units, per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
