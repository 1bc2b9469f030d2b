// topk.hip -- exact per-row top-k on gfx950.
//
// Page references:
//   [DSA-blog]  "DeepSeek Sparse Attention：从 SWA 到稀疏 Attention 计算" (kevinye.org),
//               section "Lightning Indexer": S_t = TopK_{j<=t}(I_tj, k)
//   [Handbook]  "MTP 与稀疏注意力：NSA 与 DSA" (anrans.github.io): k = min(L, 2048), so a prefix
//               shorter than k keeps every position
//
// Selection order: larger score first, equal scores by smaller position (so S_t is unique);
// -0 and +0 are equal. Output: the selected positions in ascending order, -1 padding to k.
//
// Method: one workgroup (16 waves) per row. Scores map to order-preserving 32-bit keys; four
// 8-bit radix passes (per-wave LDS histograms, then a suffix scan over the 256 digits) find the
// k-th largest key tau and how many keys equal to tau are taken. A final pass walks the row in
// index order, 1024 positions at a time: wave ballots of "key > tau" and "key == tau" give
// every lane its rank among the equal keys and its output slot, so the result is written in
// ascending position order with no sort. Rows that fit in LDS are staged there once; longer
// rows are re-read from global memory (L2) on each pass.
//
// Rows of at most 16384 positions take a register-resident variant: each of the 1024 threads
// holds 16 consecutive keys, so the row is read once. Three passes over 11-, 11- and 10-bit
// digits each fill a 2048-bin LDS histogram; a lane adds its keys that repeat one digit with a
// single atomic (the leading digit of real scores is nearly constant, and one atomic per key would
// serialise on it), and one wave picks the digit with DPP scans over coarse then fine bins. After a pass only keys sharing the decided top bits of
// the k-th largest remain undecided; once they fit, they are compacted into LDS and the remaining
// passes run over them alone. The output is one pass: a block-wide scan of each thread's
// "greater than" and "equal" counts gives every thread its first output slot and its rank among
// the equal keys.
#include "dsa_internal.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkLdsCap = 32768;  // positions staged in LDS (128 KB)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ scores,
                                                            int64_t ld_scores,
                                                            const int32_t* __restrict__ q_pos,
                                                            int max_ctx, int k,
                                                            int32_t* __restrict__ idx, int64_t ld_idx,
                                                            int lds_cap) {
  extern __shared__ uint32_t keys[];  // lds_cap entries
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ uint32_t cnt[2][kTopkWaves][2];
  __shared__ uint32_t sel_digit, sel_above;

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n = q_pos[r] + 1;
  n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
  int32_t* out = idx + (int64_t)r * ld_idx;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = scores + (int64_t)r * ld_scores;
  const bool in_lds = n <= lds_cap;
  if (in_lds)
    for (int i = tid; i < n; i += kTopkThreads) keys[i] = order_key(row[i]);

  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = in_lds ? keys[i] : order_key(row[i]);
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane owns digits 4*lane .. 4*lane+3; suffix sums over lanes give "count of larger digits"
      uint32_t c[4], local = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t s = 0;
        for (int w = 0; w < kTopkWaves; ++w) s += hist[w][4 * lane + e];
        c[e] = s;
        local += s;
      }
      uint32_t incl = local;  // inclusive suffix sum: sum over lanes >= this lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_down(incl, o);
        if (lane + o < 64) incl += v;
      }
      uint32_t above = incl - local;  // digits above this lane's block
      for (int e = 3; e >= 0; --e) {
        if (above < remaining && remaining <= above + c[e]) {
          sel_digit = 4 * lane + e;
          sel_above = above;
        }
        above += c[e];
      }
    }
    __syncthreads();
    remaining -= sel_above;
    prefix |= sel_digit << shift;
    pmask |= 255u << shift;
    __syncthreads();  // sel_* are rewritten by the next pass
  }
  const uint32_t tau = prefix;

  // ordered compaction: running counts of "== tau" and of selected positions before the chunk
  uint32_t run_eq = 0, run_sel = 0;
  int buf = 0;
  for (int base = 0; base < n; base += kTopkThreads, buf ^= 1) {
    const int i = base + tid;
    uint32_t key = 0;
    if (i < n) key = in_lds ? keys[i] : order_key(row[i]);
    const bool gt = i < n && key > tau;
    const bool eq = i < n && key == tau;
    const uint64_t gtm = __ballot(gt), eqm = __ballot(eq);
    if (lane == 0) {
      cnt[buf][wave][0] = __popcll(gtm);
      cnt[buf][wave][1] = __popcll(eqm);
    }
    __syncthreads();
    uint32_t eq_b = run_eq, sel_b = run_sel, eq_all = run_eq, sel_all = run_sel;
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t g = cnt[buf][w][0], e = cnt[buf][w][1];
      const uint32_t take = remaining > eq_all ? min(remaining - eq_all, e) : 0u;
      if (w < wave) { eq_b += e; sel_b += g + take; }
      eq_all += e;
      sel_all += g + take;
    }
    const uint32_t eq_rank = eq_b + __popcll(eqm & lanemask_lt(lane));
    const bool sel = gt || (eq && eq_rank < remaining);
    const uint64_t selm = __ballot(sel);
    const uint32_t slot = sel_b + __popcll(selm & lanemask_lt(lane));
    if (sel && slot < (uint32_t)k) out[slot] = i;
    run_eq = eq_all;
    run_sel = sel_all;
  }
}

// ---- register-resident variant (rows of at most kRegKeys positions)
constexpr int kRegE = 16;                         // consecutive keys per thread
constexpr int kRegKeys = kTopkThreads * kRegE;   // 16384
constexpr int kRegBins = 2048;                    // 11-bit digits: passes over bits 31..21, 20..10, 9..0
constexpr int kCandCap = 4096;                    // undecided keys compacted into LDS (also
                                                  // holds the k output positions, so k <= kCandCap)

__device__ __forceinline__ uint32_t digit_of(uint32_t key, int pass) {
  return pass == 0 ? key >> 21 : pass == 1 ? (key >> 10) & 2047u : key & 1023u;
}
__device__ __forceinline__ uint32_t mask_through(int pass) {  // key bits decided after `pass`
  return pass == 0 ? 0xFFE00000u : pass == 1 ? 0xFFFFFC00u : 0xFFFFFFFFu;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within rows of 16 lanes, then the row
// broadcasts carry row totals forward (DPP, no LDS round trip).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// hist[digit] += 1 for each active key. A lane adds all its keys that share the digit of its
// first active key with one atomic (the leading digits of real scores repeat a lot, and one
// atomic per key would serialise on the hot address); its other keys are added one by one.
__device__ __forceinline__ void hist_add_keys(uint32_t* hist, const uint32_t (&key)[kRegE], int cnt,
                                              uint32_t pmask, uint32_t prefix, int pass) {
  uint32_t d0 = 0, run = 0;
  bool have = false;
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    const bool act = e < cnt && (key[e] & pmask) == prefix;
    const uint32_t d = digit_of(key[e], pass);
    if (act && !have) { d0 = d; have = true; }
    run += (act && d == d0) ? 1u : 0u;
  }
  if (have) atomicAdd(&hist[d0], run);
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    const bool act = e < cnt && (key[e] & pmask) == prefix;
    const uint32_t d = digit_of(key[e], pass);
    if (act && d != d0) atomicAdd(&hist[d], 1u);
  }
}

// Wave 0 picks the digit of the remaining-th largest key from a 2048-bin histogram (digits in
// descending order): 64 coarse bins of 32 digits first, then the 32 digits of the chosen one.
// Publishes {digit, keys with larger digits, keys with that digit} in pub.
__device__ __forceinline__ void pick_digit_wave(const uint32_t* hist, uint32_t remaining, uint32_t* pub, int lane) {
  // lane l owns coarse bin 63 - l: digits 32 * (63 - l) .. + 31
  const int c = 63 - lane;
  uint32_t csum = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const uint4 q4 = *(const uint4*)(hist + 32 * c + 4 * v);
    csum += q4.x + q4.y + q4.z + q4.w;
  }
  const uint32_t cincl = wave_incl_scan(csum);
  const uint64_t cross = __ballot(cincl >= remaining);
  const int cl = __builtin_ctzll(cross);  // first lane (largest digits) reaching remaining
  const uint32_t above_c = __builtin_amdgcn_readlane(cincl - csum, cl);
  const int cc = 63 - cl;
  // lanes 0..31 own the chosen coarse bin's digits, largest first
  const uint32_t f = lane < 32 ? hist[32 * cc + 31 - lane] : 0u;
  const uint32_t fincl = wave_incl_scan(f) + above_c;
  const uint64_t fcross = __ballot(lane < 32 && fincl >= remaining);
  const int fl = __builtin_ctzll(fcross);
  if (lane == fl) {
    pub[0] = (uint32_t)(32 * cc + 31 - fl);
    pub[1] = fincl - f;
    pub[2] = f;
  }
}

__global__ void __launch_bounds__(kTopkThreads) topk_reg_kernel(const float* __restrict__ scores,
                                                                int64_t ld_scores,
                                                                const int32_t* __restrict__ q_pos,
                                                                int max_ctx, int k,
                                                                int32_t* __restrict__ idx, int64_t ld_idx) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[3][kRegBins];  // one histogram per pass
  __shared__ uint32_t cand_key[kCandCap], cand_pos[kCandCap];
  __shared__ uint32_t wtot[kTopkWaves][2];
  __shared__ uint32_t pub[3][3], ncand;

  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this thread's positions: p0 .. p0 + 15. The row is read before q_pos is known (every position
  // below max_ctx lies inside the row), so the two memory latencies overlap.
  const float* row = scores + (int64_t)r * ld_scores;
  const int p0 = kRegE * tid;
  float f[kRegE];
  if (p0 + kRegE <= max_ctx && ((uintptr_t)(row + p0) & 15) == 0) {
#pragma unroll
    for (int v = 0; v < kRegE / 4; ++v) {
      const float4 x = *(const float4*)(row + p0 + 4 * v);
      f[4 * v] = x.x; f[4 * v + 1] = x.y; f[4 * v + 2] = x.z; f[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kRegE; ++e) f[e] = p0 + e < max_ctx ? row[p0 + e] : 0.f;
  }
  int n = q_pos[r] + 1;
  n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
  int32_t* out = idx + (int64_t)r * ld_idx;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int cnt = n - p0 < 0 ? 0 : (n - p0 > kRegE ? kRegE : n - p0);
  uint32_t key[kRegE];
#pragma unroll
  for (int e = 0; e < kRegE; ++e) key[e] = e < cnt ? order_key(f[e]) : 0u;
  for (int i = tid; i < 3 * kRegBins; i += kTopkThreads) (&hist[0][0])[i] = 0;
  if (tid == 0) ncand = 0;
  __syncthreads();

  uint32_t prefix = 0, pmask = 0, remaining = (uint32_t)k;
  bool compacted = false;
  uint32_t nc = 0;
  for (int pass = 0; pass < 3; ++pass) {
    if (!compacted) {
      hist_add_keys(hist[pass], key, cnt, pmask, prefix, pass);
    } else {
      for (int i = tid; i < (int)nc; i += kTopkThreads) {
        const uint32_t kk = cand_key[i];
        if ((kk & pmask) == prefix) atomicAdd(&hist[pass][digit_of(kk, pass)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) pick_digit_wave(hist[pass], remaining, pub[pass], lane);
    __syncthreads();
    const uint32_t digit = pub[pass][0], above = pub[pass][1], count = pub[pass][2];
    remaining -= above;
    prefix |= digit << (pass == 0 ? 21 : pass == 1 ? 10 : 0);
    pmask = mask_through(pass);
    if (!compacted && pass < 2 && count <= (uint32_t)kCandCap) {
      // only keys sharing the decided top bits with the k-th largest are undecided: compact them,
      // one LDS atomic per wave for the wave's slots
      uint32_t mine = 0;
#pragma unroll
      for (int e = 0; e < kRegE; ++e) mine += (e < cnt && (key[e] & pmask) == prefix) ? 1u : 0u;
      const uint32_t incl = wave_incl_scan(mine);
      const uint32_t wsum = __builtin_amdgcn_readlane(incl, 63);
      uint32_t base = 0;
      if (lane == 0 && wsum) base = atomicAdd(&ncand, wsum);
      uint32_t slot = __builtin_amdgcn_readfirstlane(base) + incl - mine;
#pragma unroll
      for (int e = 0; e < kRegE; ++e) {
        if (e < cnt && (key[e] & pmask) == prefix) {
          cand_key[slot] = key[e];
          cand_pos[slot] = (uint32_t)(p0 + e);
          ++slot;
        }
      }
      __syncthreads();
      nc = ncand;
      compacted = true;
    }
  }
  const uint32_t tau = prefix;

  // ordered output: block-wide exclusive scan of (greater, equal) counts per thread
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    gt += (e < cnt && key[e] > tau) ? 1u : 0u;
    eq += (e < cnt && key[e] == tau) ? 1u : 0u;
  }
  const uint32_t gi = wave_incl_scan(gt), ei = wave_incl_scan(eq);
  if (lane == 63) { wtot[wave][0] = gi; wtot[wave][1] = ei; }
  __syncthreads();
  uint32_t gb = gi - gt, eb = ei - eq;
  for (int w = 0; w < wave; ++w) { gb += wtot[w][0]; eb += wtot[w][1]; }
  // stage the k positions in LDS (the candidate buffer is free now), then store them coalesced
  uint32_t* staged = cand_pos;
  uint32_t slot = gb + min(eb, remaining), eq_rank = eb;
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    if (e < cnt) {
      bool take = key[e] > tau;
      if (key[e] == tau) { take = eq_rank < remaining; ++eq_rank; }
      if (take) staged[slot++] = (uint32_t)(p0 + e);
    }
  }
  __syncthreads();
  for (int i = tid; i < k; i += kTopkThreads) out[i] = (int32_t)staged[i];
}

hipError_t launch_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                       int max_ctx, int k, int32_t* idx, int64_t ld_idx, hipStream_t stream,
                       int* path) {
  if (max_ctx <= kRegKeys && k <= kCandCap) {
    *path = (max_ctx <= k) ? DSA_PATH_TOPK_COPY : DSA_PATH_TOPK_RADIX_REG;
    hipLaunchKernelGGL(topk_reg_kernel, dim3(rows), dim3(kTopkThreads), 0, stream, scores, ld_scores, q_pos,
                       max_ctx, k, idx, ld_idx);
    return hipGetLastError();
  }
  const int cap = max_ctx < kTopkLdsCap ? max_ctx : kTopkLdsCap;
  const size_t lds = (size_t)cap * sizeof(uint32_t);
  *path = (max_ctx <= k) ? DSA_PATH_TOPK_COPY : DSA_PATH_TOPK_RADIX;
  hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kTopkThreads), lds, stream, scores, ld_scores,
                     q_pos, max_ctx, k, idx, ld_idx, cap);
  return hipGetLastError();
}

}  // namespace dsa
