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

hipError_t launch_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                       int max_ctx, int k, int32_t* idx, int64_t ld_idx, hipStream_t stream,
                       int* path) {
  const int cap = max_ctx < kTopkLdsCap ? max_ctx : kTopkLdsCap;
  const size_t lds = (size_t)cap * sizeof(uint32_t);
  *path = (max_ctx <= k) ? DSA_PATH_TOPK_COPY : DSA_PATH_TOPK_RADIX;
  hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kTopkThreads), lds, stream, scores, ld_scores,
                     q_pos, max_ctx, k, idx, ld_idx, cap);
  return hipGetLastError();
}

}  // namespace dsa
