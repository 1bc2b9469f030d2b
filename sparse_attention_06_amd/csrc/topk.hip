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
// holds 16 consecutive keys, so the row is read once (rows of at most 4096 / 8192 positions: 256 /
// 512 threads). Three passes over 11-, 11- and 10-bit
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

// A pass's digit: `width` (at most 11) key bits from bit `shift` up.
struct Digit {
  uint32_t shift, mask;
  __device__ __forceinline__ uint32_t of(uint32_t key) const { return (key >> shift) & mask; }
};

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

// hist[digit] += 1 for each active key (valid: bit e of vmask). A lane adds all its keys that
// share the digit of its first active key with one atomic (the leading digits of real scores
// repeat a lot, and one atomic per key would serialise on the hot address); its other keys are
// added one by one.
__device__ __forceinline__ void hist_add_keys(uint32_t* hist, const uint32_t (&key)[kRegE], uint32_t vmask,
                                              uint32_t pmask, uint32_t prefix, Digit dg) {
  uint32_t d0 = 0, run = 0;
  bool have = false;
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    const bool act = ((vmask >> e) & 1u) && (key[e] & pmask) == prefix;
    const uint32_t d = dg.of(key[e]);
    if (act && !have) { d0 = d; have = true; }
    run += (act && d == d0) ? 1u : 0u;
  }
  if (have) atomicAdd(&hist[d0], run);
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    const bool act = ((vmask >> e) & 1u) && (key[e] & pmask) == prefix;
    const uint32_t d = dg.of(key[e]);
    if (act && d != d0) atomicAdd(&hist[d], 1u);
  }
}

// Wave 0 picks the digit of the remaining-th largest key from a 2048-bin histogram (digits in
// descending order): 64 coarse bins of 32 digits first, then the 32 digits of the chosen one.
// Publishes {digit, keys with larger digits, keys with that digit} in pub and returns the digit
// (the same in every lane). The histogram must hold at least `remaining` keys.
__device__ __forceinline__ uint32_t pick_digit_wave(const uint32_t* hist, uint32_t remaining, uint32_t* pub, int lane) {
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
  return (uint32_t)(32 * cc + 31 - fl);
}

// Keys of `hist` (2048 bins) whose digit is at least d, summed over wave 0 (same in every lane).
__device__ __forceinline__ uint32_t count_at_or_above_wave(const uint32_t* hist, uint32_t d, int lane) {
  uint32_t s = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int b0 = 32 * lane + 4 * v;
    const uint4 q4 = *(const uint4*)(hist + b0);
    s += ((uint32_t)b0 >= d ? q4.x : 0u) + ((uint32_t)b0 + 1 >= d ? q4.y : 0u) + ((uint32_t)b0 + 2 >= d ? q4.z : 0u) +
         ((uint32_t)b0 + 3 >= d ? q4.w : 0u);
  }
  return __builtin_amdgcn_readlane(wave_incl_scan(s), 63);
}

// The register variant's LDS for a workgroup of kT threads (kT / 64 waves).
template <int kT>
struct TopkLds {
  uint32_t hist[3][kRegBins];  // one histogram per pass
  uint32_t cand_key[kCandCap], cand_pos[kCandCap];
  uint32_t wtot[kT / kWave][2];
  uint32_t pub[4][4];
  uint32_t ncand;
};

// Zero the histograms and the candidate count; the caller does this before its keys arrive and
// reg_select's first barrier publishes it. With hist0 (the row's first-digit histogram, counted
// by the producer of the scores) the first histogram is taken from there instead, and hist0 is
// zeroed for the producer's next use.
template <int kT>
__device__ __forceinline__ void reg_select_init(TopkLds<kT>& sh, int tid, uint32_t* hist0) {
  static_assert(kRegBins == kTopkDigit0Bins, "first digit: key bits 31..21");
  const int given = hist0 ? kRegBins / 4 : 0;
  for (int i = tid; i < 3 * kRegBins / 4; i += kT) {
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (i < given) {
      v = ((const uint4*)hist0)[i];
      ((uint4*)hist0)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    ((uint4*)&sh.hist[0][0])[i] = v;
  }
  if (tid == 0) sh.ncand = 0;
}

// The chunk stage of a long row whose chunks' first-digit counts are all given (hist_row: the row's
// nchunks chunks of 2048 bins each, nchunks <= kTopkFilterChunks): sh.hist[0] takes this chunk's
// counts, sh.hist[1] the row's (their sum), sh.hist[2] is zeroed. The counts stay in place, since
// every chunk of the row reads them; the merge clears them.
constexpr int kTopkFilterChunks = 8;
template <int kT>
__device__ __forceinline__ void filter_init(TopkLds<kT>& sh, int tid, const uint32_t* hist_row, int nchunks, int c) {
  for (int i = tid; i < kRegBins / 4; i += kT) {
    uint4 v[kTopkFilterChunks];
#pragma unroll
    for (int ch = 0; ch < kTopkFilterChunks; ++ch)
      v[ch] = ch < nchunks ? ((const uint4*)(hist_row + (size_t)ch * kRegBins))[i] : make_uint4(0u, 0u, 0u, 0u);
    uint4 sum = make_uint4(0u, 0u, 0u, 0u), own = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int ch = 0; ch < kTopkFilterChunks; ++ch) {
      sum.x += v[ch].x; sum.y += v[ch].y; sum.z += v[ch].z; sum.w += v[ch].w;
      if (ch == c) own = v[ch];
    }
    ((uint4*)&sh.hist[0][0])[i] = own;
    ((uint4*)&sh.hist[1][0])[i] = sum;
    ((uint4*)&sh.hist[2][0])[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) sh.ncand = 0;
}

// The key of the k-th largest valid key (tau) and how many keys equal to tau are taken, over the
// keys the block's threads hold (16 each, valid where vmask has the bit). Needs more than k valid
// keys and reg_select_init since the keys' arrival. Three passes over 11-, 11- and 10-bit digits;
// once the keys still undecided fit in LDS they are compacted there and the remaining passes run
// over them alone.
template <int kT>
__device__ __forceinline__ void reg_select(const uint32_t (&key)[kRegE], uint32_t vmask, uint32_t k, bool hist0_given,
                           TopkLds<kT>& sh, int tid, int wave, int lane, uint32_t& tau_out, uint32_t& remaining_out) {
  __syncthreads();  // publishes reg_select_init
  const int npass = 3;
  uint32_t pmask = 0u;
  uint32_t prefix = 0u, remaining = k;
  bool compacted = false;
  uint32_t nc = 0;
  for (int pass = 0; pass < npass; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const Digit dg{(uint32_t)shift, pass == 2 ? 1023u : 2047u};
    if (pass == 0 && hist0_given) {
      // counted already
    } else if (!compacted) {
      hist_add_keys(sh.hist[pass], key, vmask, pmask, prefix, dg);
    } else {
      for (int i = tid; i < (int)nc; i += kT) {
        const uint32_t kk = sh.cand_key[i];
        if ((kk & pmask) == prefix) atomicAdd(&sh.hist[pass][dg.of(kk)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) pick_digit_wave(sh.hist[pass], remaining, sh.pub[pass], lane);
    __syncthreads();
    const uint32_t digit = sh.pub[pass][0], above = sh.pub[pass][1], count = sh.pub[pass][2];
    remaining -= above;
    prefix |= digit << shift;
    pmask = shift == 0 ? 0xFFFFFFFFu : ~((1u << shift) - 1u);
    if (!compacted && pass + 1 < npass && count <= (uint32_t)kCandCap) {
      // only keys sharing the decided top bits with the k-th largest are undecided: compact them,
      // one LDS atomic per wave for the wave's slots
      uint32_t mine = 0;
#pragma unroll
      for (int e = 0; e < kRegE; ++e) mine += (((vmask >> e) & 1u) && (key[e] & pmask) == prefix) ? 1u : 0u;
      const uint32_t incl = wave_incl_scan(mine);
      const uint32_t wsum = __builtin_amdgcn_readlane(incl, 63);
      uint32_t base = 0;
      if (lane == 0 && wsum) base = atomicAdd(&sh.ncand, wsum);
      uint32_t slot = __builtin_amdgcn_readfirstlane(base) + incl - mine;
#pragma unroll
      for (int e = 0; e < kRegE; ++e) {
        if (((vmask >> e) & 1u) && (key[e] & pmask) == prefix) sh.cand_key[slot++] = key[e];
      }
      __syncthreads();
      nc = sh.ncand;
      compacted = true;
    }
  }
  tau_out = prefix;
  remaining_out = remaining;
}

// Stage the selected keys in input order: every valid key above tau and the first `remaining`
// keys equal to tau (every valid key when take_all). Their positions (pos_of(e) for this thread's
// key e) and, with_keys, their order keys land in sh.cand_pos / sh.cand_key at their output
// slots; returns how many were selected. Each thread first forms two 16-bit masks of its keys
// (above tau, equal to tau); without keys to stage it then visits only the set bits of its
// selection (about one key in eight at k = 2048 over 16384), not all sixteen keys.
template <int kT, bool with_keys, class PosOf>
__device__ __forceinline__ uint32_t stage_selected(const uint32_t (&key)[kRegE], PosOf pos_of, uint32_t vmask, bool take_all,
                                   uint32_t tau, uint32_t remaining, TopkLds<kT>& sh, int wave, int lane) {
  uint32_t gtm = 0, eqm = 0;
#pragma unroll
  for (int e = 0; e < kRegE; ++e) {
    gtm |= (key[e] > tau ? 1u : 0u) << e;
    eqm |= (key[e] == tau ? 1u : 0u) << e;
  }
  gtm = take_all ? vmask : (gtm & vmask);
  eqm = take_all ? 0u : (eqm & vmask);
  const uint32_t gt = (uint32_t)__builtin_popcount(gtm), eq = (uint32_t)__builtin_popcount(eqm);
  const uint32_t gi = wave_incl_scan(gt), ei = wave_incl_scan(eq);
  __syncthreads();  // the selection may still read the candidate buffers and the wave totals
  if (lane == 63) { sh.wtot[wave][0] = gi; sh.wtot[wave][1] = ei; }
  __syncthreads();
  uint32_t gb = gi - gt, eb = ei - eq, gall = 0, eall = 0;
  for (int w = 0; w < kT / kWave; ++w) {
    if (w < wave) { gb += sh.wtot[w][0]; eb += sh.wtot[w][1]; }
    gall += sh.wtot[w][0];
    eall += sh.wtot[w][1];
  }
  // the keys equal to tau this thread takes: the first (remaining - eb) of them, in key order
  const uint32_t allow = remaining > eb ? remaining - eb : 0u;
  uint32_t eqt = eqm;
  if (allow < eq) {
    eqt = 0u;
    uint32_t m = eqm;
    for (uint32_t i = 0; i < allow; ++i) {
      eqt |= m & (0u - m);  // lowest set bit
      m &= m - 1u;
    }
  }
  const uint32_t sel = gtm | eqt;
  uint32_t slot = gb + min(eb, remaining);
  if (with_keys) {
#pragma unroll
    for (int e = 0; e < kRegE; ++e) {
      if ((sel >> e) & 1u) {
        sh.cand_pos[slot] = pos_of(e);
        sh.cand_key[slot] = key[e];
        ++slot;
      }
    }
  } else {
    for (uint32_t m = sel; m; m &= m - 1u) sh.cand_pos[slot++] = pos_of(__builtin_ctz(m));
  }
  __syncthreads();
  return gall + min(eall, remaining);
}

// One selection over up to 16384 keys per block. With kSrcScores the keys are the scores of row r
// at positions [16384 * c, ...) below the row's length (r = blockIdx.y, c = blockIdx.x; chunk
// stages: a 1-D grid whose block b is chunk c of row r as chunk_stage_of maps it); otherwise they
// are the candidate slots of row r = blockIdx.y written by a previous stage (in_chunks chunks of k slots, the
// first in_cnt of each valid, in ascending position order). With kFinal the block writes the row's
// index list (positions ascending, -1 padded to k); otherwise this chunk's candidates (at most k
// order keys with their positions, ascending by position) and their count.
struct TopkStageArgs {
  const float* scores;
  int64_t ld_scores;
  const int32_t* q_pos;
  int max_ctx, k;
  int32_t* idx;
  int64_t ld_idx;
  const uint32_t* in_key;
  const int32_t* in_pos;
  const int32_t* in_cnt;
  int in_chunks;
  uint32_t* out_key;
  int32_t* out_pos;
  int32_t* out_cnt;
  int out_chunks;
  uint32_t* hist0;  // score rows: per row and chunk, the first-digit histogram (or null)
  uint32_t* mhist;  // per row, the first-digit histogram of the merge's candidates (or null): the
                    // chunk stage adds its selection's counts, the merge starts from them
  int rows;         // rows of the launch (chunk stages: the 1-D grid covers 8 * out_chunks * ceil(rows / 8))
  int len_first;    // score rows: read the row's length before its scores and load only positions
                    // below it (grids of many rows, bound by bytes); else load the whole chunk at once
  int row_filter;   // chunk stage with hist0 and mhist over at most kTopkFilterChunks chunks: each
                    // chunk passes on its keys whose first digit reaches the row's threshold digit
                    // (from the sum of the row's chunk counts), and the merge clears those counts
};

// kPacked: two workgroups per CU (at most 64 VGPRs, a few spilled), for grids of many rows or
// chunks, where a second workgroup's work overlaps the first's barrier-bound phases; one
// workgroup per CU otherwise (no spills). kT: threads per workgroup (1024: 16384 keys; 512 / 256:
// 8192 / 4096 keys, two workgroups per CU as LDS allows).
template <bool kSrcScores, bool kFinal, bool kPacked, int kT = kTopkThreads>
__global__ void __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kPacked ? 8 : kT / 256, 8)))
topk_stage_kernel(TopkStageArgs a) {
  constexpr int kKeys = kT * kRegE;  // keys a workgroup holds: one chunk of a row
  __shared__ __attribute__((aligned(16))) TopkLds<kT> sh;
  int r = blockIdx.y, c = blockIdx.x;
  if (kSrcScores && !kFinal) {
    // Workgroups go to the 8 XCDs round robin: the chunks of a row run on one XCD, one after the
    // other, so the row's chunk counts that each of them reads (the row filter) come from that
    // XCD's L2 after the first
    const int slot = blockIdx.x >> 3;
    r = (slot / a.out_chunks) * 8 + (int)(blockIdx.x & 7);
    c = slot % a.out_chunks;
    if (r >= a.rows) return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t key[kRegE], vmask = 0;
  const int nchunks = kFinal ? 1 : a.out_chunks;  // score chunks of a row in this launch
  uint32_t* const hist0 = kSrcScores ? (a.hist0 ? a.hist0 + ((int64_t)r * nchunks + c) * kRegBins : nullptr)
                                     : (a.mhist ? a.mhist + (int64_t)r * kRegBins : nullptr);
  const bool row_filter = kSrcScores && !kFinal && a.row_filter;
  if (kSrcScores) {
    // this thread's positions: base .. base + 15. The row is read before q_pos is known (every
    // position below max_ctx lies inside the row), and both before the first-digit histogram is
    // staged, so the memory latencies overlap.
    int n = a.q_pos[r] + 1;
    const float* row = a.scores + (int64_t)r * a.ld_scores;
    const int base = kKeys * c + kRegE * tid;
    float f[kRegE];
    auto load_keys = [&]() {
      if (base + kRegE <= a.max_ctx && ((uintptr_t)(row + base) & 15) == 0) {
#pragma unroll
        for (int v = 0; v < kRegE / 4; ++v) {
          const float4 x = *(const float4*)(row + base + 4 * v);
          f[4 * v] = x.x; f[4 * v + 1] = x.y; f[4 * v + 2] = x.z; f[4 * v + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < kRegE; ++e) f[e] = base + e < a.max_ctx ? row[base + e] : 0.f;
      }
    };
    if (a.len_first) {
      // a thread whose positions all lie past the row's end loads nothing (its keys are masked
      // off below)
      if (base < n) {
        load_keys();
      } else {
#pragma unroll
        for (int e = 0; e < kRegE; ++e) f[e] = 0.f;
      }
    } else {
      load_keys();
    }
    if (row_filter) filter_init(sh, tid, a.hist0 + (int64_t)r * nchunks * kRegBins, nchunks, c);
    else reg_select_init(sh, tid, hist0);
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
#pragma unroll
    for (int e = 0; e < kRegE; ++e) {
      const bool v = base + e < n;
      vmask |= (v ? 1u : 0u) << e;
      key[e] = v ? order_key(f[e]) : 0u;
    }
  } else {
    // candidate slot g = 16 * tid + e of the row: chunk g / k, entry g % k. Every slot below
    // in_chunks * k lies in the workspace, so the keys and counts are loaded without waiting on
    // each other (a slot past its chunk's count holds stale data and is masked off).
    const int64_t rb = (int64_t)r * a.in_chunks * a.k;
    const int total = a.in_chunks * a.k, g0 = kRegE * tid;
    const int32_t* cnt = a.in_cnt + (int64_t)r * a.in_chunks;
    if (g0 + kRegE <= total && ((uintptr_t)(a.in_key + rb + g0) & 15) == 0) {
#pragma unroll
      for (int v = 0; v < kRegE / 4; ++v) {
        const uint4 x = *(const uint4*)(a.in_key + rb + g0 + 4 * v);
        key[4 * v] = x.x; key[4 * v + 1] = x.y; key[4 * v + 2] = x.z; key[4 * v + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kRegE; ++e) key[e] = g0 + e < total ? a.in_key[rb + g0 + e] : 0u;
    }
    const int ch0 = g0 / a.k, ch1 = (g0 + kRegE - 1) / a.k;
    const int n0 = (ch0 == ch1 && ch0 < a.in_chunks) ? cnt[ch0] : 0;
    reg_select_init(sh, tid, hist0);
    if (ch0 == ch1) {  // the thread's slots share one chunk (always when k is a multiple of 16)
      const int e_end = ch0 * a.k + n0 - g0;
#pragma unroll
      for (int e = 0; e < kRegE; ++e) vmask |= (e < e_end ? 1u : 0u) << e;
    } else {
#pragma unroll
      for (int e = 0; e < kRegE; ++e) {
        const int g = g0 + e, ch = g / a.k;
        const bool v = ch < a.in_chunks && g - ch * a.k < cnt[ch];
        vmask |= (v ? 1u : 0u) << e;
      }
    }
#pragma unroll
    for (int e = 0; e < kRegE; ++e) key[e] = ((vmask >> e) & 1u) ? key[e] : 0u;
  }
  // keys held by the block: the chunk's share of the row, or the sum of the input chunks' counts
  uint32_t nvalid = 0;
  if (kSrcScores) {
    int n = a.q_pos[r] + 1;
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    const int len = n - kKeys * c;
    nvalid = len < 0 ? 0u : (uint32_t)min(len, kKeys);
  } else {
    // lanes load the counts side by side (a loop of dependent loads would serialise them)
    uint32_t part = 0;
    for (int ch = lane; ch < a.in_chunks; ch += kWave) part += (uint32_t)a.in_cnt[(int64_t)r * a.in_chunks + ch];
    nvalid = __builtin_amdgcn_readlane(wave_incl_scan(part), 63);
  }
  const uint32_t k = (uint32_t)a.k;
  const bool take_all = nvalid <= k;
  uint32_t tau = 0, remaining = k;
  // Row filter: every key of the row's top k has a first digit of at least dstar, the first digit
  // of the row's k-th largest key. A chunk with at most k such keys passes on all of them (a
  // superset of its share of the row's top k, like its own top k), with no selection of its own;
  // a chunk with more selects its own top k.
  bool filt = false;
  uint32_t dstar = 0;
  if (row_filter) {
    int n = a.q_pos[r] + 1;
    n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
    if ((uint32_t)n > k) {  // else every chunk keeps every key
      __syncthreads();      // publishes filter_init
      if (wave == 0) {
        const uint32_t d = pick_digit_wave(sh.hist[1], k, sh.pub[3], lane);  // the row holds n > k keys
        const uint32_t own = count_at_or_above_wave(sh.hist[0], d, lane);
        if (lane == 0) sh.pub[3][3] = own;
      }
      __syncthreads();
      dstar = sh.pub[3][0];
      filt = sh.pub[3][3] <= k;  // block-uniform
      if (filt) {
        tau = dstar == 0 ? 0u : (dstar << 21) - 1u;  // keys above tau: first digit >= dstar
        remaining = 0;
      } else {
        // reg_select counts its second digit into sh.hist[1]; its first barrier publishes this
        for (int i = tid; i < kRegBins / 4; i += kT) ((uint4*)&sh.hist[1][0])[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  if (!take_all && !filt) reg_select(key, vmask, k, hist0 != nullptr, sh, tid, wave, lane, tau, remaining);
  // keys staged without a selection: all valid ones (a chunk that keeps every key, or a filter
  // threshold of digit 0), else those above tau and the first `remaining` equal to it
  const bool stage_all = filt ? dstar == 0 : take_all;
  if (kSrcScores && !kFinal && hist0 && a.mhist) {
    // this chunk's selection by first digit, from its full counts (still in the first LDS
    // histogram): with the row filter every bin from dstar up; otherwise every bin above the k-th
    // key's, and k - (keys above) from its bin; all of them when the chunk keeps every key
    // A chunk that keeps every key skipped reg_select and its barriers: publish the histogram
    // reg_select_init wrote (each thread wrote other bins than it reads here) before reading it.
    if (take_all) __syncthreads();  // block-uniform
    const uint32_t d0 = sh.pub[0][0], above0 = sh.pub[0][1];
    uint32_t* mh = a.mhist + (int64_t)r * kRegBins;
    for (int b = tid; b < kRegBins; b += kT) {
      uint32_t n;
      if (filt) n = (uint32_t)b >= dstar ? sh.hist[0][b] : 0u;
      else n = take_all || (uint32_t)b > d0 ? sh.hist[0][b] : ((uint32_t)b == d0 ? k - above0 : 0u);
      if (n) __hip_atomic_fetch_add(mh + b, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // staged per selected key: its position for a score row, its input slot for candidates (the
  // slot's position is read when the result is written, by every thread at once)
  int obase = kSrcScores ? kKeys * c + kRegE * tid : kRegE * tid;
  asm volatile("" : "+v"(obase));  // opaque: the 16 values are formed when they are stored
  const int64_t rb = (int64_t)r * a.in_chunks * a.k;
  const uint32_t nsel = stage_selected<kT, !kFinal>(key, [&](int e) { return (uint32_t)(obase + e); }, vmask, stage_all, tau,
                                                remaining, sh, wave, lane);
  auto pos_at = [&](int i) { return kSrcScores ? (int32_t)sh.cand_pos[i] : a.in_pos[rb + sh.cand_pos[i]]; };
  if (kFinal) {
    // all of a thread's (at most kCandCap / kT) reads are issued before its stores
    int32_t* out = a.idx + (int64_t)r * a.ld_idx;
    int32_t v[kCandCap / kT];
#pragma unroll
    for (int j = 0; j < kCandCap / kT; ++j) {
      const int i = tid + j * kT;
      v[j] = i < (int)nsel ? pos_at(i) : -1;
    }
#pragma unroll
    for (int j = 0; j < kCandCap / kT; ++j) {
      const int i = tid + j * kT;
      if (i < a.k) out[i] = v[j];
    }
    if (!kSrcScores && a.row_filter) {
      // the chunk stage left the row's chunk counts in place: clear them for the producer's next use
      uint4* h = (uint4*)(a.hist0 + (int64_t)r * a.in_chunks * kRegBins);
      for (int i = tid; i < a.in_chunks * kRegBins / 4; i += kT) h[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    const int64_t ob = ((int64_t)r * a.out_chunks + c) * a.k;
    for (int i = tid; i < (int)nsel; i += kT) {
      a.out_key[ob + i] = sh.cand_key[i];
      a.out_pos[ob + i] = pos_at(i);
    }
    if (tid == 0) a.out_cnt[(int64_t)r * a.out_chunks + c] = (int32_t)nsel;
  }
}

// Long rows: candidates per chunk of kRegKeys positions (at most k each), then one selection over
// them. The union of the chunks' top-k sets holds the row's top-k under the same order (value,
// then position), and the candidates stay in ascending position order, so ties still go to the
// smaller position. Usable while every row's candidates fit one block. With every chunk's
// first-digit counts given, a chunk with at most k keys whose first digit reaches the row's
// threshold digit passes on those instead of its own top-k: they too hold its share of the row's
// top-k.
static_assert(kRegKeys == kTopkChunkKeys, "chunks of the first-digit counts");
// Stage grids of at least this many workgroups (two per CU) take the packed stage kernel.
constexpr int kTopkPackedGrid = 512;
// Rows of at most 4096 (8192) positions take 256-thread (512-thread) workgroups: the same 16 keys
// per thread, fewer waves to synchronise and no threads without keys.
constexpr int kTopkSmallThreads = 256;
int topk_reg_max_ctx() { return kRegKeys; }
int topk_reg_max_k() { return kCandCap; }
int topk_chunks(int max_ctx) { return (max_ctx + kRegKeys - 1) / kRegKeys; }
bool topk_staged_ok(int max_ctx, int k) {
  return max_ctx > kRegKeys && k <= kCandCap && (int64_t)topk_chunks(max_ctx) * k <= kRegKeys;
}
size_t topk_staged_ws_bytes(int rows, int max_ctx, int k) {
  if (!topk_staged_ok(max_ctx, k)) return 0;
  const size_t slots = (size_t)rows * topk_chunks(max_ctx) * k;
  return slots * 8 + (size_t)rows * topk_chunks(max_ctx) * 4 + 256;
}

hipError_t launch_topk(const float* scores, int64_t ld_scores, const int32_t* q_pos, int rows,
                       int max_ctx, int k, int32_t* idx, int64_t ld_idx, void* ws, size_t ws_bytes,
                       uint32_t* hist0, hipStream_t stream, int* path) {
  TopkStageArgs a{};
  a.scores = scores; a.ld_scores = ld_scores; a.q_pos = q_pos; a.max_ctx = max_ctx; a.k = k;
  a.idx = idx; a.ld_idx = ld_idx;
  if (max_ctx <= kRegKeys && k <= kCandCap) {
    a.hist0 = hist0;
    // many rows (prefill blocks): bound by the bytes read, so causal rows skip their tails
    a.len_first = rows >= kTopkPackedGrid ? 1 : 0;
    *path = (max_ctx <= k) ? DSA_PATH_TOPK_COPY : DSA_PATH_TOPK_RADIX_REG;
    if (max_ctx <= kTopkSmallThreads * kRegE)
      hipLaunchKernelGGL((topk_stage_kernel<true, true, false, kTopkSmallThreads>), dim3(1, rows), dim3(kTopkSmallThreads), 0,
                         stream, a);
    else if (max_ctx <= 2 * kTopkSmallThreads * kRegE)
      hipLaunchKernelGGL((topk_stage_kernel<true, true, false, 2 * kTopkSmallThreads>), dim3(1, rows),
                         dim3(2 * kTopkSmallThreads), 0, stream, a);
    else if (rows >= kTopkPackedGrid)
      hipLaunchKernelGGL((topk_stage_kernel<true, true, true>), dim3(1, rows), dim3(kTopkThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((topk_stage_kernel<true, true, false>), dim3(1, rows), dim3(kTopkThreads), 0, stream, a);
    return hipGetLastError();
  }
  const size_t need = topk_staged_ws_bytes(rows, max_ctx, k);
  if (need && ws && ws_bytes >= need) {
    *path = DSA_PATH_TOPK_RADIX_STAGED;
    const int C = topk_chunks(max_ctx);
    uint8_t* p = (uint8_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    const size_t slots = (size_t)rows * C * k;
    a.out_key = (uint32_t*)p;
    a.out_pos = (int32_t*)(p + slots * 4);
    a.out_cnt = (int32_t*)(p + slots * 8);
    a.out_chunks = C;
    a.hist0 = hist0;
    // with the chunks' counts given, the merge's candidate counts follow the chunks' histograms
    a.mhist = hist0 ? hist0 + (size_t)rows * C * kRegBins : nullptr;
    a.row_filter = hist0 && C <= kTopkFilterChunks ? 1 : 0;
    a.rows = rows;
    const dim3 cgrid((unsigned)(8 * C * ((rows + 7) / 8)));
    if ((int64_t)C * rows >= kTopkPackedGrid)
      hipLaunchKernelGGL((topk_stage_kernel<true, false, true>), cgrid, dim3(kTopkThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((topk_stage_kernel<true, false, false>), cgrid, dim3(kTopkThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    TopkStageArgs b = a;
    b.in_key = a.out_key; b.in_pos = a.out_pos; b.in_cnt = a.out_cnt; b.in_chunks = C;
    b.out_key = nullptr; b.out_pos = nullptr; b.out_cnt = nullptr; b.out_chunks = 0;
    b.hist0 = a.row_filter ? a.hist0 : nullptr;  // the chunk counts the merge clears
    if (rows >= kTopkPackedGrid)
      hipLaunchKernelGGL((topk_stage_kernel<false, true, true>), dim3(1, rows), dim3(kTopkThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((topk_stage_kernel<false, true, false>), dim3(1, rows), dim3(kTopkThreads), 0, stream, b);
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
