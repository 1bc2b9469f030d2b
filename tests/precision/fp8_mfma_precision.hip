// fp8_mfma_precision.hip -- how exactly gfx950's matrix cores sum the Lightning Indexer's head dots.
//
// The indexer score ([DSA-blog] "Lightning Indexer"; [Handbook] "稀疏注意力：NSA 与 DSA": 64 heads of
// 128 dims, FP8) is a head-weighted sum of ReLU'd 128-long dot products of E4M3 codes. Scores must
// agree with an exact evaluation to 1e-5 of the row's largest score. This program measures, on
// synthetic operands shaped like the indexer's (keys ~ N(0,1) scaled to a per-key maximum of 448
// and rounded to E4M3, queries ~ N(0,1) rounded to E4M3, head weights ~ N(0,1)/8; 8192 keys x 64
// heads), the error of four ways to form the dots on the matrix cores:
//   f16_widened_16x16x32              E4M3 widened exactly to f16, v_mfma_f32_16x16x32_f16
//   fp8_16x16x32_chained              v_mfma_f32_16x16x32_fp8_fp8, the four K steps accumulated in C
//   fp8_16x16x32_per_kstep_valu_sum   the same instruction per K step from zero, summed in fp32 VALU
//   fp8_16x16x128_scaled              v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales, K = 128
// against the exact sums (E4M3 products and sums of 128 of them are exact in double). One JSON line
// per method: the largest dot error relative to the sum of |products|, the largest absolute dot
// error, the share of dots equal to the fp32 rounding of the exact sum, and the largest score error
// relative to the row's largest |score|. Test infrastructure: built by __graft_entry__.build(), run
// by tests/test_gpu_fp8_precision.py; the library does not use it.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include <random>
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
constexpr int NK = 8192, NH = 64, D = 128, NM = 4;

__device__ h8 widen(long v) {
  int lo = (int)(v & 0xffffffff), hi = (int)(v >> 32);
  h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false), b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false), d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__global__ void dot_methods(const uint8_t* keys, const uint8_t* heads, float* out) {
  const int lane = threadIdx.x, blk = blockIdx.x;   // 64 threads, NK/16 blocks
  const int r = lane % 16, g = lane / 16;
  const uint8_t* krow = keys + (size_t)(blk * 16 + r) * D;
  for (int hb = 0; hb < NH / 16; ++hb) {
    const uint8_t* hrow = heads + (size_t)(hb * 16 + r) * D;
    v4f m0 = {0, 0, 0, 0}, m1 = {0, 0, 0, 0}, m2 = {0, 0, 0, 0}, m3 = {0, 0, 0, 0};
    for (int ks = 0; ks < 4; ++ks) {
      const long a = *(const long*)(krow + 32 * ks + 8 * g), b = *(const long*)(hrow + 32 * ks + 8 * g);
      m0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(widen(a), widen(b), m0, 0, 0, 0);          // f16 after exact widening
      m1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, m1, 0, 0, 0);                  // fp8, chained
      v4f z = {0, 0, 0, 0};
      z = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, z, 0, 0, 0);                    // fp8, per K-step
      m2 += z;
    }
    const v8i A = *(const v8i*)(krow + 32 * g), B = *(const v8i*)(hrow + 32 * g);
    m3 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, m3, 0, 0, 0, 127, 0, 127);  // fp8, K = 128 at once
    for (int i = 0; i < 4; ++i) {
      const int key = blk * 16 + 4 * g + i, head = hb * 16 + r;
      out[((size_t)0 * NK + key) * NH + head] = m0[i];
      out[((size_t)1 * NK + key) * NH + head] = m1[i];
      out[((size_t)2 * NK + key) * NH + head] = m2[i];
      out[((size_t)3 * NK + key) * NH + head] = m3[i];
    }
  }
}

static double e4m3(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v = e ? std::ldexp(1.0 + m / 8.0, e - 7) : std::ldexp(m / 8.0, -6);
  return s ? -v : v;
}
static uint8_t enc(double x, const std::vector<std::pair<double, uint8_t>>& tab) {
  // nearest finite code, ties to the even code
  auto it = std::lower_bound(tab.begin(), tab.end(), std::make_pair(x, (uint8_t)0));
  if (it == tab.end()) return tab.back().second;
  if (it == tab.begin()) return it->second;
  auto lo = it - 1;
  double dl = x - lo->first, dh = it->first - x;
  if (dl < dh) return lo->second;
  if (dh < dl) return it->second;
  return (lo->second & 1) ? it->second : lo->second;
}

int main() {
  std::vector<std::pair<double, uint8_t>> tab;
  for (int c = 0; c < 256; ++c) if ((c & 0x7f) != 0x7f && c != 0x80) tab.push_back({e4m3(c), (uint8_t)c});
  std::sort(tab.begin(), tab.end());
  std::mt19937_64 rng(7);
  std::normal_distribution<double> nd;
  std::vector<uint8_t> keys((size_t)NK * D), heads((size_t)NH * D);
  std::vector<double> kscale(NK), w(NH);
  for (int j = 0; j < NK; ++j) {
    double v[D], mx = 0;
    for (int c = 0; c < D; ++c) { v[c] = nd(rng); mx = std::max(mx, std::fabs(v[c])); }
    kscale[j] = mx / 448.0;
    for (int c = 0; c < D; ++c) keys[(size_t)j * D + c] = enc(v[c] / kscale[j], tab);
  }
  for (size_t i = 0; i < heads.size(); ++i) heads[i] = enc(nd(rng), tab);
  for (int h = 0; h < NH; ++h) w[h] = nd(rng) / 8.0;
  uint8_t *dk, *dh; float* dout;
  if (hipMalloc(&dk, keys.size()) != hipSuccess || hipMalloc(&dh, heads.size()) != hipSuccess ||
      hipMalloc(&dout, sizeof(float) * NM * NK * NH) != hipSuccess) { printf("hipMalloc failed\n"); return 1; }
  if (hipMemcpy(dk, keys.data(), keys.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dh, heads.data(), heads.size(), hipMemcpyHostToDevice) != hipSuccess) { printf("copy failed\n"); return 1; }
  // grid: NK / 16 waves, each 16 keys (rows of keys) x all NH heads; every load stays inside a
  // 128-byte key or head row, every store inside out[NM][NK][NH]
  hipLaunchKernelGGL(dot_methods, dim3(NK / 16), dim3(64), 0, 0, dk, dh, dout);
  std::vector<float> out((size_t)NM * NK * NH);
  if (hipMemcpy(out.data(), dout, sizeof(float) * out.size(), hipMemcpyDeviceToHost) != hipSuccess) { printf("copy failed\n"); return 1; }
  const char* names[NM] = {"f16_widened_16x16x32", "fp8_16x16x32_chained", "fp8_16x16x32_per_kstep_valu_sum", "fp8_16x16x128_scaled"};
  // exact dots and scores (one row of NK keys, 64 heads); errors per dot and per score
  std::vector<double> exact((size_t)NK * NH), sabs((size_t)NK * NH), Iex(NK);
  double Imax = 0;
  for (int j = 0; j < NK; ++j) {
    double I = 0;
    for (int h = 0; h < NH; ++h) {
      double s = 0, a = 0;
      for (int c = 0; c < D; ++c) { double p = e4m3(keys[(size_t)j * D + c]) * e4m3(heads[(size_t)h * D + c]); s += p; a += std::fabs(p); }
      exact[(size_t)j * NH + h] = s; sabs[(size_t)j * NH + h] = a;
      I += w[h] * std::max(s, 0.0);
    }
    Iex[j] = kscale[j] * I; Imax = std::max(Imax, std::fabs(Iex[j]));
  }
  for (int m = 0; m < NM; ++m) {
    double e_rel_abs = 0, e_max = 0, e_score = 0; long nexact = 0;
    for (int j = 0; j < NK; ++j) {
      double I = 0;
      for (int h = 0; h < NH; ++h) {
        const double g = out[((size_t)m * NK + j) * NH + h], x = exact[(size_t)j * NH + h];
        e_rel_abs = std::max(e_rel_abs, std::fabs(g - x) / sabs[(size_t)j * NH + h]);
        e_max = std::max(e_max, std::fabs(g - x));
        nexact += (g == (float)x);
        I += w[h] * std::max(g, 0.0);
      }
      e_score = std::max(e_score, std::fabs(kscale[j] * I - Iex[j]) / Imax);
    }
    printf("{\"method\": \"%s\", \"max_err_over_sum_abs_products\": %.3e, \"max_abs_err\": %.3e, \"dots_equal_fp32_rounded_exact\": %.4f, \"score_err_over_row_max\": %.3e}\n",
           names[m], e_rel_abs, e_max, (double)nexact / ((double)NK * NH), e_score);
  }
  return 0;
}
