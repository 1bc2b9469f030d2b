/* abi_driver.c -- calls every entry point of libdsa.so with host arguments it must reject
 * before any launch (NULL or misaligned pointers, bad sizes, small workspaces, unsupported
 * shapes) and the workspace-size queries at extreme sizes, for a build of the library's host
 * code under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py). No GPU
 * is needed: nothing reaches a kernel launch. Exit status 0: every call returned the expected
 * status and no sanitizer reported. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "dsa.h"

static int fails = 0;
#define EXPECT(call, want)                                                                         \
  do {                                                                                             \
    dsa_status_t s_ = (call);                                                                      \
    if (s_ != (want)) {                                                                            \
      fprintf(stderr, "line %d: %s -> %s (%s), want %s\n", __LINE__, #call, dsa_status_string(s_), \
              dsa_last_error(), dsa_status_string(want));                                          \
      ++fails;                                                                                     \
    }                                                                                              \
  } while (0)

int main(void) {
  void* f = (void*)(uintptr_t)0x1000;  /* never dereferenced: validation fails first */
  void* mis = (void*)(uintptr_t)0x1004;
  const int32_t* fi = (const int32_t*)f;
  EXPECT(dsa_indexer_scores(NULL, NULL, NULL, NULL, NULL, 1, 64, 1, NULL, NULL, 1, 1, 1, 64, 64, 128, DSA_E4M3, NULL,
                            64, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_scores(mis, f, f, NULL, fi, 2, 64, 1, NULL, fi, 1, 1, 1, 128, 64, 128, DSA_E4M3, f, 128, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 64, 1, NULL, fi, 1, 1, 1, INT_MAX, 64, 128, DSA_E4M3, f, INT_MAX,
                            NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 0, 1, NULL, fi, 1, 1, 1, 64, 64, 128, DSA_E4M3, f, 64, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 64, 1, NULL, fi, INT_MAX, INT_MAX, INT_MAX, 64, 64, 128, DSA_E4M3,
                            f, 64, NULL),
         DSA_ERR_INVALID_ARG);                                   /* rows != n_seq * q_per_seq */
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 64, 1, fi, fi, 3, 2, 2, 64, 64, 128, DSA_E4M3, f, 64, NULL),
         DSA_ERR_INVALID_ARG);                                   /* q_seq with q_per_seq != 1 */
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 64, 1, fi, fi, 3, 0, 1, 64, 64, 128, DSA_E4M3, f, 64, NULL),
         DSA_ERR_INVALID_ARG);                                   /* rows without any sequence */
  EXPECT(dsa_indexer_scores(f, f, f, NULL, fi, 1, 64, 1, NULL, fi, 0, 0, 1, 64, 64, 128, DSA_E4M3, f, 64, NULL),
         DSA_OK);
  EXPECT(dsa_topk(f, 64, fi, 4, 64, 0, f, 64, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_topk(f, 64, fi, 4, 64, 32, f, 16, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_topk(f, 32, fi, 4, 64, 32, f, 64, NULL, 0, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_topk(f, 64, fi, 0, 64, 32, f, 64, NULL, 0, NULL), DSA_OK);
  EXPECT(dsa_indexer_topk(f, f, f, f, fi, 256, 64, 256, NULL, fi, 128, 64, 2, 16384, 64, 128, DSA_E4M3, f, 16384,
                          2048, f, 2048, NULL, 0, NULL),
         DSA_ERR_WORKSPACE);
  EXPECT(dsa_indexer_topk(f, f, f, f, fi, 256, 64, 256, NULL, fi, 128, 64, 2, 16384, 64, 128, DSA_E4M3, f, 16384, 0,
                          f, 2048, f, 1 << 30, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_sparse_mla_decode(f, f, fi, 1, 64, 1, NULL, fi, 1, 1, 1, fi, 8, 8, 128, 576, 512, 576, 65, 0.1f, f, NULL, NULL,
                               0, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_sparse_mla_decode(f, f, fi, 1, 64, 1, NULL, fi, 1, 1, 1, fi, 8, 8, 4, 2048, 64, 2048, 0, 0.1f, f, NULL, NULL, 0,
                               NULL),
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_sparse_mla_decode(f, f, fi, 64, 64, 64, NULL, fi, 4, 4, 1, fi, 2048, 2048, 128, 576, 512, 576, 0, 0.1f, f, NULL,
                               NULL, 0, NULL),
         DSA_ERR_WORKSPACE);
  EXPECT(dsa_sparse_mla_prefill(mis, f, fi, 1, 64, 1, NULL, fi, 1, 1, 1, fi, 8, 8, 128, 576, 512, 576, 0, 0.1f, f, NULL, NULL,
                                0, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_dense_mla_prefill(f, f, fi, 1, 64, 1, NULL, fi, 4, 1, 4, 0, 128, 576, 512, 576, 0, 0.1f, f, NULL, NULL, 0, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_expanded_mha_prefill(f, f, f, f, 1 << 20, fi, 1, 1, NULL, 0, 0, 128, 128, 64, 128, 0.1f, f, NULL, NULL,
                                  0, NULL),
         DSA_ERR_INVALID_ARG);
  EXPECT(dsa_expanded_mha_prefill(f, f, f, f, 64, fi, 1, 1, NULL, 0, 0, 128, 64, 64, 128, 0.1f, f, NULL, NULL, 0,
                                  NULL),
         DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_expanded_mha_prefill(f, f, f, f, 64, fi, 1, 1, fi, 16, 16, 128, 128, 64, 128, 0.1f, f, NULL, NULL, 0,
                                  NULL),
         DSA_ERR_WORKSPACE);
  EXPECT(dsa_indexer_cache_write(f, DSA_F32, 1, 64, fi, fi, 1, fi, 1, 64, 1, f, f, NULL), DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_indexer_cache_write(NULL, DSA_F32, 1, 128, fi, fi, 1, fi, 1, 64, 1, f, f, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_latent_cache_write(f, 1, 570, fi, fi, 1, fi, 1, 64, 1, f, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_e4m3_quantize(f, -1, f, NULL), DSA_ERR_INVALID_ARG);
  EXPECT(dsa_e4m3_quantize(mis, 16, f, NULL), DSA_ERR_INVALID_ARG);
  /* size queries at extreme sizes: no overflow, no crash */
  const int big[] = {-1, 0, 1, 2047, 2048, 16384, 16385, 131072, 1 << 20, INT_MAX};
  size_t acc = 0;
  for (int a = 0; a < 10; ++a)
    for (int b = 0; b < 10; ++b) {
      acc += dsa_topk_workspace_size(big[a], big[b], 2048);
      acc += dsa_indexer_topk_workspace_size(big[a], big[b], 2048);
      acc += dsa_sparse_mla_workspace_size(big[a], 128, 512, big[b]);
      acc += dsa_dense_mla_workspace_size(big[a], 128, 512, big[b]);
      acc += dsa_expanded_mha_workspace_size(big[a], big[b], 2048);
    }
  (void)dsa_last_path();
  printf("abi driver: %s (%zu)\n", fails ? "FAILED" : "ok", acc & 1);
  return fails ? 1 : 0;
}
