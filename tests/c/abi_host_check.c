/* Plain-C user of the library's C ABI (no device work): compiled with gcc
 * against include/dsa_indexer.h, it checks that the header is valid C, that
 * the host-only calls behave as declared, and that errors come back as
 * statuses with a message.  Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <string.h>

#include "dsa_indexer.h"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

/* additive loss: the cost of turning layer l into S is cost[l] */
static double additive_loss(const char* pattern, int N, void* user) {
  const double* cost = (const double*)user;
  double s = 0.0;
  for (int l = 0; l < N; ++l)
    if (pattern[l] == 'S') s += cost[l];
  return s;
}

int main(void) {
  int32_t src[8];
  CHECK(dsa_abi_version() >= 1);
  CHECK(indexcache_resolve("FSSFS", 5, src) == DSA_OK);
  CHECK(src[0] == 0 && src[1] == 0 && src[2] == 0 && src[3] == 3 && src[4] == 3);
  CHECK(indexcache_resolve("SFF", 3, src) == DSA_ERR_INVALID_ARG);
  CHECK(strlen(dsa_last_error()) > 0);
  CHECK(mli_resolve("FSFFS", 5, src) == DSA_OK);
  CHECK(src[0] == 0 && src[1] == 0 && src[2] == 0 && src[3] == 2 && src[4] == 3);

  /* greedy search with a C callback: layers flip in increasing cost order */
  const double cost[6] = {0.0, 5.0, 1.0, 4.0, 2.0, 3.0};
  char pattern[7];
  double trace[4];
  int32_t flipped[3];
  CHECK(indexcache_greedy_search(6, 3, additive_loss, (void*)cost, pattern, trace, flipped) == DSA_OK);
  CHECK(strcmp(pattern, "FFSFSS") == 0);
  CHECK(flipped[0] == 2 && flipped[1] == 4 && flipped[2] == 5);
  CHECK(trace[0] == 0.0 && trace[1] == 1.0 && trace[2] == 3.0 && trace[3] == 6.0);
  CHECK(indexcache_greedy_search(6, 6, additive_loss, (void*)cost, pattern, NULL, NULL) == DSA_ERR_INVALID_ARG);

  /* overlap proxy on a hand matrix: layer 1 reuses 0 (lost 0.2), layer 3 reuses 2 (lost 0.1) */
  const double ratio[16] = {1.0, 0.8, 0.5, 0.4, 0.8, 1.0, 0.7, 0.6, 0.5, 0.7, 1.0, 0.9, 0.4, 0.6, 0.9, 1.0};
  double loss = -1.0;
  CHECK(indexcache_overlap_proxy_loss("FSFS", 4, ratio, &loss) == DSA_OK);
  CHECK(loss > 0.3 / 4 - 1e-15 && loss < 0.3 / 4 + 1e-15);

  /* workspace queries and argument rejection before any device call */
  size_t bytes = 0;
  CHECK(dsa_indexer_topk_decode_workspace(32, 131072, 64, 128, 2048, &bytes) == DSA_OK && bytes > 0);
  CHECK(dsa_indexer_topk_prefill_varlen_workspace(4, 1000, 64, 128, 2048, DSA_FP8_E4M3, &bytes) == DSA_OK);
  CHECK(dsa_indexer_topk_decode_workspace(32, 131072, 12, 128, 2048, &bytes) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa_indexer_topk_decode_workspace(32, 131072, 136, 128, 2048, &bytes) == DSA_ERR_UNSUPPORTED);
  CHECK(standin_sparse_attention_workspace(0, 16, &bytes) == DSA_ERR_INVALID_ARG);
  /* workspace sizes across the supported range (the sanitizer build checks
     every layout on the way) */
  {
    static const int Ls[] = {1, 7, 2048, 32768, 196608};
    static const int Hs[] = {8, 16, 32, 64, 128, 72};
    for (int a = 0; a < 5; ++a)
      for (int h = 0; h < 6; ++h) {
        CHECK(dsa_indexer_topk_prefill_workspace(Ls[a], Hs[h], 128, 2048, DSA_FP8_E4M3, &bytes) == DSA_OK && bytes > 0);
        CHECK(dsa_indexer_topk_prefill_workspace(Ls[a], Hs[h], 64, 1, DSA_BF16, &bytes) == DSA_OK && bytes > 0);
        CHECK(dsa_indexer_topk_prefill_workspace(Ls[a], Hs[h], 128, 64, DSA_BF16, &bytes) == DSA_OK && bytes > 0);
      }
    CHECK(dsa_indexer_topk_prefill_workspace(1024, 136, 128, 64, DSA_FP8_E4M3, &bytes) == DSA_ERR_UNSUPPORTED);
    static const int Lmaxs[] = {1, 31, 8192, 8193, 131072, 262144};
    for (int a = 0; a < 6; ++a) {
      CHECK(dsa_indexer_topk_decode_workspace(1, Lmaxs[a], 64, 128, 4096, &bytes) == DSA_OK && bytes > 0);
      CHECK(dsa_indexer_topk_decode_workspace(257, Lmaxs[a], 16, 64, 1, &bytes) == DSA_OK && bytes > 0);
      CHECK(dsa_indexer_topk_decode_workspace(3, Lmaxs[a], 128, 128, 2048, &bytes) == DSA_OK && bytes > 0);
    }
    CHECK(dsa_indexer_topk_decode_workspace(1, 262145, 64, 128, 2048, &bytes) == DSA_ERR_UNSUPPORTED);
    CHECK(dsa_indexer_topk_prefill_varlen_workspace(1000, 2000000, 64, 128, 2048, DSA_FP8_E4M3, &bytes) == DSA_OK);
    CHECK(dsa_indexer_topk_prefill_varlen_workspace(1, 0, 8, 64, 16, DSA_BF16, &bytes) == DSA_OK);
    CHECK(dsa_indexer_topk_prefill_varlen_workspace(1, 2000000000, 8, 64, 16, DSA_BF16, &bytes) == DSA_OK && bytes > 2000000000ull / 64 * 16);
  }
  printf("ok\n");
  return 0;
}
