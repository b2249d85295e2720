/* Host-side checks of libmedusa's C ABI, built against a copy of the library
 * whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitizers.py builds both and runs this program; no GPU
 * is used: every call here returns from the host-side argument checks or is
 * host-only code).
 *
 * Covered: status strings and the ABI version; the tree-template check on
 * valid and malformed templates; the accuracy-driven sparse tree over a
 * sweep of head counts, list lengths and tree sizes (each result must pass
 * the template check); every workspace query at ordinary, zero, negative and
 * extreme sizes; and the rejection of bad arguments by every device entry
 * point.  A sanitizer report aborts the program; a wrong status code makes
 * it exit 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "medusa.h"

static int failures = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                         \
      fprintf(stderr, "\n");                                \
      ++failures;                                           \
    }                                                       \
  } while (0)

static uint64_t lcg_state = 12345;
static double uniform01(void) {  /* Knuth's MMIX LCG, top 53 bits */
  lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(lcg_state >> 11) / 9007199254740992.0;
}

static void check_strings(void) {
  EXPECT(medusa_abi_version() >= 1, "abi version");
  for (int s = -3; s <= 8; ++s) {
    const char* t = medusa_status_string(s);
    EXPECT(t != NULL && strlen(t) > 0, "status string %d", s);
  }
  EXPECT(medusa_last_error() != NULL, "last error");
}

static void check_tree_validate(void) {
  const int32_t chain_p[4] = {-1, 0, 1, 2}, chain_r[4] = {0, 0, 0, 0};
  EXPECT(medusa_tree_validate(chain_p, chain_r, 4, 3, 1) == MEDUSA_OK, "chain");
  EXPECT(medusa_tree_validate(chain_p, chain_r, 4, 2, 1) == MEDUSA_ERR_INVALID_ARG, "chain deeper than K");
  const int32_t star_p[5] = {-1, 0, 0, 0, 0}, star_r[5] = {0, 0, 1, 2, 3};
  EXPECT(medusa_tree_validate(star_p, star_r, 5, 1, 4) == MEDUSA_OK, "star");
  EXPECT(medusa_tree_validate(star_p, star_r, 5, 1, 3) == MEDUSA_ERR_INVALID_ARG, "rank >= topk");
  const int32_t dup_r[5] = {0, 0, 1, 1, 3};
  EXPECT(medusa_tree_validate(star_p, dup_r, 5, 1, 4) == MEDUSA_ERR_INVALID_ARG, "sibling ranks repeat");
  const int32_t fwd_p[3] = {-1, 2, 0}, z3[3] = {0, 0, 1};
  EXPECT(medusa_tree_validate(fwd_p, z3, 3, 4, 4) == MEDUSA_ERR_INVALID_ARG, "parent after child");
  const int32_t neg_p[3] = {-1, -5, 0};
  EXPECT(medusa_tree_validate(neg_p, z3, 3, 4, 4) == MEDUSA_ERR_INVALID_ARG, "parent below -1");
  const int32_t root_p[3] = {0, 0, 0};
  EXPECT(medusa_tree_validate(root_p, z3, 3, 4, 4) == MEDUSA_ERR_INVALID_ARG, "root with a parent");
  const int32_t negr[3] = {0, -1, 0};
  EXPECT(medusa_tree_validate(star_p, negr, 3, 4, 4) == MEDUSA_ERR_INVALID_ARG, "negative rank");
  EXPECT(medusa_tree_validate(chain_p, chain_r, 0, 3, 1) == MEDUSA_ERR_INVALID_ARG, "N = 0");
  EXPECT(medusa_tree_validate(chain_p, chain_r, 65, 3, 1) == MEDUSA_ERR_INVALID_ARG, "N = 65");
  EXPECT(medusa_tree_validate(NULL, chain_r, 4, 3, 1) == MEDUSA_ERR_INVALID_ARG, "NULL parent");
  EXPECT(medusa_tree_validate(chain_p, NULL, 4, 3, 1) == MEDUSA_ERR_INVALID_ARG, "NULL rank");
  /* a full 64-node chain of depth 63 */
  int32_t p64[64], r64[64];
  for (int i = 0; i < 64; ++i) { p64[i] = i - 1; r64[i] = 0; }
  EXPECT(medusa_tree_validate(p64, r64, 64, 63, 1) == MEDUSA_ERR_INVALID_ARG || 63 > MEDUSA_MAX_HEADS,
         "64-chain");
}

/* number of prefix-closed combinations of depth <= K with ranks < topk, capped */
static int64_t combos(int K, int topk) {
  int64_t total = 1, level = 1;
  for (int d = 1; d <= K; ++d) {
    level *= topk;
    total += level;
    if (total > 1000) return 1000;
  }
  return total;
}

static void check_tree_from_accuracy(void) {
  float acc[MEDUSA_MAX_HEADS * MEDUSA_MAX_TOPK];
  int32_t parent[MEDUSA_MAX_NODES], rank[MEDUSA_MAX_NODES];
  const int topks[] = {1, 2, 3, 4, 10, 64};
  for (int K = 1; K <= MEDUSA_MAX_HEADS; ++K)
    for (unsigned ti = 0; ti < sizeof(topks) / sizeof(topks[0]); ++ti) {
      const int topk = topks[ti];
      for (int i = 0; i < K * topk; ++i) acc[i] = (float)uniform01();
      if (K == 2 && topk == 4) for (int i = 0; i < K * topk; ++i) acc[i] = 0.5f;  /* all tied */
      if (K == 3 && topk == 3) for (int i = 0; i < K * topk; ++i) acc[i] = 0.f;   /* all zero */
      for (int N = 1; N <= MEDUSA_MAX_NODES; N += (N < 10 ? 1 : 7)) {
        double expected = -1.0;
        memset(parent, 0x7f, sizeof(parent));
        const int32_t st = medusa_tree_from_accuracy(acc, K, topk, N, parent, rank, &expected);
        if (N <= combos(K, topk)) {
          EXPECT(st == MEDUSA_OK, "tree_from_accuracy K=%d topk=%d N=%d: %d", K, topk, N, st);
          if (st == MEDUSA_OK) {
            EXPECT(medusa_tree_validate(parent, rank, N, K, topk) == MEDUSA_OK,
                   "sparse tree K=%d topk=%d N=%d does not validate", K, topk, N);
            EXPECT(isfinite(expected) && expected >= 0.0, "expected %g", expected);
          }
        } else {
          EXPECT(st != MEDUSA_OK, "K=%d topk=%d N=%d exceeds the combinations", K, topk, N);
        }
        EXPECT(medusa_tree_from_accuracy(acc, K, topk, N, parent, rank, NULL) == st, "NULL expected");
      }
    }
  for (int i = 0; i < 8; ++i) acc[i] = 0.5f;
  EXPECT(medusa_tree_from_accuracy(acc, 0, 4, 8, parent, rank, NULL) != MEDUSA_OK, "K = 0");
  EXPECT(medusa_tree_from_accuracy(acc, MEDUSA_MAX_HEADS + 1, 1, 8, parent, rank, NULL) != MEDUSA_OK, "K = 9");
  EXPECT(medusa_tree_from_accuracy(acc, 2, 0, 8, parent, rank, NULL) != MEDUSA_OK, "topk = 0");
  EXPECT(medusa_tree_from_accuracy(acc, 1, MEDUSA_MAX_TOPK + 1, 8, parent, rank, NULL) != MEDUSA_OK, "topk = 65");
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 0, parent, rank, NULL) != MEDUSA_OK, "N = 0");
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 65, parent, rank, NULL) != MEDUSA_OK, "N = 65");
  EXPECT(medusa_tree_from_accuracy(NULL, 2, 4, 8, parent, rank, NULL) != MEDUSA_OK, "NULL accuracy");
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 8, NULL, rank, NULL) != MEDUSA_OK, "NULL parent");
  acc[3] = 1.5f;
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 8, parent, rank, NULL) != MEDUSA_OK, "accuracy above 1");
  acc[3] = NAN;
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 8, parent, rank, NULL) != MEDUSA_OK, "NaN accuracy");
  acc[3] = -0.25f;
  EXPECT(medusa_tree_from_accuracy(acc, 2, 4, 8, parent, rank, NULL) != MEDUSA_OK, "negative accuracy");
}

/* The workspace queries must return (0 for impossible sizes) without
 * undefined behaviour for any argument values. */
static void check_workspace_queries(void) {
  const int64_t big[] = {-1, 0, 1, 64, 4096, 32000, INT32_MAX, (int64_t)INT32_MAX + 1, INT64_MAX / 2,
                         INT64_MAX};
  const int32_t small[] = {-1, 0, 1, 5, 64, 65, INT32_MAX};
  const int nb = sizeof(big) / sizeof(big[0]), ns = sizeof(small) / sizeof(small[0]);
  volatile size_t sink = 0;
  for (int a = 0; a < nb; ++a)
    for (int b = 0; b < nb; ++b)
      for (int c = 0; c < nb; ++c) {
        for (int dt = 0; dt <= 2; ++dt) {
          sink += medusa_linear_ws(big[a], big[b], big[c], 1, dt);
          sink += medusa_linear_ws(big[a], big[b], big[c], 7, dt);
        }
        for (int k = 0; k < ns; ++k) {
          sink += medusa_topk_ws(big[a], big[b], small[k]);
          sink += medusa_heads_ws(big[a], big[b], small[k], big[c], 10, 1);
          sink += medusa_heads_ws(big[a], big[b], 5, big[c], small[k], 0);
        }
      }
  for (int a = 0; a < nb; ++a)
    for (int b = 0; b < nb; ++b)
      for (int h = 0; h < ns; ++h)
        for (int d = 0; d < ns; ++d) sink += medusa_linear_qkv_rope_ws(big[a], big[b], small[h], small[h], small[d], 1);
  const int32_t heads[] = {-1, 0, 1, 32, 40, 64, INT32_MAX};
  const int32_t dims[] = {-1, 0, 64, 96, 128, 256, INT32_MAX};
  const int32_t ctxs[] = {-1, 0, 1, 2048, 1 << 20, INT32_MAX};
  const int32_t pages[] = {-1, 0, 3, 4, 12, 16, 4096, 4097, INT32_MAX};
  for (int b = 0; b < ns; ++b)
    for (int n = 0; n < ns; ++n) {
      sink += medusa_accept_ws(small[b], small[n]);
      sink += medusa_decode_tail_ws(small[b], small[n]);
      for (int h = 0; h < 7; ++h)
        for (int d = 0; d < 7; ++d)
          for (int c = 0; c < 6; ++c)
            for (int p = 0; p < 9; ++p) {
              sink += medusa_tree_attention_ws(small[b], small[n], heads[h], heads[h], dims[d], ctxs[c], pages[p]);
              for (int dt = -1; dt <= 2; ++dt)
                sink += (size_t)(medusa_tree_attention_splits(small[b], small[n], heads[h], heads[h],
                                                              dims[d], ctxs[c], pages[p], dt) + 1);
            }
    }
  (void)sink;
  /* the attention plan: one launch for a single 7B sequence's decode step,
     key splits for long ranges, large batches and fp32; -1 where the call
     rejects the shapes */
  EXPECT(medusa_tree_attention_splits(1, 64, 32, 32, 128, 928, 16, MEDUSA_BF16) == 0, "one launch");
  EXPECT(medusa_tree_attention_splits(1, 64, 32, 32, 128, 2048, 16, MEDUSA_BF16) > 0, "long range splits");
  EXPECT(medusa_tree_attention_splits(16, 64, 32, 32, 128, 928, 16, MEDUSA_BF16) > 0, "batch splits");
  EXPECT(medusa_tree_attention_splits(1, 64, 32, 32, 128, 928, 16, MEDUSA_F32) > 0, "fp32 splits");
  EXPECT(medusa_tree_attention_splits(1, 64, 32, 32, 96, 928, 16, MEDUSA_BF16) == -1, "D = 96");
  EXPECT(medusa_tree_attention_splits(1, 64, 32, 32, 128, 928, 16, 7) == -1, "unknown dtype");
  EXPECT(medusa_tree_attention_splits(0, 64, 32, 32, 128, 928, 16, MEDUSA_BF16) == -1, "B = 0");
  /* ordinary sizes stay exact */
  EXPECT(medusa_topk_ws(5, 4096, 10) == 0, "one chunk needs no workspace");
  EXPECT(medusa_topk_ws(5, 32000, 10) >= (size_t)5 * 8 * 10 * 8, "several chunks keep their candidates");
  EXPECT(medusa_accept_ws(1, 64) > 0, "accept ws");
}

static void check_rejections(void) {
  /* unknown dtype / epilogue; zero rows succeed without pointers */
  EXPECT(medusa_linear(NULL, 0, 4, 8, NULL, 4, 1, 7, 0, NULL, NULL, NULL, 0, NULL, 0, NULL) ==
             MEDUSA_ERR_UNSUPPORTED, "linear dtype");
  EXPECT(medusa_linear(NULL, 0, 4, 8, NULL, 4, 1, 1, 9, NULL, NULL, NULL, 0, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "linear epilogue");
  EXPECT(medusa_linear(NULL, 0, 0, 8, NULL, 4, 1, 1, 0, NULL, NULL, NULL, 0, NULL, 0, NULL) == MEDUSA_OK,
         "linear zero rows");
  EXPECT(medusa_linear(NULL, 0, 4, 8, NULL, 4, 1, 1, 0, NULL, NULL, NULL, 0, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "linear NULL operands");
  EXPECT(medusa_linear(NULL, 0, -4, 8, NULL, 4, 1, 1, 0, NULL, NULL, NULL, 0, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "linear negative rows");
  EXPECT(medusa_linear(NULL, 0, INT64_MAX, INT64_MAX, NULL, INT64_MAX, 1, 1, 0, NULL, NULL, NULL, 0, NULL, 0,
                       NULL) != MEDUSA_OK, "linear huge sizes");
  /* heads: K outside [1, 8], topk above 64, NULL weights */
  EXPECT(medusa_heads(NULL, 4, 256, 0, NULL, NULL, NULL, 1000, 1, NULL, 0, NULL, NULL, NULL, 0, NULL) != MEDUSA_OK,
         "heads K = 0");
  EXPECT(medusa_heads(NULL, 4, 256, 9, NULL, NULL, NULL, 1000, 1, NULL, 0, NULL, NULL, NULL, 0, NULL) != MEDUSA_OK,
         "heads K = 9");
  EXPECT(medusa_heads(NULL, 4, 256, 2, NULL, NULL, NULL, 1000, 1, NULL, 65, NULL, NULL, NULL, 0, NULL) != MEDUSA_OK,
         "heads topk = 65");
  EXPECT(medusa_heads(NULL, 4, 256, 2, NULL, NULL, NULL, 1000, 1, NULL, 4, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "heads NULL operands");
  EXPECT(medusa_heads_lists(NULL, 4, 256, 2, NULL, NULL, NULL, 1000, 1, 0, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_UNSUPPORTED, "heads lists topk = 0");
  EXPECT(medusa_heads_lists(NULL, 4, 256, 2, NULL, NULL, NULL, 1000, 1, 4, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "heads lists NULL operands");
  for (int64_t v = -2; v <= 3 * 4096 + 2; v += 2047)
    EXPECT(medusa_topk_lists(v) == (v >= 1 ? (int32_t)((v + 4095) / 4096) : 0), "topk lists V=%lld", (long long)v);
  EXPECT(medusa_topk_lists(INT64_MAX) == 0, "topk lists huge V");
  /* top-k: k outside [1, min(64, V)], NULL pointers, too small a workspace */
  EXPECT(medusa_topk(NULL, 2, 100, 0, NULL, NULL, NULL, 0, NULL) != MEDUSA_OK, "topk k = 0");
  EXPECT(medusa_topk(NULL, 2, 10, 11, NULL, NULL, NULL, 0, NULL) != MEDUSA_OK, "topk k > V");
  EXPECT(medusa_topk(NULL, 2, 100, 4, NULL, NULL, NULL, 0, NULL) == MEDUSA_ERR_INVALID_ARG, "topk NULL");
  EXPECT(medusa_topk(NULL, 0, 100, 4, NULL, NULL, NULL, 0, NULL) == MEDUSA_OK, "topk no rows");
  {
    const float* fake = (const float*)(uintptr_t)4096; /* never dereferenced: rejected first */
    EXPECT(medusa_topk(fake, 2, 32000, 4, (int32_t*)(uintptr_t)4096, (float*)(uintptr_t)4096, NULL, 0, NULL) ==
               MEDUSA_ERR_WORKSPACE, "topk workspace");
  }
  /* tree build: N outside [1, 64] */
  EXPECT(medusa_build_tree(1, 65, NULL, NULL, NULL, NULL, 2, 3, NULL, NULL, NULL, NULL, NULL) != MEDUSA_OK,
         "build_tree N = 65");
  EXPECT(medusa_build_tree(1, 0, NULL, NULL, NULL, NULL, 2, 3, NULL, NULL, NULL, NULL, NULL) != MEDUSA_OK,
         "build_tree N = 0");
  EXPECT(medusa_build_tree(1, 9, NULL, NULL, NULL, NULL, 2, 3, NULL, NULL, NULL, NULL, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "build_tree NULL");
  /* tree attention: head dim, GQA ratio, page size, N, NULL pointers */
  EXPECT(medusa_tree_attention(NULL, NULL, NULL, NULL, NULL, NULL, 8, 16, NULL, 100, NULL, 1, 9, 4, 4, 96, 0.1f,
                               1, NULL, NULL, 0, NULL) != MEDUSA_OK, "attention D = 96");
  EXPECT(medusa_tree_attention(NULL, NULL, NULL, NULL, NULL, NULL, 8, 16, NULL, 100, NULL, 1, 9, 6, 4, 128, 0.1f,
                               1, NULL, NULL, 0, NULL) != MEDUSA_OK, "attention Hq not a multiple of Hkv");
  EXPECT(medusa_tree_attention(NULL, NULL, NULL, NULL, NULL, NULL, 8, 3, NULL, 100, NULL, 1, 9, 4, 4, 128, 0.1f,
                               1, NULL, NULL, 0, NULL) != MEDUSA_OK, "attention P = 3");
  EXPECT(medusa_tree_attention(NULL, NULL, NULL, NULL, NULL, NULL, 8, 16, NULL, 100, NULL, 1, 65, 4, 4, 128, 0.1f,
                               1, NULL, NULL, 0, NULL) != MEDUSA_OK, "attention N = 65");
  EXPECT(medusa_tree_attention(NULL, NULL, NULL, NULL, NULL, NULL, 8, 16, NULL, 100, NULL, 1, 9, 4, 4, 128, 0.1f,
                               1, NULL, NULL, 0, NULL) == MEDUSA_ERR_INVALID_ARG, "attention NULL");
  EXPECT(medusa_tree_attention_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, 8, 16, NULL, 100, NULL, 1, 9, 4, 4,
                                       96, 0.1f, 1, NULL, NULL) != MEDUSA_OK, "noalloc D = 96");
  EXPECT(medusa_tree_attention_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, 1 << 20, 16, NULL, 1 << 24, NULL, 64,
                                       64, 64, 64, 128, 0.1f, 1, NULL, NULL) != MEDUSA_OK,
         "noalloc beyond its array");
  /* acceptance: mode, N, temperature */
  EXPECT(medusa_accept(NULL, 100, NULL, NULL, 1, 9, 2, 5, 1.f, 0.3f, 0.09f, NULL, NULL, NULL, NULL, 0, NULL) !=
             MEDUSA_OK, "accept mode");
  EXPECT(medusa_accept(NULL, 100, NULL, NULL, 1, 65, 2, 0, 1.f, 0.3f, 0.09f, NULL, NULL, NULL, NULL, 0, NULL) !=
             MEDUSA_OK, "accept N = 65");
  EXPECT(medusa_accept_sample(NULL, 100, NULL, NULL, 1, 9, 2, 0.f, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_INVALID_ARG, "sample T = 0");
  EXPECT(medusa_accept_sample(NULL, 100, NULL, NULL, 1, 65, 2, 1.f, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_UNSUPPORTED, "sample N = 65");
  EXPECT(medusa_accept_sample(NULL, 100, NULL, NULL, 0, 9, 2, 1.f, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_OK, "sample empty batch");
  /* norms and small kernels: eps < 0, H not a multiple of 4, dtype */
  EXPECT(medusa_rmsnorm(NULL, 2, 64, NULL, -1.f, 1, NULL, NULL) == MEDUSA_ERR_INVALID_ARG, "rmsnorm eps");
  EXPECT(medusa_rmsnorm(NULL, 2, 62, NULL, 1e-5f, 1, NULL, NULL) != MEDUSA_OK, "rmsnorm H");
  EXPECT(medusa_rmsnorm(NULL, 2, 64, NULL, 1e-5f, 5, NULL, NULL) != MEDUSA_OK, "rmsnorm dtype");
  EXPECT(medusa_linear_rmsnorm(NULL, 4, 64, NULL, 10, 1, NULL, NULL, 1e-5f, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_UNSUPPORTED, "linear_rmsnorm N");
  EXPECT(medusa_linear_qkv_rope(NULL, 4, 64, NULL, 2, 2, 6, NULL, 10000.f, 1, NULL, NULL, NULL, NULL, 0, NULL) ==
             MEDUSA_ERR_UNSUPPORTED, "qkv_rope D");
  /* 16-byte alignment of every tensor the projections and the rotary pass
     touch with vector accesses (addresses never read: rejected before any
     launch) */
  {
    void* const al = (void*)(uintptr_t)256;
    void* const mis8 = (void*)(uintptr_t)(256 + 8);
    void* const mis4 = (void*)(uintptr_t)(256 + 4);
    EXPECT(medusa_linear(al, 0, 4, 8, al, 4, 1, MEDUSA_BF16, MEDUSA_EPI_NONE, NULL, NULL, mis8, 0, NULL, 0,
                         NULL) == MEDUSA_ERR_INVALID_ARG, "linear Y alignment");
    EXPECT(medusa_linear(al, 0, 4, 8, al, 4, 1, MEDUSA_BF16, MEDUSA_EPI_RES_ADD_F32, NULL, mis4, al, 0, NULL, 0,
                         NULL) == MEDUSA_ERR_INVALID_ARG, "linear aux alignment");
    EXPECT(medusa_linear(al, 0, 4, 8, al, 8, 1, MEDUSA_BF16, MEDUSA_EPI_BIAS_SILU_RES, mis8, al, al, 0, NULL, 0,
                         NULL) == MEDUSA_ERR_INVALID_ARG, "linear bias alignment");
    EXPECT(medusa_linear_qkv_rope(al, 4, 64, al, 2, 2, 8, (const int32_t*)al, 10000.f, MEDUSA_BF16, mis8, al, al,
                                  NULL, 0, NULL) == MEDUSA_ERR_INVALID_ARG, "linear_qkv_rope q alignment");
    EXPECT(medusa_qkv_rope(al, 4, 2, 2, 8, (const int32_t*)al, 10000.f, MEDUSA_BF16, al, mis8, al, NULL) ==
               MEDUSA_ERR_INVALID_ARG, "qkv_rope k alignment");
  }
  /* fused decode tail and fused tree embedding (addresses never read) */
  {
    const uintptr_t a = 256;
    const void* pools[1] = {(const void*)(uintptr_t)256};
#define TAIL(K, mode, T, D, H, B, ws, nbytes)                                                             \
  medusa_decode_tail((const float*)a, 1000, (const int32_t*)a, (const int32_t*)a, B, 64, K, mode, T, 0.3f,  \
                     0.09f, (uint64_t*)a, (void* const*)pools, (void* const*)pools, 1, (const int32_t*)a, 8, \
                     16, 2, D, 1, (const void*)a, H, (int32_t*)a, (int32_t*)a, (int32_t*)a, (int32_t*)a,      \
                     (int32_t*)a, (int32_t*)a, (int32_t*)a, 16, ws, nbytes, NULL)
    EXPECT(TAIL(9, 0, 1.f, 128, 256, 1, NULL, 0) == MEDUSA_ERR_UNSUPPORTED, "tail K = 9");
    EXPECT(TAIL(5, 3, 1.f, 128, 256, 1, NULL, 0) == MEDUSA_ERR_INVALID_ARG, "tail mode");
    EXPECT(TAIL(5, 2, 0.f, 128, 256, 1, NULL, 0) == MEDUSA_ERR_INVALID_ARG, "tail T");
    EXPECT(TAIL(5, 0, 1.f, 96, 256, 1, NULL, 0) == MEDUSA_ERR_UNSUPPORTED, "tail D");
    EXPECT(TAIL(5, 0, 1.f, 128, 4, 1, NULL, 0) == MEDUSA_ERR_INVALID_ARG, "tail H");
    EXPECT(TAIL(5, 0, 1.f, 128, 256, 0, NULL, 0) == MEDUSA_OK, "tail empty batch");
    EXPECT(TAIL(5, 0, 1.f, 128, 256, 1, NULL, 0) == MEDUSA_ERR_WORKSPACE, "tail workspace");
#undef TAIL
    EXPECT(medusa_tree_embed(1, 9, NULL, NULL, NULL, NULL, NULL, 1, 2, 3, NULL, NULL, NULL, NULL, NULL, 100, 250,
                             1, NULL, 1e-5f, NULL, NULL, NULL) == MEDUSA_ERR_UNSUPPORTED, "embed H");
    EXPECT(medusa_tree_embed(1, 65, NULL, NULL, NULL, NULL, NULL, 1, 2, 3, NULL, NULL, NULL, NULL, NULL, 100, 256,
                             1, NULL, 1e-5f, NULL, NULL, NULL) == MEDUSA_ERR_INVALID_ARG, "embed N");
    EXPECT(medusa_tree_embed(1, 9, NULL, NULL, NULL, NULL, NULL, 0, 2, 3, NULL, NULL, NULL, NULL, NULL, 100, 256,
                             1, NULL, 1e-5f, NULL, NULL, NULL) == MEDUSA_ERR_INVALID_ARG, "embed lists = 0");
    EXPECT(medusa_tree_embed(1, 9, NULL, NULL, NULL, NULL, NULL, 65, 2, 3, NULL, NULL, NULL, NULL, NULL, 100, 256,
                             1, NULL, 1e-5f, NULL, NULL, NULL) == MEDUSA_ERR_INVALID_ARG, "embed lists = 65");
    EXPECT(medusa_tree_embed(0, 9, NULL, NULL, NULL, NULL, NULL, 1, 2, 3, NULL, NULL, NULL, NULL, NULL, 100, 256,
                             1, NULL, 1e-5f, NULL, NULL, NULL) == MEDUSA_OK, "embed empty batch");
  }
  EXPECT(strlen(medusa_last_error()) > 0, "a rejection leaves a message");
}

int main(void) {
  check_strings();
  check_tree_validate();
  check_tree_from_accuracy();
  check_workspace_queries();
  check_rejections();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
