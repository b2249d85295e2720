// medusa_heads: K Medusa heads on M hidden rows, then per-head top-k.
// ("Medusa Heads", section "Come le teste prevedono i token successivi":
// head k = one feed-forward layer with SiLU and a residual connection, then a
// vocabulary projection, all reading the hidden state lm_head reads.)
//
// Two batched GEMM launches (batch = heads):
//   U_k      = X + SiLU(X W1_k^T + b1_k)     fused epilogue, U kept in ws
//   logits_k = U_k W2_k^T                     fp32
// then one top-k launch over the K*M logits rows.  Stage 2 and a plain
// lm_head projection run the same kernel with the same contraction length,
// so zero-initialised heads reproduce lm_head's logits bit for bit.
#include <algorithm>

#include "common.h"

namespace medusa_host {
void launch_gemm(const void* X, int64_t xbs, int64_t M, int64_t Kd, const void* W, int64_t Nw,
                 int batch, int dt, int epi, const void* bias, const void* aux, void* Y,
                 int y_f32, void* ws, hipStream_t st);
size_t gemm_ws_bytes(int64_t M, int64_t Kd, int64_t Nw, int batch, int dt);
void launch_topk(const float* logits, int64_t R, int64_t V, int k, int* ids, float* vals, void* ws,
                 hipStream_t st);
size_t topk_ws_bytes(int64_t R, int64_t V, int k);
void launch_topk_lists(const float* logits, int64_t R, int64_t V, int k, int* ids, float* vals,
                       hipStream_t st);
}  // namespace medusa_host

extern "C" size_t medusa_heads_ws(int64_t M, int64_t H, int32_t K, int64_t V, int32_t topk,
                                  int32_t dt) {
  // shapes medusa_heads rejects (or M = 0) need nothing
  if (M <= 0 || H <= 0 || V <= 0 || K < 1 || K > MEDUSA_MAX_HEADS || topk < 0 ||
      topk > MEDUSA_MAX_TOPK || M > INT32_MAX || H > INT32_MAX || V > INT32_MAX ||
      (dt != MEDUSA_F32 && dt != MEDUSA_BF16))
    return 0;
  const size_t es = dt == MEDUSA_BF16 ? 2 : 4;
  using namespace medusa_host;
  const size_t gws = std::max(gemm_ws_bytes(M, H, H, K, dt), gemm_ws_bytes(M, H, V, K, dt));
  return align_up((size_t)K * M * H * es, 256) + align_up((size_t)K * M * V * 4, 256) +
         std::max(topk_ws_bytes((int64_t)K * M, V, topk), gws);
}

// lists: topk_ids/topk_vals receive the per-chunk lists [K, M, S, topk]
// instead of the merged top-k (stage 2 left to the consumer)
static int32_t heads_impl(const void* X, int64_t M, int64_t H, int32_t K, const void* W1,
                          const void* b1, const void* W2, int64_t V, int32_t dt, float* logits,
                          int32_t topk, int32_t* topk_ids, float* topk_vals, void* ws,
                          size_t ws_bytes, void* stream, bool lists) {
  using namespace medusa_host;
  const char* fn = lists ? "medusa_heads_lists" : "medusa_heads";
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "%s: unknown dtype %d", fn, dt);
  MEDUSA_REQUIRE(M >= 0 && H > 0 && V > 0 && M <= INT32_MAX && H <= INT32_MAX && V <= INT32_MAX,
                 MEDUSA_ERR_INVALID_ARG, "%s: bad sizes M=%lld H=%lld V=%lld", fn,
                 (long long)M, (long long)H, (long long)V);
  MEDUSA_REQUIRE(K >= 1 && K <= MEDUSA_MAX_HEADS, MEDUSA_ERR_UNSUPPORTED,
                 "%s: K=%d outside [1, %d]", fn, K, MEDUSA_MAX_HEADS);
  MEDUSA_REQUIRE(topk >= 0 && topk <= MEDUSA_MAX_TOPK && topk <= V, MEDUSA_ERR_UNSUPPORTED,
                 "%s: topk=%d outside [0, min(64, V)]", fn, topk);
  const int p16 = dt == MEDUSA_BF16 ? 8 : 4;
  MEDUSA_REQUIRE(H % p16 == 0, MEDUSA_ERR_UNSUPPORTED, "%s: H must be a multiple of %d", fn, p16);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(X && W1 && W2, MEDUSA_ERR_INVALID_ARG, "%s: NULL X, W1 or W2", fn);
  MEDUSA_REQUIRE(((uintptr_t)X | (uintptr_t)W1 | (uintptr_t)W2) % 16 == 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: X, W1, W2 must be 16-byte aligned", fn);
  MEDUSA_REQUIRE(topk == 0 || (topk_ids && topk_vals), MEDUSA_ERR_INVALID_ARG,
                 "%s: NULL top-k outputs", fn);
  const size_t need = medusa_heads_ws(M, H, K, V, topk, dt);
  MEDUSA_REQUIRE(ws != NULL && ws_bytes >= need, MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  MEDUSA_REQUIRE((uintptr_t)ws % 256 == 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: ws must be 256-byte aligned", fn);
  const size_t es = dt == MEDUSA_BF16 ? 2 : 4;
  char* U = (char*)ws;
  char* lg_ws = U + align_up((size_t)K * M * H * es, 256);
  float* lg = logits ? logits : (float*)lg_ws;
  void* tk_ws = lg_ws + align_up((size_t)K * M * V * 4, 256);  // also the projections' split space
  hipStream_t st = (hipStream_t)stream;
  launch_gemm(X, 0, M, H, W1, H, K, dt, MEDUSA_EPI_BIAS_SILU_RES, b1, X, U, 0, tk_ws, st);
  launch_gemm(U, M * H, M, H, W2, V, K, dt, MEDUSA_EPI_NONE, nullptr, nullptr, lg, 1, tk_ws, st);
  if (topk > 0 && lists) launch_topk_lists(lg, (int64_t)K * M, V, topk, topk_ids, topk_vals, st);
  else if (topk > 0) launch_topk(lg, (int64_t)K * M, V, topk, topk_ids, topk_vals, tk_ws, st);
  return check_launch(fn);
}

extern "C" int32_t medusa_heads(const void* X, int64_t M, int64_t H, int32_t K, const void* W1,
                                const void* b1, const void* W2, int64_t V, int32_t dt,
                                float* logits, int32_t topk, int32_t* topk_ids,
                                float* topk_vals, void* ws, size_t ws_bytes, void* stream) {
  return heads_impl(X, M, H, K, W1, b1, W2, V, dt, logits, topk, topk_ids, topk_vals, ws, ws_bytes,
                    stream, false);
}

extern "C" int32_t medusa_heads_lists(const void* X, int64_t M, int64_t H, int32_t K,
                                      const void* W1, const void* b1, const void* W2, int64_t V,
                                      int32_t dt, int32_t topk, int32_t* list_ids,
                                      float* list_vals, void* ws, size_t ws_bytes, void* stream) {
  MEDUSA_REQUIRE(topk >= 1, MEDUSA_ERR_UNSUPPORTED, "medusa_heads_lists: topk=%d below 1", topk);
  return heads_impl(X, M, H, K, W1, b1, W2, V, dt, nullptr, topk, list_ids, list_vals, ws, ws_bytes,
                    stream, true);
}
