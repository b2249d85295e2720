// Host-side parts of the C ABI: status strings, the thread-local last error,
// the tree-template check and the accuracy-driven sparse tree.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace medusa_host {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_last_error[0] = 0;
  return MEDUSA_OK;
}

}  // namespace medusa_host

extern "C" const char* medusa_status_string(int32_t status) {
  switch (status) {
    case MEDUSA_OK: return "ok";
    case MEDUSA_ERR_INVALID_ARG: return "invalid argument";
    case MEDUSA_ERR_UNSUPPORTED: return "unsupported dtype, shape or size";
    case MEDUSA_ERR_WORKSPACE: return "workspace too small";
    case MEDUSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

extern "C" const char* medusa_last_error(void) { return medusa_host::g_last_error; }

extern "C" int32_t medusa_abi_version(void) { return 1; }

extern "C" int32_t medusa_tree_validate(const int32_t* parent, const int32_t* rank, int32_t N,
                                        int32_t K, int32_t topk) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(parent && rank, MEDUSA_ERR_INVALID_ARG, "tree_validate: NULL template");
  MEDUSA_REQUIRE(N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_INVALID_ARG,
                 "tree_validate: N=%d outside [1, %d]", N, MEDUSA_MAX_NODES);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_HEADS, MEDUSA_ERR_INVALID_ARG,
                 "tree_validate: K=%d outside [0, %d]", K, MEDUSA_MAX_HEADS);
  MEDUSA_REQUIRE(topk >= 1 && topk <= MEDUSA_MAX_TOPK, MEDUSA_ERR_INVALID_ARG,
                 "tree_validate: topk=%d outside [1, %d]", topk, MEDUSA_MAX_TOPK);
  MEDUSA_REQUIRE(parent[0] == -1, MEDUSA_ERR_INVALID_ARG, "tree_validate: parent[0] must be -1");
  int depth[MEDUSA_MAX_NODES];
  depth[0] = 0;
  for (int i = 1; i < N; ++i) {
    const int p = parent[i];
    MEDUSA_REQUIRE(p >= 0 && p < i, MEDUSA_ERR_INVALID_ARG,
                   "tree_validate: parent[%d]=%d must be in [0, %d)", i, p, i);
    depth[i] = depth[p] + 1;
    MEDUSA_REQUIRE(depth[i] <= K, MEDUSA_ERR_INVALID_ARG,
                   "tree_validate: node %d has depth %d > K=%d", i, depth[i], K);
    MEDUSA_REQUIRE(rank[i] >= 0 && rank[i] < topk, MEDUSA_ERR_INVALID_ARG,
                   "tree_validate: rank[%d]=%d outside [0, %d)", i, rank[i], topk);
    for (int j = 1; j < i; ++j)
      MEDUSA_REQUIRE(!(parent[j] == p && rank[j] == rank[i]), MEDUSA_ERR_INVALID_ARG,
                     "tree_validate: siblings %d and %d share rank %d", j, i, rank[i]);
  }
  return MEDUSA_OK;
}

// The sparse tree of the most accurate head combinations ("Medusa Heads",
// section "Attenzione sull'albero e accettazione": a sparse 64-node tree
// built from the most accurate combinations beat a dense 256-node one).
// A combination (r1..rd) has accuracy prod_j accuracy[j][r_j]; the root and
// the N-1 most accurate combinations are kept (ties: shallower, then the
// lexicographically smaller rank tuple).  Accuracies are at most 1, so a
// combination never beats its prefix and the best remaining combination
// always has its whole prefix kept: a frontier of the kept nodes' children
// yields the global order without enumerating every combination.
namespace {
struct Combo {
  double value;
  int depth;
  int r[MEDUSA_MAX_HEADS];
};
// a before b in the selection order
bool combo_first(const Combo& a, const Combo& b) {
  if (a.value != b.value) return a.value > b.value;
  if (a.depth != b.depth) return a.depth < b.depth;
  for (int j = 0; j < a.depth; ++j)
    if (a.r[j] != b.r[j]) return a.r[j] < b.r[j];
  return false;
}
// a before b in the canonical order (depth, then rank tuple)
bool combo_canonical(const Combo& a, const Combo& b) {
  if (a.depth != b.depth) return a.depth < b.depth;
  for (int j = 0; j < a.depth; ++j)
    if (a.r[j] != b.r[j]) return a.r[j] < b.r[j];
  return false;
}
}  // namespace

extern "C" int32_t medusa_tree_from_accuracy(const float* accuracy, int32_t K, int32_t topk, int32_t N,
                                             int32_t* parent, int32_t* rank, double* expected) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(accuracy && parent && rank, MEDUSA_ERR_INVALID_ARG, "tree_from_accuracy: NULL pointer");
  MEDUSA_REQUIRE(K >= 1 && K <= MEDUSA_MAX_HEADS, MEDUSA_ERR_INVALID_ARG,
                 "tree_from_accuracy: K=%d outside [1, %d]", K, MEDUSA_MAX_HEADS);
  MEDUSA_REQUIRE(topk >= 1 && topk <= MEDUSA_MAX_TOPK, MEDUSA_ERR_INVALID_ARG,
                 "tree_from_accuracy: topk=%d outside [1, %d]", topk, MEDUSA_MAX_TOPK);
  MEDUSA_REQUIRE(N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_INVALID_ARG,
                 "tree_from_accuracy: N=%d outside [1, %d]", N, MEDUSA_MAX_NODES);
  int64_t avail = 1, level = 1;
  for (int d = 0; d < K && avail < N; ++d) {
    level *= topk;
    avail += level;
  }
  MEDUSA_REQUIRE(avail >= N, MEDUSA_ERR_INVALID_ARG,
                 "tree_from_accuracy: only %lld combinations for N=%d", (long long)avail, N);
  for (int i = 0; i < K * topk; ++i)
    MEDUSA_REQUIRE(isfinite(accuracy[i]) && accuracy[i] >= 0.f && accuracy[i] <= 1.f,
                   MEDUSA_ERR_INVALID_ARG, "tree_from_accuracy: accuracy[%d]=%g outside [0, 1]", i,
                   (double)accuracy[i]);
  // kept nodes (root first) and the frontier of their children
  Combo kept[MEDUSA_MAX_NODES];
  static thread_local Combo frontier[MEDUSA_MAX_NODES * MEDUSA_MAX_TOPK];
  int nkept = 0, nfront = 0;
  kept[nkept++] = Combo{1.0, 0, {}};
  double sum = 0.0;
  auto push_children = [&](const Combo& c) {
    if (c.depth >= K) return;
    for (int r = 0; r < topk; ++r) {
      Combo ch = c;
      ch.value = c.value * (double)accuracy[c.depth * topk + r];
      ch.r[c.depth] = r;
      ch.depth = c.depth + 1;
      frontier[nfront++] = ch;
    }
  };
  push_children(kept[0]);
  while (nkept < N) {
    int best = 0;
    for (int i = 1; i < nfront; ++i)
      if (combo_first(frontier[i], frontier[best])) best = i;
    const Combo c = frontier[best];
    frontier[best] = frontier[--nfront];
    kept[nkept++] = c;
    sum += c.value;
    push_children(c);
  }
  // canonical order, then parents by prefix
  for (int i = 1; i < nkept; ++i)  // insertion sort (N <= 64)
    for (int j = i; j > 1 && combo_canonical(kept[j], kept[j - 1]); --j) {
      const Combo t = kept[j];
      kept[j] = kept[j - 1];
      kept[j - 1] = t;
    }
  parent[0] = -1;
  rank[0] = 0;
  for (int i = 1; i < nkept; ++i) {
    const Combo& c = kept[i];
    int p = 0;
    for (int j = 0; j < i; ++j)
      if (kept[j].depth == c.depth - 1) {
        bool prefix = true;
        for (int q = 0; q < c.depth - 1; ++q) prefix = prefix && kept[j].r[q] == c.r[q];
        if (prefix) { p = j; break; }
      }
    parent[i] = p;
    rank[i] = c.r[c.depth - 1];
  }
  if (expected) *expected = sum;
  set_error("");
  return MEDUSA_OK;
}
