// Host-side parts of the C ABI: status strings, the thread-local last error,
// and the tree-template check.
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
