// medusa_build_tree: tokens, positions and ancestor masks of B candidate
// trees ("Medusa Heads", section "Attenzione sull'albero e accettazione": the
// Cartesian product of the heads' top-k is a prefix-sharing tree, and each
// candidate token may see only its own ancestors).
//
// One thread per node.  A node walks its parent links (at most 64 steps) to
// find its depth and to OR its ancestors' bits into its mask.
#include "common.h"

namespace medusa {

__global__ __launch_bounds__(64) void build_tree_kernel(int N, const int* __restrict__ parent,
                                                        const int* __restrict__ rank,
                                                        const int* __restrict__ root_tok,
                                                        const int* __restrict__ topk_ids,
                                                        int B, int topk,
                                                        const int* __restrict__ ctx,
                                                        int* __restrict__ tokens,
                                                        int* __restrict__ pos,
                                                        uint64_t* __restrict__ mask) {
  const int b = blockIdx.x, i = threadIdx.x;
  if (i >= N) return;
  const int* par = parent + (int64_t)b * N;
  uint64_t m = 0;
  int depth = 0, j = i;
  for (int step = 0; step < MEDUSA_MAX_NODES && j >= 0; ++step) {
    m |= 1ull << j;
    j = par[j];
    depth += (j >= 0);
  }
  const int64_t o = (int64_t)b * N + i;
  tokens[o] = depth == 0 ? root_tok[b]
                         : topk_ids[((int64_t)(depth - 1) * B + b) * topk + rank[o]];
  pos[o] = ctx[b] + depth;
  mask[o] = m;
}

}  // namespace medusa

extern "C" int32_t medusa_build_tree(int32_t B, int32_t N, const int32_t* parent,
                                     const int32_t* rank, const int32_t* root_tok,
                                     const int32_t* topk_ids, int32_t K, int32_t topk,
                                     const int32_t* ctx, int32_t* tokens, int32_t* pos,
                                     uint64_t* mask, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_INVALID_ARG,
                 "medusa_build_tree: B=%d N=%d (N must be in [1, 64])", B, N);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_HEADS && topk >= 1 && topk <= MEDUSA_MAX_TOPK,
                 MEDUSA_ERR_INVALID_ARG, "medusa_build_tree: K=%d topk=%d", K, topk);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(parent && rank && root_tok && ctx && tokens && pos && mask &&
                     (topk_ids || N == 1),
                 MEDUSA_ERR_INVALID_ARG, "medusa_build_tree: NULL pointer");
  hipLaunchKernelGGL(medusa::build_tree_kernel, dim3(B), dim3(64), 0, (hipStream_t)stream, N,
                     parent, rank, root_tok, topk_ids, B, topk, ctx, tokens, pos, mask);
  return check_launch("medusa_build_tree");
}
