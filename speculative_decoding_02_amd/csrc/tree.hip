// medusa_build_tree: tokens, positions and ancestor masks of B candidate
// trees ("Medusa Heads", section "Attenzione sull'albero e accettazione": the
// Cartesian product of the heads' top-k is a prefix-sharing tree, and each
// candidate token may see only its own ancestors).
//
// One thread per node.  A node walks its parent links (at most 64 steps) to
// find its depth and to OR its ancestors' bits into its mask.
#include "common.h"
#include "topk_wave.h"

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

// medusa_build_tree, the embedding of the tree's rows and the first RMSNorm
// in one launch: one workgroup per (node, sequence).  Wave 0 finds the
// node's ancestors by walking the parent links through lane shuffles (lane j
// holds parent[j]; one step per tree level), picks the node's token and
// writes the tree outputs; then the workgroup copies the token's embedding
// row into the fp32 residual stream and normalises it (the RMSNorm kernel's
// helpers, so the results equal the separate calls' bit for bit).  With
// lists > 1 the heads' rows come as per-chunk candidate lists (ids and
// values, lists x topk per row) and wave 0 merges its row's lists to find the
// token of the node's rank: the same total order (value descending, lower id
// first) as the top-k's own merge, so the same token.
template <typename T>
__global__ __launch_bounds__(256) void tree_embed_kernel(
    int N, const int* __restrict__ parent, const int* __restrict__ rank,
    const int* __restrict__ root_tok, const int* __restrict__ topk_ids,
    const float* __restrict__ topk_vals, int lists, int B, int topk,
    const int* __restrict__ ctx, int* __restrict__ tokens, int* __restrict__ pos,
    uint64_t* __restrict__ mask, const T* __restrict__ table, int64_t H,
    const T* __restrict__ gain, float eps, float* __restrict__ x, T* __restrict__ h) {
  const int n = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t o = (int64_t)b * N + n;
  __shared__ int s_tok;
  f32x4 g[RMS_V4];
  rms_row_gain<T>(gain, H, g);
  if (tid < 64) {
    const int par = tid < N ? min(parent[(int64_t)b * N + tid], MEDUSA_MAX_NODES - 1) : -1;
    uint64_t anc = tid < N ? 1ull << tid : 0ull;
    int j = par;
    for (int it = 0; it < MEDUSA_MAX_NODES && __ballot(j >= 0) != 0; ++it) {
      const int jn = __shfl(par, max(j, 0), 64);
      if (j >= 0) {
        anc |= 1ull << j;
        j = jn;
      }
    }
    const uint32_t lo = __shfl((uint32_t)anc, n, 64), hi = __shfl((uint32_t)(anc >> 32), n, 64);
    const uint64_t an = ((uint64_t)hi << 32) | lo;
    const int depth = __popcll(an) - 1;  // the same in every lane
    const int64_t hrow = (int64_t)max(depth - 1, 0) * B + b;  // the heads' row of this node
    int tok = 0;
    if (depth > 0 && lists > 1) {
      const int64_t c0 = hrow * lists * topk;
      const uint64_t top = merge_lists_wave(topk_ids + c0, topk_vals + c0, lists * topk);
      tok = key_index(((uint64_t)__shfl((uint32_t)(top >> 32), rank[o], 64) << 32) |
                      __shfl((uint32_t)top, rank[o], 64));
    }
    if (tid == 0) {
      if (depth == 0) tok = root_tok[b];
      else if (lists == 1) tok = topk_ids[hrow * topk + rank[o]];
      tokens[o] = tok;
      pos[o] = ctx[b] + depth;
      mask[o] = an;
      s_tok = tok;
    }
  }
  __syncthreads();
  const T* row = table + (int64_t)s_tok * H;
  const int64_t H4 = H / 4;
  f32x4 v[RMS_V4];
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    const int64_t e = tid + (int64_t)i * 256;
    v[i] = Elem<T>::load4(row, e < H4 ? e : 0);
  }
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    const int64_t e = tid + (int64_t)i * 256;
    if (e < H4) Elem<float>::store4(x + o * H, e, v[i]);
  }
  const float rs = rms_row_scale(v, H, eps);
  rms_row_store<T>(v, H, rs, g, h + o * H);
}

}  // namespace medusa

extern "C" int32_t medusa_tree_embed(int32_t B, int32_t N, const int32_t* parent,
                                     const int32_t* rank, const int32_t* root_tok,
                                     const int32_t* topk_ids, const float* topk_vals,
                                     int32_t lists, int32_t K, int32_t topk,
                                     const int32_t* ctx, int32_t* tokens, int32_t* pos,
                                     uint64_t* mask, const void* table, int64_t V, int64_t H,
                                     int32_t dt, const void* gain, float eps, float* x, void* h,
                                     void* stream) {
  using namespace medusa_host;
  const char* fn = "medusa_tree_embed";
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_INVALID_ARG,
                 "%s: B=%d N=%d (N must be in [1, 64])", fn, B, N);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_HEADS && topk >= 1 && topk <= MEDUSA_MAX_TOPK,
                 MEDUSA_ERR_INVALID_ARG, "%s: K=%d topk=%d", fn, K, topk);
  MEDUSA_REQUIRE(lists >= 1 && lists <= MEDUSA_MAX_TOPK_LISTS, MEDUSA_ERR_INVALID_ARG,
                 "%s: lists=%d outside [1, %d]", fn, lists, MEDUSA_MAX_TOPK_LISTS);
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "%s: dtype", fn);
  MEDUSA_REQUIRE(V >= 1 && eps >= 0.f && H % 4 == 0 && H >= 4 && H <= 4 * 256 * medusa::RMS_V4,
                 MEDUSA_ERR_UNSUPPORTED, "%s: needs V >= 1, eps >= 0, H a multiple of 4 and H <= %d",
                 fn, 4 * 256 * medusa::RMS_V4);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(parent && rank && root_tok && ctx && tokens && pos && mask && table && x && h &&
                     (topk_ids || N == 1) && (topk_vals || lists == 1 || N == 1),
                 MEDUSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  const int a4 = dt == MEDUSA_BF16 ? 8 : 16;  // four elements of table, gain and h
  MEDUSA_REQUIRE(((uintptr_t)x) % 16 == 0 && ((uintptr_t)table | (uintptr_t)gain | (uintptr_t)h) % a4 == 0,
                 MEDUSA_ERR_INVALID_ARG, "%s: x must be 16-byte aligned, table, gain and h %d", fn, a4);
  hipStream_t st = (hipStream_t)stream;
  if (dt == MEDUSA_BF16)
    hipLaunchKernelGGL(medusa::tree_embed_kernel<medusa::bf16_t>, dim3(N, B), dim3(256), 0, st, N,
                       parent, rank, root_tok, topk_ids, topk_vals, lists, B, topk, ctx, tokens,
                       pos, mask,
                       (const medusa::bf16_t*)table, H, (const medusa::bf16_t*)gain, eps, x,
                       (medusa::bf16_t*)h);
  else
    hipLaunchKernelGGL(medusa::tree_embed_kernel<float>, dim3(N, B), dim3(256), 0, st, N, parent,
                       rank, root_tok, topk_ids, topk_vals, lists, B, topk, ctx, tokens, pos, mask,
                       (const float*)table, H, (const float*)gain, eps, x, (float*)h);
  return check_launch(fn);
}

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
