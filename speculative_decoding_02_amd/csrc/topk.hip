// Row-wise top-k of float logits ("Medusa Heads", section "Attenzione
// sull'albero e accettazione": the heads' best guesses feed the tree).
// Order: value descending, equal values by lower index.
//
// One workgroup (256 threads) per row.  Each thread streams its strided
// share of the row (coalesced: consecutive lanes read consecutive floats)
// and keeps a sorted candidate list in registers; the lists are then merged
// by k rounds of a block-wide "best head" selection.
#include "common.h"

namespace medusa {

struct Cand {
  float v;
  int i;
};
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int KMAX>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int64_t V,
                                                   int k, int* __restrict__ ids,
                                                   float* __restrict__ vals) {
  const int64_t row = blockIdx.x;
  const float* x = logits + row * V;
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }

  for (int64_t e = threadIdx.x; e < V; e += 256) {
    float cv = x[e];
    int ci = (int)e;
    if (!better(cv, ci, lv[KMAX - 1], li[KMAX - 1])) continue;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool b = better(cv, ci, lv[j], li[j]);
      const float tv = lv[j];
      const int ti = li[j];
      lv[j] = b ? cv : tv;
      li[j] = b ? ci : ti;
      cv = b ? tv : cv;
      ci = b ? ti : ci;
    }
  }

  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int winner_i;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int r = 0; r < k; ++r) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float wv = sv[0];
      int wi = si[0];
      for (int w = 1; w < 4; ++w)
        if (better(sv[w], si[w], wv, wi)) { wv = sv[w]; wi = si[w]; }
      winner_i = wi;
      ids[row * k + r] = wi;
      vals[row * k + r] = wv;
    }
    __syncthreads();
    if (li[0] == winner_i) {  // ids are unique: exactly one thread pops its head
#pragma unroll
      for (int j = 0; j + 1 < KMAX; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
      lv[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = 0x7fffffff;
    }
  }
}

}  // namespace medusa

namespace medusa_host {
void launch_topk(const float* logits, int64_t R, int64_t V, int k, int* ids, float* vals,
                 hipStream_t st) {
  using namespace medusa;
  if (R <= 0) return;
  if (k <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, dim3((unsigned)R), dim3(256), 0, st, logits, V, k, ids, vals);
  else if (k <= 16)
    hipLaunchKernelGGL(topk_kernel<16>, dim3((unsigned)R), dim3(256), 0, st, logits, V, k, ids, vals);
  else
    hipLaunchKernelGGL(topk_kernel<64>, dim3((unsigned)R), dim3(256), 0, st, logits, V, k, ids, vals);
}
}  // namespace medusa_host

extern "C" int32_t medusa_topk(const float* logits, int64_t R, int64_t V, int32_t k, int32_t* ids,
                               float* vals, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(R >= 0 && V >= 1 && R <= INT32_MAX && V <= INT32_MAX, MEDUSA_ERR_INVALID_ARG,
                 "medusa_topk: bad sizes R=%lld V=%lld", (long long)R, (long long)V);
  MEDUSA_REQUIRE(k >= 1 && k <= MEDUSA_MAX_TOPK && k <= V, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_topk: k=%d outside [1, min(64, V)]", k);
  if (R == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && ids && vals, MEDUSA_ERR_INVALID_ARG, "medusa_topk: NULL pointer");
  launch_topk(logits, R, V, k, ids, vals, (hipStream_t)stream);
  return check_launch("medusa_topk");
}
