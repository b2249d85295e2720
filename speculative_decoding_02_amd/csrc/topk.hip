// Row-wise top-k of float logits ("Medusa Heads", section "Attenzione
// sull'albero e accettazione": the heads' best guesses feed the tree).
// Order: value descending, equal values by lower index.
//
// Two launches.  Stage 1, grid (chunks, rows): a workgroup takes a 4096-wide
// slice of a row; each thread reads its 16 values with 16-byte loads issued
// together (no load waits on a comparison), keeps a sorted register list,
// and the workgroup merges the lists by k rounds of a block-wide selection
// into k candidates.  Stage 2, one workgroup per row: the same selection over
// the chunks' candidates.  With one chunk, stage 1 writes the result.
#include "common.h"

namespace medusa {

constexpr int TOPK_THREADS = 256;
constexpr int TOPK_PER_THREAD = 16;
constexpr int TOPK_CHUNK = TOPK_THREADS * TOPK_PER_THREAD;  // 4096

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int KMAX>
__device__ __forceinline__ void list_insert(float (&lv)[KMAX], int (&li)[KMAX], float cv, int ci) {
  if (!better(cv, ci, lv[KMAX - 1], li[KMAX - 1])) return;
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

// Best (value, index) over a wave without LDS traffic: quad permutes (xor 1,
// xor 2), the 8- and 16-lane mirrors, then gfx950's 16- and 32-row swaps.
// The selection is a total order (ties: lower index), so every lane ends with
// the same winner.
__device__ __forceinline__ void pick(float& bv, int& bi, float ov, int oi) {
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}
template <int CTRL>
__device__ __forceinline__ void dpp_pick(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(bi, CTRL, 0xF, 0xF, false);
  pick(bv, bi, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  dpp_pick<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
  dpp_pick<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
  dpp_pick<0x141>(bv, bi);  // row_half_mirror: lane i <-> 7-i
  dpp_pick<0x140>(bv, bi);  // row_mirror: lane i <-> 15-i
  {
    const auto sv = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto si = __builtin_amdgcn_permlane16_swap((unsigned)bi, (unsigned)bi, false, false);
    bv = __uint_as_float(sv[0]); bi = (int)si[0];
    pick(bv, bi, __uint_as_float(sv[1]), (int)si[1]);
  }
  {
    const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
    const auto si = __builtin_amdgcn_permlane32_swap((unsigned)bi, (unsigned)bi, false, false);
    bv = __uint_as_float(sv[0]); bi = (int)si[0];
    pick(bv, bi, __uint_as_float(sv[1]), (int)si[1]);
  }
}

// k best of the threads' sorted lists.  k <= 16: every wave emits its own k
// best (k rounds of a wave argmax over the list heads; the owner pops, ids
// being unique), the four lists meet in LDS, and wave 0 selects k of those
// 4k (one candidate per lane).  k > 16: k rounds of a block-wide argmax.
template <int KMAX>
__device__ __forceinline__ void block_select(float (&lv)[KMAX], int (&li)[KMAX], int k,
                                             int* __restrict__ ids, float* __restrict__ vals) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if constexpr (KMAX <= 16) {
    __shared__ float cv[TOPK_THREADS / 64][KMAX];
    __shared__ int ci[TOPK_THREADS / 64][KMAX];
    for (int r = 0; r < k; ++r) {
      float bv = lv[0];
      int bi = li[0];
      wave_argmax(bv, bi);
      if (lane == 0) { cv[wave][r] = bv; ci[wave][r] = bi; }
      if (li[0] == bi) {
#pragma unroll
        for (int j = 0; j + 1 < KMAX; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
        lv[KMAX - 1] = -INFINITY;
        li[KMAX - 1] = 0x7fffffff;
      }
    }
    __syncthreads();
    if (wave != 0) return;
    static_assert(TOPK_THREADS / 64 * KMAX <= 64, "one candidate per lane");
    const int w = lane / KMAX, j = lane % KMAX;
    float v = -INFINITY;
    int i = 0x7fffffff;
    if (w < TOPK_THREADS / 64 && j < k) { v = cv[w][j]; i = ci[w][j]; }
    for (int r = 0; r < k; ++r) {
      float bv = v;
      int bi = i;
      wave_argmax(bv, bi);
      if (lane == 0) { ids[r] = bi; vals[r] = bv; }
      if (i == bi) { v = -INFINITY; i = 0x7fffffff; }
    }
  } else {
    __shared__ float sv[TOPK_THREADS / 64];
    __shared__ int si[TOPK_THREADS / 64];
    __shared__ int winner_i;
    for (int r = 0; r < k; ++r) {
      float bv = lv[0];
      int bi = li[0];
      wave_argmax(bv, bi);
      if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
      __syncthreads();
      if (threadIdx.x == 0) {
        float wv = sv[0];
        int wi = si[0];
        for (int w = 1; w < TOPK_THREADS / 64; ++w)
          if (better(sv[w], si[w], wv, wi)) { wv = sv[w]; wi = si[w]; }
        winner_i = wi;
        ids[r] = wi;
        vals[r] = wv;
      }
      __syncthreads();
      if (li[0] == winner_i) {
#pragma unroll
        for (int j = 0; j + 1 < KMAX; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
        lv[KMAX - 1] = -INFINITY;
        li[KMAX - 1] = 0x7fffffff;
      }
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(TOPK_THREADS) void topk_chunk_kernel(const float* __restrict__ logits,
                                                                  int64_t V, int k,
                                                                  int* __restrict__ ids,
                                                                  float* __restrict__ vals,
                                                                  int out_stride) {
  const int s = blockIdx.x;
  const int64_t row = blockIdx.y;
  const float* x = logits + row * V;
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  const int64_t base = (int64_t)s * TOPK_CHUNK;
  // 16 values per thread: four 16-byte groups, strided by the block width
  float v[TOPK_PER_THREAD];
  const bool vec = (V % 4 == 0) && (((uintptr_t)x) % 16 == 0);
#pragma unroll
  for (int g = 0; g < TOPK_PER_THREAD / 4; ++g) {
    const int64_t e0 = base + (int64_t)(g * TOPK_THREADS + threadIdx.x) * 4;
    if (vec && e0 + 3 < V) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(x + e0);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[g * 4 + r] = q[r];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[g * 4 + r] = (e0 + r < V) ? x[e0 + r] : -INFINITY;
    }
  }
#pragma unroll
  for (int g = 0; g < TOPK_PER_THREAD / 4; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t e = base + (int64_t)(g * TOPK_THREADS + threadIdx.x) * 4 + r;
      if (e < V) list_insert<KMAX>(lv, li, v[g * 4 + r], (int)e);
    }
  const int64_t o = (row * gridDim.x + s) * (int64_t)out_stride;
  block_select<KMAX>(lv, li, k, ids + o, vals + o);
}

template <int KMAX>
__global__ __launch_bounds__(TOPK_THREADS) void topk_merge_kernel(const int* __restrict__ cids,
                                                                  const float* __restrict__ cvals,
                                                                  int ncand, int k,
                                                                  int* __restrict__ ids,
                                                                  float* __restrict__ vals) {
  const int64_t row = blockIdx.x;
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  for (int c = threadIdx.x; c < ncand; c += TOPK_THREADS)
    list_insert<KMAX>(lv, li, cvals[row * ncand + c], cids[row * ncand + c]);
  block_select<KMAX>(lv, li, k, ids + row * k, vals + row * k);
}

}  // namespace medusa

namespace medusa_host {
static int topk_chunks(int64_t V) { return (int)((V + medusa::TOPK_CHUNK - 1) / medusa::TOPK_CHUNK); }

size_t topk_ws_bytes(int64_t R, int64_t V, int k) {
  const int S = topk_chunks(V);
  if (S <= 1 || R <= 0 || k <= 0) return 0;
  return align_up((size_t)R * S * k * sizeof(int), 256) + align_up((size_t)R * S * k * sizeof(float), 256);
}

void launch_topk(const float* logits, int64_t R, int64_t V, int k, int* ids, float* vals, void* ws,
                 hipStream_t st) {
  using namespace medusa;
  if (R <= 0) return;
  const int S = topk_chunks(V);
  int* cid = ids;
  float* cval = vals;
  if (S > 1) {
    cid = (int*)ws;
    cval = (float*)((char*)ws + align_up((size_t)R * S * k * sizeof(int), 256));
  }
  const dim3 g1((unsigned)S, (unsigned)R), blk(TOPK_THREADS);
#define MEDUSA_TOPK(KM)                                                                       \
  do {                                                                                        \
    hipLaunchKernelGGL(topk_chunk_kernel<KM>, g1, blk, 0, st, logits, V, k, cid, cval, k);    \
    if (S > 1)                                                                                \
      hipLaunchKernelGGL(topk_merge_kernel<KM>, dim3((unsigned)R), blk, 0, st, cid, cval,     \
                         S * k, k, ids, vals);                                                \
  } while (0)
  if (k <= 4) MEDUSA_TOPK(4);
  else if (k <= 10) MEDUSA_TOPK(10);
  else if (k <= 16) MEDUSA_TOPK(16);
  else MEDUSA_TOPK(64);
#undef MEDUSA_TOPK
}
}  // namespace medusa_host

extern "C" size_t medusa_topk_ws(int64_t R, int64_t V, int32_t k) {
  return medusa_host::topk_ws_bytes(R, V, k);
}

extern "C" int32_t medusa_topk(const float* logits, int64_t R, int64_t V, int32_t k, int32_t* ids,
                               float* vals, void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(R >= 0 && V >= 1 && R <= INT32_MAX && V <= INT32_MAX, MEDUSA_ERR_INVALID_ARG,
                 "medusa_topk: bad sizes R=%lld V=%lld", (long long)R, (long long)V);
  MEDUSA_REQUIRE(k >= 1 && k <= MEDUSA_MAX_TOPK && k <= V, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_topk: k=%d outside [1, min(64, V)]", k);
  if (R == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && ids && vals, MEDUSA_ERR_INVALID_ARG, "medusa_topk: NULL pointer");
  const size_t need = topk_ws_bytes(R, V, k);
  MEDUSA_REQUIRE(need == 0 || (ws != NULL && ws_bytes >= need), MEDUSA_ERR_WORKSPACE,
                 "medusa_topk: workspace %zu < %zu bytes", ws_bytes, need);
  launch_topk(logits, R, V, k, ids, vals, ws, (hipStream_t)stream);
  return check_launch("medusa_topk");
}
