// Row-wise top-k of float logits ("Medusa Heads", section "Attenzione
// sull'albero e accettazione": the heads' best guesses feed the tree).
// Order: value descending, equal values by lower index.
//
// Two launches.  Stage 1, grid (chunks, rows): a workgroup takes a 4096-wide
// slice of a row, each thread 16 values read with 16-byte loads issued
// together.  For k <= 16 each wave then filters its 1024 values by a
// threshold T, the k-th largest of its 64 lane maxima: at least k values
// reach T, so no value below it can be among the k best, and on ordinary
// data only a few more than k do.  The survivors are packed into LDS by
// ballot and sorted across the wave by a bitonic network on 64-bit keys
// (order-preserving value bits, then the complemented index); lanes 0..k-1
// hold the wave's k best.  A wave whose survivors do not fit one per lane
// (long runs of equal values) takes the sorted per-lane lists and k rounds
// of a wave argmax instead.  Wave 0 sorts the four waves' lists the same
// way.  Stage 2 merges a row's chunk candidates, one wave per row: 64 at a
// time sorted, each batch folded into the running best by the bitonic
// merge step.  For k > 16 both stages keep a block-wide selection.  With one
// chunk, stage 1 writes the result.
#include "common.h"
#include "topk_wave.h"

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

// One wave's k best (k <= KMAX <= 16) of its lanes' 16 values each, written
// as keys to out[0..k-1].  v[j] is element e(j) = base + (g*256 + t)*4 + r for
// j = 4g + r; elements past V hold -inf and are never taken.
template <int KMAX>
__device__ __forceinline__ void wave_topk16(const float (&v)[TOPK_PER_THREAD], int64_t base,
                                            int64_t V, int k, float* __restrict__ stage_v,
                                            int* __restrict__ stage_i, uint64_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < TOPK_PER_THREAD; ++j) m = fmaxf(m, v[j]);
  const float sorted = wave_sort(m, lane, true);
  const float T = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sorted), k - 1));
  // survivors v >= T packed into the stage by ballot; count C is wave-uniform
  int C = 0;
#pragma unroll
  for (int j = 0; j < TOPK_PER_THREAD; ++j) {
    const int64_t e = base + (int64_t)((j / 4) * TOPK_THREADS + threadIdx.x) * 4 + (j % 4);
    const bool pred = e < V && v[j] >= T;
    const uint64_t bal = __ballot(pred);
    const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (pred && pos < 64) { stage_v[pos] = v[j]; stage_i[pos] = (int)e; }
    C += __popcll(bal);
  }
  if (C >= k && C <= 64) {
    __builtin_amdgcn_wave_barrier();
    uint64_t x = lane < C ? topk_key(stage_v[lane], stage_i[lane]) : TOPK_PAD_KEY;
    // sort only as many lanes as hold survivors
    if (C <= 16) x = wave_sort<16>(x, lane, true);
    else if (C <= 32) x = wave_sort<32>(x, lane, true);
    else x = wave_sort<64>(x, lane, true);
    if (lane < k) out[lane] = x;
    return;
  }
  // too many equal values at the threshold (or fewer than k real ones):
  // sorted per-lane lists, then k rounds of the wave argmax
  float lv[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
#pragma unroll
  for (int j = 0; j < TOPK_PER_THREAD; ++j) {
    const int64_t e = base + (int64_t)((j / 4) * TOPK_THREADS + threadIdx.x) * 4 + (j % 4);
    if (e < V) list_insert<KMAX>(lv, li, v[j], (int)e);
  }
  for (int r = 0; r < k; ++r) {
    float bv = lv[0];
    int bi = li[0];
    wave_argmax(bv, bi);
    if (lane == 0) out[r] = topk_key(bv, bi);
    if (li[0] == bi) {
#pragma unroll
      for (int j = 0; j + 1 < KMAX; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
      lv[KMAX - 1] = -INFINITY;
      li[KMAX - 1] = 0x7fffffff;
    }
  }
}

// k best of the threads' sorted lists (k > 16): k rounds of a block-wide
// argmax over the list heads; the owner pops (ids are unique).
template <int KMAX>
__device__ __forceinline__ void block_select(float (&lv)[KMAX], int (&li)[KMAX], int k,
                                             int* __restrict__ ids, float* __restrict__ vals) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

template <int KMAX>
__global__ __launch_bounds__(TOPK_THREADS) void topk_chunk_kernel(const float* __restrict__ logits,
                                                                  int64_t V, int k,
                                                                  int* __restrict__ ids,
                                                                  float* __restrict__ vals,
                                                                  int out_stride) {
  const int s = blockIdx.x;
  const int64_t row = blockIdx.y;
  const float* x = logits + row * V;
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
  const int64_t o = (row * gridDim.x + s) * (int64_t)out_stride;
  if constexpr (KMAX <= 16) {
    constexpr int NW = TOPK_THREADS / 64;
    __shared__ float stage_v[NW][64];
    __shared__ int stage_i[NW][64];
    __shared__ uint64_t best[NW][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wave_topk16<KMAX>(v, base, V, k, stage_v[wave], stage_i[wave], best[wave]);
    __syncthreads();
    if (wave != 0) return;
    // four descending runs of 16 (padded past k); odd runs read reversed, so
    // lanes 0-31 and 32-63 are bitonic: two merge levels sort the wave
    static_assert(NW == 4, "four runs of 16 fill the wave");
    const int run = lane / 16, r = (run & 1) ? 15 - lane % 16 : lane % 16;
    uint64_t key = r < k ? best[run][r] : TOPK_PAD_KEY;
    key = bitonic_pass<32, 16>(key, lane, true);
    key = bitonic_pass<64, 32>(key, lane, true);
    if (lane < k) {
      ids[o + lane] = key_index(key);
      vals[o + lane] = key_value(key);
    }
  } else {
    float lv[KMAX];
    int li[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
#pragma unroll
    for (int g = 0; g < TOPK_PER_THREAD / 4; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t e = base + (int64_t)(g * TOPK_THREADS + threadIdx.x) * 4 + r;
        if (e < V) list_insert<KMAX>(lv, li, v[g * 4 + r], (int)e);
      }
    block_select<KMAX>(lv, li, k, ids + o, vals + o);
  }
}

// Stage 2 for k <= 16: one wave per row merges the row's chunk lists.
__global__ __launch_bounds__(TOPK_THREADS) void topk_merge_wave_kernel(
    const int* __restrict__ cids, const float* __restrict__ cvals, int64_t R, int ncand, int k,
    int* __restrict__ ids, float* __restrict__ vals) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (TOPK_THREADS / 64) + (threadIdx.x >> 6);
  if (row >= R) return;
  const uint64_t top = merge_lists_wave(cids + row * ncand, cvals + row * ncand, ncand);
  if (lane < k) {
    ids[row * k + lane] = key_index(top);
    vals[row * k + lane] = key_value(top);
  }
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
  // sizes the entry points reject need nothing (and keep the products below in range)
  if (R <= 0 || k <= 0 || k > MEDUSA_MAX_TOPK || V <= 0 || R > INT32_MAX || V > INT32_MAX) return 0;
  const int S = topk_chunks(V);
  if (S <= 1) return 0;
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
    if (S > 1 && KM <= 16)                                                                    \
      hipLaunchKernelGGL(topk_merge_wave_kernel, dim3((unsigned)((R + 3) / 4)), blk, 0, st,   \
                         cid, cval, R, S * k, k, ids, vals);                                  \
    else if (S > 1)                                                                           \
      hipLaunchKernelGGL(topk_merge_kernel<64>, dim3((unsigned)R), blk, 0, st, cid, cval,     \
                         S * k, k, ids, vals);                                                \
  } while (0)
  if (k <= 4) MEDUSA_TOPK(4);
  else if (k <= 10) MEDUSA_TOPK(10);
  else if (k <= 16) MEDUSA_TOPK(16);
  else MEDUSA_TOPK(64);
#undef MEDUSA_TOPK
}
// Stage 1 only: each row's per-chunk lists straight into ids/vals [R][S][k]
// (with one chunk, the row's top-k).
void launch_topk_lists(const float* logits, int64_t R, int64_t V, int k, int* ids, float* vals,
                       hipStream_t st) {
  using namespace medusa;
  if (R <= 0) return;
  const dim3 g1((unsigned)topk_chunks(V), (unsigned)R), blk(TOPK_THREADS);
  if (k <= 4) hipLaunchKernelGGL(topk_chunk_kernel<4>, g1, blk, 0, st, logits, V, k, ids, vals, k);
  else if (k <= 10) hipLaunchKernelGGL(topk_chunk_kernel<10>, g1, blk, 0, st, logits, V, k, ids, vals, k);
  else if (k <= 16) hipLaunchKernelGGL(topk_chunk_kernel<16>, g1, blk, 0, st, logits, V, k, ids, vals, k);
  else hipLaunchKernelGGL(topk_chunk_kernel<64>, g1, blk, 0, st, logits, V, k, ids, vals, k);
}
}  // namespace medusa_host

extern "C" int32_t medusa_topk_lists(int64_t V) {
  return V >= 1 && V <= INT32_MAX ? medusa_host::topk_chunks(V) : 0;
}

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
