// Wave-wide pieces of the top-k selection shared by the top-k kernels and
// the tree build that merges per-chunk candidate lists: order-preserving
// 64-bit sort keys for (value, index) pairs and a bitonic network over the
// 64 lanes of a wave.
#pragma once
#include "common.h"

namespace medusa {

// Sort keys: the float's bits made order-preserving as unsigned (-0 taken
// as +0, so signed zeros tie as they compare), then the index complemented,
// so a larger key is the better (value, index) pair.  NaN never becomes a
// key: it fails every comparison that admits a value.
__device__ __forceinline__ uint64_t topk_key(float v, int i) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
// The list padding (-inf, 0x7fffffff): below every real entry.
constexpr uint64_t TOPK_PAD_KEY = (uint64_t)0x007fffffu << 32 | 0x80000000u;

// Lane l's copy of lane l ^ J's register.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else return (uint32_t)__shfl_xor((int)v, J, 64);
}
template <int J>
__device__ __forceinline__ uint64_t lane_xor(uint64_t v) {
  return ((uint64_t)lane_xor<J>((uint32_t)(v >> 32)) << 32) | lane_xor<J>((uint32_t)v);
}
template <int J>
__device__ __forceinline__ float lane_xor(float v) {
  return __uint_as_float(lane_xor<J>(__float_as_uint(v)));
}

// Bitonic network over the 64 lanes of a wave (one key per lane).  Stage
// (KK, J) compares lanes l and l ^ J; the pair belongs to a block of KK lanes
// ordered descending when (l & KK) == 0 matches `desc`, and the lower lane
// of the pair keeps the larger key in a descending block.
template <int KK, int J, typename Key>
__device__ __forceinline__ Key bitonic_pass(Key x, int lane, bool desc) {
  const Key y = lane_xor<J>(x);
  const bool block_desc = ((lane & KK) == 0) == desc;
  const bool keep_larger = ((lane & J) == 0) == block_desc;
  x = ((x > y) == keep_larger) ? x : y;
  if constexpr (J > 1) return bitonic_pass<KK, J / 2>(x, lane, desc);
  else return x;
}
template <int KK, int WIDTH, typename Key>
__device__ __forceinline__ Key bitonic_sort_from(Key x, int lane, bool desc) {
  x = bitonic_pass<KK, KK / 2>(x, lane, desc);
  if constexpr (KK < WIDTH) return bitonic_sort_from<KK * 2, WIDTH>(x, lane, desc);
  else return x;
}
// Each block of WIDTH lanes sorted; lanes 0..WIDTH-1 in the order asked
// (lane 0 holds the largest when desc).  WIDTH = 64 sorts the whole wave.
template <int WIDTH = 64, typename Key>
__device__ __forceinline__ Key wave_sort(Key x, int lane, bool desc) {
  return bitonic_sort_from<2, WIDTH>(x, lane, desc);
}
// A bitonic sequence over the wave, sorted.
template <typename Key>
__device__ __forceinline__ Key wave_bitonic_merge(Key x, int lane, bool desc) {
  return bitonic_pass<64, 32>(x, lane, desc);
}

// The 64 best keys of a row's ncand candidates (ids ci, values cv; ncand
// >= 1), sorted descending over the lanes: taken 64 at a time, the first batch
// sorted descending, every later one sorted ascending and folded in by the
// lane-wise maximum (which leaves the 64 best of both as a bitonic sequence)
// and one bitonic merge.  Lanes past the candidates hold TOPK_PAD_KEY.
__device__ __forceinline__ uint64_t merge_lists_wave(const int* ci, const float* cv, int ncand) {
  const int lane = threadIdx.x & 63;
  int nid = lane < ncand ? ci[lane] : 0;
  float nv = lane < ncand ? cv[lane] : 0.f;
  uint64_t top = TOPK_PAD_KEY;
  for (int c0 = 0; c0 < ncand; c0 += 64) {
    uint64_t x = c0 + lane < ncand ? topk_key(nv, nid) : TOPK_PAD_KEY;
    const int c1 = c0 + 64 + lane;  // next batch in flight during this one's sort
    if (c1 < ncand) { nid = ci[c1]; nv = cv[c1]; }
    if (c0 == 0) {
      top = wave_sort(x, lane, true);
    } else {
      x = wave_sort(x, lane, false);
      top = top > x ? top : x;
      top = wave_bitonic_merge(top, lane, true);
    }
  }
  return top;
}

}  // namespace medusa
