// kv_compact: keep only the accepted branch in the KV cache ("Medusa Heads",
// section "Attenzione sull'albero e accettazione": the longest accepted branch
// is kept).  Slot ctx+d receives slot ctx+path[d] for d = 0..accept_len, for
// K and V of every layer and kv head.
//
// One workgroup per (kv head, layer, sequence).  A source slot ctx+path[d] may
// be another row's destination (path (0, 2, 3) moves 12 -> 11 and 13 -> 12),
// so the workgroup first reads every source row into LDS, then writes them:
// read-all / barrier / write-all.
#include "common.h"

namespace medusa {

template <int D, int ES>
__global__ __launch_bounds__(256) void kv_compact_kernel(LayerPtrs lp, int Hkv, int P,
                                                         const int* __restrict__ page_table,
                                                         int max_pages,
                                                         const int* __restrict__ ctx,
                                                         const int* __restrict__ path,
                                                         const int* __restrict__ accept_len,
                                                         int K, int* __restrict__ src_slots,
                                                         int* __restrict__ dst_slots,
                                                         int* __restrict__ new_ctx) {
  constexpr int CPR = D * ES / 16;  // 16-byte chunks per row
  __shared__ uint4 buf[2 * (MEDUSA_MAX_HEADS + 1) * CPR];
  const int kvh = blockIdx.x, l = blockIdx.y, b = blockIdx.z;
  const int c = ctx[b];
  const int a = min(accept_len[b], K);
  const int* pth = path + (int64_t)b * (K + 1);
  const int* pt = page_table + (int64_t)b * max_pages;
  auto row_ptr = [&](char* pool, int slot) -> uint4* {
    const int page = pt[slot / P];
    return reinterpret_cast<uint4*>(pool + ((((int64_t)page * Hkv + kvh) * P + slot % P) * D) * ES);
  };
  char* pools[2] = {(char*)lp.k[l], (char*)lp.v[l]};
  const int rows = a + 1;
  const int items = 2 * rows * CPR;
  for (int e = threadIdx.x; e < items; e += 256) {
    const int which = e / (rows * CPR), rem = e % (rows * CPR), d = rem / CPR, ch = rem % CPR;
    buf[e] = row_ptr(pools[which], c + pth[d])[ch];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < items; e += 256) {
    const int which = e / (rows * CPR), rem = e % (rows * CPR), d = rem / CPR, ch = rem % CPR;
    if (pth[d] != d) row_ptr(pools[which], c + d)[ch] = buf[e];
  }
  if (kvh == 0 && l == 0 && threadIdx.x <= K) {
    const int d = threadIdx.x;
    if (src_slots) src_slots[(int64_t)b * (K + 1) + d] = d <= a ? c + pth[d] : -1;
    if (dst_slots) dst_slots[(int64_t)b * (K + 1) + d] = d <= a ? c + d : -1;
    if (d == 0) new_ctx[b] = c + a + 1;
  }
}

}  // namespace medusa

extern "C" int32_t kv_compact(void* const* Kc, void* const* Vc, int32_t L,
                              const int32_t* page_table, int32_t max_pages, int32_t P,
                              const int32_t* ctx, const int32_t* path, const int32_t* accept_len,
                              int32_t B, int32_t K, int32_t Hkv, int32_t D, int32_t dt,
                              int32_t* src_slots, int32_t* dst_slots, int32_t* new_ctx,
                              void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "kv_compact: unknown dtype %d", dt);
  MEDUSA_REQUIRE(D == 64 || D == 128, MEDUSA_ERR_UNSUPPORTED, "kv_compact: head dim %d", D);
  MEDUSA_REQUIRE(L >= 1 && L <= MEDUSA_MAX_LAYERS, MEDUSA_ERR_UNSUPPORTED,
                 "kv_compact: L=%d outside [1, %d]", L, MEDUSA_MAX_LAYERS);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_HEADS, MEDUSA_ERR_UNSUPPORTED,
                 "kv_compact: K=%d outside [0, %d]", K, MEDUSA_MAX_HEADS);
  MEDUSA_REQUIRE(B >= 0 && Hkv >= 1 && P >= 1 && max_pages >= 1, MEDUSA_ERR_INVALID_ARG,
                 "kv_compact: B=%d Hkv=%d P=%d max_pages=%d", B, Hkv, P, max_pages);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(Kc && Vc && page_table && ctx && path && accept_len && new_ctx,
                 MEDUSA_ERR_INVALID_ARG, "kv_compact: NULL pointer");
  MEDUSA_REQUIRE(new_ctx != ctx, MEDUSA_ERR_INVALID_ARG, "kv_compact: new_ctx must not alias ctx");
  medusa::LayerPtrs lp;
  for (int l = 0; l < L; ++l) {
    MEDUSA_REQUIRE(Kc[l] && Vc[l], MEDUSA_ERR_INVALID_ARG, "kv_compact: NULL pool for layer %d", l);
    MEDUSA_REQUIRE(((uintptr_t)Kc[l] | (uintptr_t)Vc[l]) % 16 == 0, MEDUSA_ERR_INVALID_ARG,
                   "kv_compact: pools must be 16-byte aligned");
    lp.k[l] = Kc[l];
    lp.v[l] = Vc[l];
  }
  dim3 grid(Hkv, L, B);
  hipStream_t st = (hipStream_t)stream;
#define MEDUSA_KVC(DD, ES)                                                                   \
  hipLaunchKernelGGL((medusa::kv_compact_kernel<DD, ES>), grid, dim3(256), 0, st, lp, Hkv, P, \
                     page_table, max_pages, ctx, path, accept_len, K, src_slots, dst_slots,  \
                     new_ctx)
  if (dt == MEDUSA_BF16) { if (D == 128) MEDUSA_KVC(128, 2); else MEDUSA_KVC(64, 2); }
  else { if (D == 128) MEDUSA_KVC(128, 4); else MEDUSA_KVC(64, 4); }
#undef MEDUSA_KVC
  return check_launch("kv_compact");
}
