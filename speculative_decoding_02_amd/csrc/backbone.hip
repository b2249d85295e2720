// Element-wise and row-wise pieces of the Llama-style verification forward
// pass (the base model checks every tree node in one pass: "Têtes de décodage
// Medusa", section "Plongée profonde").  The projections themselves run in
// gemm.hip.  The residual stream is fp32; GEMM inputs are in the model dtype.
#include "common.h"

namespace medusa {

// One workgroup per row.  Rows of whole 4-element vectors (H a multiple of 4,
// aligned table and output) are copied with every thread's loads issued
// before its stores; other rows element by element.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int* __restrict__ tokens,
                                                    const T* __restrict__ table, int64_t H,
                                                    float* __restrict__ out, int vec) {
  const int64_t m = blockIdx.x;
  const T* row = table + (int64_t)tokens[m] * H;
  if (vec) {
    const int64_t H4 = H / 4;
    for (int64_t e0 = threadIdx.x; e0 < H4; e0 += 256 * RMS_V4) {
      f32x4 v[RMS_V4];
#pragma unroll
      for (int i = 0; i < RMS_V4; ++i) {
        const int64_t e = e0 + i * 256;
        v[i] = Elem<T>::load4(row, e < H4 ? e : 0);
      }
#pragma unroll
      for (int i = 0; i < RMS_V4; ++i)
        if (e0 + i * 256 < H4) Elem<float>::store4(out + m * H, e0 + i * 256, v[i]);
    }
    return;
  }
  for (int64_t e = threadIdx.x; e < H; e += 256) out[m * H + e] = ld<T>(row, e);
}

// One workgroup per row.  Every thread issues all of its 16-byte loads before
// using any (up to RMS_V4 per thread, enough for H = 8192 in fp32), so a row
// costs one memory round trip; the sum of squares is reduced in a fixed order
// (per-thread, then a butterfly per wave, then the 4 waves in order) and the
// normalised values are written from registers.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int64_t M,
                                                      int64_t H, const T* __restrict__ gain,
                                                      float eps, T* __restrict__ out) {
  const int64_t m = blockIdx.x;
  const float* xr = x + m * H;
  const int64_t H4 = H / 4;
  f32x4 g[RMS_V4], v[RMS_V4];
  rms_row_gain<T>(gain, H, g);
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    const int64_t e = threadIdx.x + (int64_t)i * 256;
    v[i] = reinterpret_cast<const f32x4*>(xr)[e < H4 ? e : 0];
  }
  const float rs = rms_row_scale(v, H, eps);
  rms_row_store<T>(v, H, rs, g, out + m * H);
}

// Rotary positions, rotate-half pairs (j, j + D/2), angle pos * base^(-2j/D)
// (rope_inv_freq / rope_cs / rope_rot); one pass per row over 4 consecutive j
// per thread.  PAIRS: the q and k heads of qkv hold each pair side by side
// (columns 2j, 2j+1 of a head = elements j, j + D/2), the layout of a
// projection whose weight rows were interleaved that way.
template <typename T, bool PAIRS>
__global__ __launch_bounds__(256) void qkv_rope_kernel(const T* __restrict__ qkv, int Hq, int Hkv,
                                                       int D, const int* __restrict__ pos,
                                                       double log2_base, T* __restrict__ q,
                                                       T* __restrict__ k, T* __restrict__ v) {
  const int64_t m = blockIdx.x;
  __shared__ float cs[64], sn[64];
  const int half = D / 2;
  if (threadIdx.x < half) {
    float c, sv;
    rope_cs(pos[m], rope_inv_freq(threadIdx.x, D, log2_base), c, sv);
    cs[threadIdx.x] = c;
    sn[threadIdx.x] = sv;
  }
  __syncthreads();
  const int W = (Hq + 2 * Hkv) * D;
  const T* in = qkv + m * W;
  const int quads = (Hq + Hkv) * (half / 4);   // 4 consecutive j per item
  // each item: four pairs j0 .. j0+3 read and written with vector accesses
  // (every offset is a multiple of four elements: D % 8 == 0)
  for (int e = threadIdx.x; e < quads; e += 256) {
    const int hh = e / (half / 4), j0 = (e % (half / 4)) * 4;
    T* dst = hh < Hq ? q + (m * Hq + hh) * D : k + (m * Hkv + (hh - Hq)) * D;
    float x1[4], x2[4];
    if (PAIRS) {  // elements (j, j + D/2) side by side: 8 consecutive values
      const int64_t i4 = ((int64_t)hh * D + 2 * j0) / 4;
      const f32x4 a = Elem<T>::load4(in, i4), b = Elem<T>::load4(in, i4 + 1);
      x1[0] = a.x; x2[0] = a.y; x1[1] = a.z; x2[1] = a.w;
      x1[2] = b.x; x2[2] = b.y; x1[3] = b.z; x2[3] = b.w;
    } else {
      const f32x4 a = Elem<T>::load4(in, ((int64_t)hh * D + j0) / 4);
      const f32x4 b = Elem<T>::load4(in, ((int64_t)hh * D + j0 + half) / 4);
      x1[0] = a.x; x1[1] = a.y; x1[2] = a.z; x1[3] = a.w;
      x2[0] = b.x; x2[1] = b.y; x2[2] = b.z; x2[3] = b.w;
    }
    float y1[4], y2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rope_rot(x1[r], x2[r], cs[j0 + r], sn[j0 + r], y1[r], y2[r]);
    Elem<T>::store4(dst, j0 / 4, f32x4{y1[0], y1[1], y1[2], y1[3]});
    Elem<T>::store4(dst, (j0 + half) / 4, f32x4{y2[0], y2[1], y2[2], y2[3]});
  }
  // v: straight copy in 16-byte pieces
  const int vb = Hkv * D * (int)sizeof(T) / 16;
  const u32x4* vin = reinterpret_cast<const u32x4*>(in + (int64_t)(Hq + Hkv) * D);
  u32x4* vout = reinterpret_cast<u32x4*>(v + m * Hkv * D);
  for (int e = threadIdx.x; e < vb; e += 256) vout[e] = vin[e];
}

template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const T* __restrict__ gu, int64_t F,
                                                     T* __restrict__ out) {
  const int64_t m = blockIdx.x;
  for (int64_t e = threadIdx.x; e < F; e += 256) {
    const float g = ld<T>(gu, m * 2 * F + e), u = ld<T>(gu, m * 2 * F + F + e);
    st<T>(out, m * F + e, silu_f(g) * u);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ h, int N, int64_t H,
                                                          const int* __restrict__ path,
                                                          const int* __restrict__ accept_len,
                                                          int K, T* __restrict__ out) {
  const int b = blockIdx.x;
  const int a = min(accept_len[b], K);
  const int node = path[(int64_t)b * (K + 1) + a];
  const T* src = h + ((int64_t)b * N + node) * H;
  for (int64_t e = threadIdx.x; e < H; e += 256) out[(int64_t)b * H + e] = src[e];
}

}  // namespace medusa

#define MEDUSA_DT_DISPATCH(dt, ...)                 \
  do {                                              \
    if ((dt) == MEDUSA_BF16) {                      \
      using T = medusa::bf16_t;                     \
      __VA_ARGS__;                                  \
    } else {                                        \
      using T = float;                              \
      __VA_ARGS__;                                  \
    }                                               \
  } while (0)

extern "C" int32_t medusa_embed(const int32_t* tokens, int64_t M, const void* table, int64_t V,
                                int64_t H, int32_t dt, float* out, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "medusa_embed: dtype");
  MEDUSA_REQUIRE(M >= 0 && V >= 1 && H >= 1 && M <= INT32_MAX, MEDUSA_ERR_INVALID_ARG,
                 "medusa_embed: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(tokens && table && out, MEDUSA_ERR_INVALID_ARG, "medusa_embed: NULL pointer");
  const int vec = H % 4 == 0 && ((uintptr_t)out) % 16 == 0 &&
                  ((uintptr_t)table) % (dt == MEDUSA_BF16 ? 8 : 16) == 0;
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL(medusa::embed_kernel<T>, dim3((unsigned)M), dim3(256), 0,
                                            (hipStream_t)stream, tokens, (const T*)table, H, out, vec));
  return check_launch("medusa_embed");
}

extern "C" int32_t medusa_rmsnorm(const float* x, int64_t M, int64_t H, const void* gain, float eps,
                                  int32_t dt, void* out, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "medusa_rmsnorm: dtype");
  MEDUSA_REQUIRE(M >= 0 && H >= 1 && M <= INT32_MAX && eps >= 0.f, MEDUSA_ERR_INVALID_ARG,
                 "medusa_rmsnorm: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(x && out, MEDUSA_ERR_INVALID_ARG, "medusa_rmsnorm: NULL pointer");
  MEDUSA_REQUIRE(((uintptr_t)x) % 16 == 0 && H % 4 == 0 && H <= 4 * 256 * medusa::RMS_V4,
                 MEDUSA_ERR_UNSUPPORTED,
                 "medusa_rmsnorm: needs 16-byte aligned x, H a multiple of 4 and H <= %d",
                 4 * 256 * medusa::RMS_V4);
  const int a4 = dt == MEDUSA_BF16 ? 8 : 16;  // four elements of gain and out
  MEDUSA_REQUIRE(((uintptr_t)gain | (uintptr_t)out) % a4 == 0, MEDUSA_ERR_INVALID_ARG,
                 "medusa_rmsnorm: gain and out must be %d-byte aligned", a4);
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL(medusa::rmsnorm_kernel<T>, dim3((unsigned)M), dim3(256),
                                            0, (hipStream_t)stream, x, M, H, (const T*)gain, eps,
                                            (T*)out));
  return check_launch("medusa_rmsnorm");
}

extern "C" int32_t medusa_qkv_rope(const void* qkv, int64_t M, int32_t Hq, int32_t Hkv, int32_t D,
                                   const int32_t* pos, float base, int32_t dt, void* q, void* k,
                                   void* v, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "medusa_qkv_rope: dtype");
  MEDUSA_REQUIRE(D >= 8 && D <= 128 && D % 8 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_qkv_rope: head dim %d (multiple of 8 up to 128)", D);
  MEDUSA_REQUIRE(((uintptr_t)qkv | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) % 16 == 0,
                 MEDUSA_ERR_INVALID_ARG, "medusa_qkv_rope: qkv, q, k and v must be 16-byte aligned");
  MEDUSA_REQUIRE(M >= 0 && M <= INT32_MAX && Hq >= 1 && Hkv >= 1 && base > 1.f,
                 MEDUSA_ERR_INVALID_ARG, "medusa_qkv_rope: bad sizes or base");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(qkv && pos && q && k && v, MEDUSA_ERR_INVALID_ARG, "medusa_qkv_rope: NULL pointer");
  const double lb = log2((double)base);
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL((medusa::qkv_rope_kernel<T, false>), dim3((unsigned)M), dim3(256), 0,
                                            (hipStream_t)stream, (const T*)qkv, Hq, Hkv, D, pos, lb,
                                            (T*)q, (T*)k, (T*)v));
  return check_launch("medusa_qkv_rope");
}

extern "C" int32_t medusa_swiglu(const void* gu, int64_t M, int64_t F, int32_t dt, void* out,
                                 void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "medusa_swiglu: dtype");
  MEDUSA_REQUIRE(M >= 0 && M <= INT32_MAX && F >= 1, MEDUSA_ERR_INVALID_ARG, "medusa_swiglu: bad sizes");
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(gu && out, MEDUSA_ERR_INVALID_ARG, "medusa_swiglu: NULL pointer");
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL(medusa::swiglu_kernel<T>, dim3((unsigned)M), dim3(256), 0,
                                            (hipStream_t)stream, (const T*)gu, F, (T*)out));
  return check_launch("medusa_swiglu");
}

extern "C" int32_t medusa_gather_rows(const void* h, int32_t B, int32_t N, int64_t H,
                                      const int32_t* path, const int32_t* accept_len, int32_t K,
                                      int32_t dt, void* out, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "medusa_gather_rows: dtype");
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES && H >= 1 && K >= 0 &&
                     K <= MEDUSA_MAX_NODES - 1,
                 MEDUSA_ERR_INVALID_ARG, "medusa_gather_rows: bad sizes");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(h && path && accept_len && out, MEDUSA_ERR_INVALID_ARG,
                 "medusa_gather_rows: NULL pointer");
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL(medusa::gather_rows_kernel<T>, dim3(B), dim3(256), 0,
                                            (hipStream_t)stream, (const T*)h, N, H, path, accept_len,
                                            K, (T*)out));
  return check_launch("medusa_gather_rows");
}

namespace medusa_host {
// Rotary kernel on a pair-interleaved qkv (arguments validated by the caller).
void launch_qkv_rope_pairs(const void* qkv, int64_t M, int Hq, int Hkv, int D, const int32_t* pos,
                           double log2_base, int dt, void* q, void* k, void* v, hipStream_t st) {
  MEDUSA_DT_DISPATCH(dt, hipLaunchKernelGGL((medusa::qkv_rope_kernel<T, true>), dim3((unsigned)M), dim3(256),
                                            0, st, (const T*)qkv, Hq, Hkv, D, pos, log2_base, (T*)q,
                                            (T*)k, (T*)v));
}
}  // namespace medusa_host
