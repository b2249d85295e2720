// Internal helpers shared by the HIP kernels of libmedusa (CDNA4 / gfx950).
//
// Storage types: MEDUSA_F32 tensors are `float`, MEDUSA_BF16 tensors are raw
// bfloat16 bit patterns (`uint16_t`).  All arithmetic is fp32; bf16 values are
// widened exactly and narrowed round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/medusa.h"

namespace medusa {

typedef uint16_t bf16_t;

// Native clang vectors for register data: selects and element access stay in
// VGPRs (HIP's uint4/float4 are structs, and a select on them goes through
// scratch memory).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Pack two fp32 values into one dword of two bf16 (lo = a, hi = b), RNE, with
// gfx950's packed conversion (the same rounding as f2bf for every non-NaN).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
  // elements 4*i4 .. 4*i4+3 (16-byte aligned)
  static __device__ __forceinline__ f32x4 load4(const float* p, size_t i4) {
    return reinterpret_cast<const f32x4*>(p)[i4];
  }
  static __device__ __forceinline__ void store4(float* p, size_t i4, f32x4 v) {
    reinterpret_cast<f32x4*>(p)[i4] = v;
  }
  static constexpr int per16 = 4;  // elements per 16-byte vector
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, size_t i, float v) { p[i] = f2bf(v); }
  // elements 4*i4 .. 4*i4+3 (8-byte aligned)
  static __device__ __forceinline__ f32x4 load4(const bf16_t* p, size_t i4) {
    const u32x2 u = reinterpret_cast<const u32x2*>(p)[i4];
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
  }
  static __device__ __forceinline__ void store4(bf16_t* p, size_t i4, f32x4 v) {
    reinterpret_cast<u32x2*>(p)[i4] = u32x2{pack_bf2(v.x, v.y), pack_bf2(v.z, v.w)};
  }
  static constexpr int per16 = 8;
};

template <typename T> __device__ __forceinline__ float ld(const T* p, size_t i) { return Elem<T>::load(p, i); }
template <typename T> __device__ __forceinline__ void st(T* p, size_t i, float v) { Elem<T>::store(p, i, v); }

// ---------------------------------------------------------------------------
// MFMA wrappers.  Layout of a 16x16 fp32 result (both wrappers): lane l holds
// column (l % 16) and rows 4*(l/16) + r in element r.  For the operands, lane
// l supplies row (l % 16) of A and column (l % 16) of B; the lanes with the
// same l/16 supply the same contraction indices for A and B.
// ---------------------------------------------------------------------------

// bf16: one 16-byte vector per lane = 8 contraction elements (16x16x32).
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// bf16: 4 contraction elements per lane (16x16x16); lane l's elements are
// contraction indices 4*(l/16)+r.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// bf16, 32x32x16 (twice the issue rate of the 16x16 shapes on gfx950): lane
// l supplies row l%32 of A and column l%32 of B with contraction indices
// 8(l/32) .. +7; element e of the result holds row 8(e/4) + 4(l/32) + e%4,
// column l%32.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// fp32: one contraction element per lane (16x16x4), index l/16.
__device__ __forceinline__ f32x4 mfma_f32_16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Wavefront-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over the four lanes {l, l^16, l^32, l^48} (the 16-lane rows of a
// wave that hold the same MFMA output column), with gfx950's row-swap
// permutes instead of LDS round trips: after a 16-row swap of x with itself
// each lane holds {x_l, x_(l^16)}, after a 32-row swap {x_l, x_(l^32)}.  The
// operations are commutative, so all four lanes get bitwise the same result.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One 256-thread workgroup normalises one row of H floats held as up to
// RMS_V4 f32x4 per thread (vector e = threadIdx.x + 256 i, e < H/4): the
// row's sum of squares in a fixed order (per thread, then per wave, then the
// four waves in pairs) and the scale 1/sqrt(mean + eps).  Both the plain
// RMSNorm and the one fused behind a split projection use it, so their
// results agree bit for bit.
constexpr int RMS_V4 = 8;  // H <= 4 * 256 * RMS_V4
__device__ __forceinline__ float rms_row_scale(const f32x4 (&v)[RMS_V4], int64_t H, float eps) {
  const int64_t H4 = H / 4;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i)
    if (threadIdx.x + (int64_t)i * 256 < H4)
      ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  ss = wave_sum(ss);
  __shared__ float rms_part[4];
  if ((threadIdx.x & 63) == 0) rms_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (rms_part[0] + rms_part[1]) + (rms_part[2] + rms_part[3]);
  return 1.0f / sqrtf(tot / (float)H + eps);
}
// gain [H] (NULL: 1) for this thread's vectors, loaded ahead of the row
template <typename T>
__device__ __forceinline__ void rms_row_gain(const T* __restrict__ gain, int64_t H, f32x4 (&g)[RMS_V4]) {
  const int64_t H4 = H / 4;
  if (gain) {
#pragma unroll
    for (int i = 0; i < RMS_V4; ++i) {
      const int64_t e = threadIdx.x + (int64_t)i * 256;
      g[i] = Elem<T>::load4(gain, e < H4 ? e : 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RMS_V4; ++i) g[i] = f32x4{1.f, 1.f, 1.f, 1.f};
  }
}
template <typename T>
__device__ __forceinline__ void rms_row_store(const f32x4 (&v)[RMS_V4], int64_t H, float rs,
                                              const f32x4 (&g)[RMS_V4], T* __restrict__ orow) {
  const int64_t H4 = H / 4;
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    const int64_t e = threadIdx.x + (int64_t)i * 256;
    if (e < H4) Elem<T>::store4(orow, e, (v[i] * rs) * g[i]);
  }
}

// Rotary positions, rotate-half pairs (j, j + D/2): the pair's frequency
// base^(-2j/D) and, at position pos, the angle in fp64, reduced by quarter
// turns, with its cosine and sine in fp32; the rotation with explicit FMAs.  Shared
// by the standalone rotary kernel and the projection epilogue that fuses it,
// so the two agree bit for bit.
__device__ __forceinline__ double rope_inv_freq(int j, int D, double log2_base) {
  return exp2(-(2.0 * j / D) * log2_base);
}
__device__ __forceinline__ void rope_cs(int pos, double inv, float& c, float& s) {
  // quarter turns q = rint(ang / (pi/2)) taken off in fp64, leaving
  // |r| <= pi/4; sin r and cos r from their Taylor series in fp32 (the first
  // omitted terms, r^11/11! and r^12/12!, are below 2e-9 there), then turned
  // by q quarter turns.  Within fp32 rounding of sin and cos (7.9e-8 worst
  // of 2e5 random positions and frequencies against fp64), in ~30
  // instructions instead of a library sincosf.
  const double ang = (double)pos * inv;
  const double half_pi = 1.5707963267948966192313216916398;
  const double inv_half_pi = 0.63661977236758134307553505349006;  // only rounded to an integer
  const double qd = rint(ang * inv_half_pi);
  const float r = (float)__builtin_fma(-half_pi, qd, ang);
  const float r2 = r * r;
  float ps = __builtin_fmaf(r2, 1.f / 362880.f, -1.f / 5040.f);
  ps = __builtin_fmaf(r2, ps, 1.f / 120.f);
  ps = __builtin_fmaf(r2, ps, -1.f / 6.f);
  const float sr = __builtin_fmaf(r * r2, ps, r);
  float pc = __builtin_fmaf(r2, -1.f / 3628800.f, 1.f / 40320.f);
  pc = __builtin_fmaf(r2, pc, -1.f / 720.f);
  pc = __builtin_fmaf(r2, pc, 1.f / 24.f);
  pc = __builtin_fmaf(r2, pc, -0.5f);
  const float cr = __builtin_fmaf(r2, pc, 1.f);
  const int q = (int)(long long)qd & 3;
  const float a = (q & 1) ? cr : sr, b = (q & 1) ? sr : cr;  // sin, cos of r + (q & 1) pi/2 up to sign
  s = (q & 2) ? -a : a;
  c = ((q + 1) & 2) ? -b : b;
}
// (x1, x2) = elements j and j + D/2 -> their rotated values
__device__ __forceinline__ void rope_rot(float x1, float x2, float c, float s, float& y1, float& y2) {
  y1 = __builtin_fmaf(x1, c, -(x2 * s));
  y2 = __builtin_fmaf(x2, c, x1 * s);
}

// One LDS-DMA instruction: every lane's 16 bytes at gptr land at LDS byte
// address lds_addr + 16 * lane (lds_addr is wave-uniform, set in m0).  It is
// issued from inline asm so that the compiler does not treat it as an LDS
// store it must wait for before every LDS read (it would wait for all DMA in
// flight); the kernel's own vmcnt waits and barriers order the accesses.
// The instruction writes no register.  m0 is reserved (it cannot be named
// as clobbered), so the block saves it in a scratch SGPR and restores it
// after the instruction has issued: whatever value the compiler keeps in m0
// around the call survives it.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(m0v), "v"(gptr)
               : "memory");
}

// s_waitcnt immediate that waits for at most n vector-memory operations in
// flight and leaves the LDS/scalar and export counters alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
__host__ __device__ constexpr int waitcnt_vm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
constexpr int WAITCNT_LGKM0 = 0xC07F;  // lgkmcnt(0) only

// One KV pool per layer (K and V), passed by value to the kernels that touch
// every layer's cache.
struct LayerPtrs {
  void* k[MEDUSA_MAX_LAYERS];
  void* v[MEDUSA_MAX_LAYERS];
};

}  // namespace medusa

// ---------------------------------------------------------------------------
// Host side: status handling shared by the entry points.
// ---------------------------------------------------------------------------
namespace medusa_host {
void set_error(const char* fmt, ...);
int32_t fail(int32_t status, const char* fmt, ...);
int32_t check_launch(const char* what);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace medusa_host

#define MEDUSA_REQUIRE(cond, status, ...)                                    \
  do {                                                                       \
    if (!(cond)) return medusa_host::fail((status), __VA_ARGS__);            \
  } while (0)
