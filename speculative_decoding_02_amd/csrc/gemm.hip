// Skinny projection GEMM  Y = epilogue(X W^T)  on MFMA (gfx950).
//
// Serves the heads' two layers ("Medusa Heads", section "Come le teste
// prevedono i token successivi": a residual SiLU feed-forward layer, then a
// vocabulary projection) and every projection of the verification forward
// pass.  At decode shapes (M <= 64 rows) the work is bound by streaming W
// from HBM, so the design goal is many independent 16-byte weight loads in
// flight, not MFMA throughput:
//   * one workgroup = 4 waves computes a [16*MB x 32] output tile over the
//     full contraction; the contraction steps are split evenly over the
//     waves, each wave streaming its slice of 32 weight rows straight from
//     HBM into registers (no LDS for W: no wave shares W data);
//   * the 4 partial tiles are added in LDS in wave order, so an output's
//     reduction order depends on Kd only (never on M or the batch);
//   * the epilogue (bias + SiLU + residual, residual add, SwiGLU) is fused.
#include <algorithm>

#include "common.h"

namespace medusa {

template <typename T> struct GemmTraits;
template <> struct GemmTraits<bf16_t> {
  static constexpr int per16 = 8;   // contraction elements per 16-byte vector
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return mfma_bf16_16x16x32(a, b, c);
  }
};
template <> struct GemmTraits<float> {
  static constexpr int per16 = 4;
  static __device__ __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    c = mfma_f32_16x16x4(__uint_as_float(a.x), __uint_as_float(b.x), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.y), __uint_as_float(b.y), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.z), __uint_as_float(b.z), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.w), __uint_as_float(b.w), c);
    return c;
  }
};

// Register-ring depth (contraction steps in flight per wave) for a given
// number of 16-row blocks of X: the ring holds MB + NB 16-byte vectors per
// step, kept near 150 VGPRs so two waves fit on each SIMD.
#ifndef MEDUSA_GEMM_PF
#define MEDUSA_GEMM_PF 0
#endif
template <int MB, int NB> struct GemmRing {
  static constexpr int per_step = MB + NB;
  static constexpr int PF = MEDUSA_GEMM_PF > 0 ? MEDUSA_GEMM_PF
                          : per_step >= 8 ? 4 : per_step >= 6 ? 6 : per_step >= 4 ? 8 : 12;
};

template <typename T, int MB, int NB, int KS, int EPI>
__global__ __launch_bounds__(64 * KS) void gemm_kernel(const T* __restrict__ X, int64_t xbs,
                                                       int M, int Kd, const T* __restrict__ W,
                                                       int Nw, const T* __restrict__ bias,
                                                       const void* aux, void* Y, int y_f32) {
  using TR = GemmTraits<T>;
  constexpr int P16 = TR::per16;
  constexpr int KSTEP = 4 * P16;
  constexpr int TM = 16 * MB, TN = 16 * NB;
  constexpr int LDR = TN + 1;  // padded LDS row (floats)
  constexpr int PF = GemmRing<MB, NB>::PF;
  constexpr int NT = 64 * KS;
  static_assert(EPI != MEDUSA_EPI_SWIGLU || NB % 2 == 0, "SwiGLU needs gate/up block pairs in a tile");
  __shared__ float red[KS][TM * LDR];

  const int g = blockIdx.z;
  const int n0 = blockIdx.x * TN;
  const int m0 = blockIdx.y * TM;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;

  const T* Xg = X + (int64_t)g * xbs;
  const T* Wg = W + (int64_t)g * Nw * Kd;
  const T* xrow[MB];
  const T* wrow[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int r = min(m0 + mb * 16 + lr, M - 1);
    xrow[mb] = Xg + (int64_t)r * Kd + lg * P16;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    int r = min(n0 + nb * 16 + lr, Nw - 1);
    wrow[nb] = Wg + (int64_t)r * Kd + lg * P16;
  }

  // Contraction steps: nfull full steps (every lane's 16-byte vector in
  // range) split evenly over the KS waves, plus at most one ragged tail step
  // done by the last wave.  Loads in the main loop are unconditional (clamped
  // to a valid step) and never feed a select, so the ring really keeps PF
  // steps of loads in flight; out-of-range steps are skipped at compute.
  const int nfull = Kd / KSTEP;
  const int s_beg = (int)((int64_t)nfull * wave / KS);
  const int s_end = (int)((int64_t)nfull * (wave + 1) / KS);
  const int s_last = max(s_end - 1, 0);

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 fa[PF][MB], fb[PF][NB];
  auto load = [&](int u, int st) {
    const int k = st * KSTEP;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[u][mb] = *reinterpret_cast<const u32x4*>(xrow[mb] + k);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fb[u][nb] = *reinterpret_cast<const u32x4*>(wrow[nb] + k);
  };
  auto compute = [&](int u) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = TR::mma(fa[u][mb], fb[u][nb], acc[mb][nb]);
  };

  if (s_beg < s_end) {
    // ring of PF steps in flight; slot u holds step s + u.  The loop body has
    // no branches, so the compiler's wait before each slot's compute counts
    // exactly the later slots' loads.
#pragma unroll
    for (int u = 0; u < PF; ++u) load(u, min(s_beg + u, s_last));
    int s = s_beg;
    for (; s + PF <= s_end; s += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        compute(u);
        load(u, min(s + u + PF, s_last));
      }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
      if (u < s_end - s) compute(u);  // remainder: already in slots 0..r-1
  }
  if (Kd % KSTEP != 0 && wave == KS - 1) {
    // ragged tail step: lanes whose vector starts past Kd contribute zeros
    const int k = nfull * KSTEP;
    const bool ok = k + lg * P16 < Kd;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) fa[0][mb] = ok ? *reinterpret_cast<const u32x4*>(xrow[mb] + k) : zero;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fb[0][nb] = ok ? *reinterpret_cast<const u32x4*>(wrow[nb] + k) : zero;
    compute(0);
  }

  // partial tiles -> LDS, summed in wave order
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[wave][(mb * 16 + lg * 4 + r) * LDR + nb * 16 + lr] = acc[mb][nb][r];
  __syncthreads();

  if (EPI == MEDUSA_EPI_SWIGLU) {
    // each 32-column pair of blocks: [0,16) gate rows, [16,32) the matching up rows
    const int F = Nw / 2;
    T* Yg = reinterpret_cast<T*>(Y) + (int64_t)g * M * F;
    for (int e = threadIdx.x; e < TM * (TN / 2); e += NT) {
      const int row = e / (TN / 2), cc = e % (TN / 2);
      const int pair = cc >> 4, c = cc & 15;
      const int m = m0 + row, f = (n0 >> 1) + pair * 16 + c;
      if (m >= M || f >= F) continue;
      float gte = 0.f, up = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        gte += red[w][row * LDR + pair * 32 + c];
        up += red[w][row * LDR + pair * 32 + 16 + c];
      }
      st<T>(Yg, (int64_t)m * F + f, silu_f(gte) * up);
    }
    return;
  }

  for (int e = threadIdx.x; e < TM * TN; e += NT) {
    const int row = e / TN, col = e % TN;
    const int m = m0 + row, n = n0 + col;
    if (m >= M || n >= Nw) continue;
    float v = red[0][row * LDR + col];
#pragma unroll
    for (int w = 1; w < KS; ++w) v += red[w][row * LDR + col];
    const int64_t o = (int64_t)g * M * Nw + (int64_t)m * Nw + n;
    if (EPI == MEDUSA_EPI_NONE) {
      if (y_f32) reinterpret_cast<float*>(Y)[o] = v;
      else st<T>(reinterpret_cast<T*>(Y), o, v);
    } else if (EPI == MEDUSA_EPI_BIAS_SILU_RES) {
      const T* R = reinterpret_cast<const T*>(aux) + (int64_t)g * xbs;
      const float res = ld<T>(R, (int64_t)m * Nw + n);
      const float b = bias ? ld<T>(bias, (int64_t)g * Nw + n) : 0.f;
      st<T>(reinterpret_cast<T*>(Y), o, res + silu_f(v + b));
    } else {  // MEDUSA_EPI_RES_ADD_F32
      const float res = reinterpret_cast<const float*>(aux)[(int64_t)m * Nw + n];
      reinterpret_cast<float*>(Y)[(int64_t)m * Nw + n] = res + v;
    }
  }
}

// Variant for M > 16 rows: the 4 waves split the OUTPUT rows (16*NB weight
// rows each, full contraction per wave) and share the activation rows
// through LDS, loaded cooperatively one 256-wide contraction chunk at a time
// (the next chunk is staged in registers while the current one is used).
// Each activation byte then costs one load instruction per workgroup instead
// of one per wave, which keeps the weight stream's loads in flight.  Each
// output is one wave's single accumulation chain in step order, so results
// do not depend on M or the batch.
constexpr int XL_KC = 256;  // contraction chunk (elements) held in LDS
template <typename T, int MB, int NB, int EPI>
__global__ __launch_bounds__(256) void gemm_xlds_kernel(const T* __restrict__ X, int64_t xbs,
                                                        int M, int Kd, const T* __restrict__ W,
                                                        int Nw, const T* __restrict__ bias,
                                                        const void* aux, void* Y, int y_f32,
                                                        int ksplit, float* __restrict__ part) {
  using TR = GemmTraits<T>;
  constexpr int P16 = TR::per16;
  constexpr int KSTEP = 4 * P16;
  constexpr int SC = XL_KC / KSTEP;          // steps per chunk
  constexpr int TM = 16 * MB;
  constexpr int LDX = XL_KC + P16;           // padded LDS row (elements)
  constexpr int XV = TM * XL_KC / P16 / 256; // 16-byte vectors per thread per chunk
  constexpr int PF = MEDUSA_GEMM_PF > 0 ? MEDUSA_GEMM_PF : (NB >= 4 ? 4 : 8);
  static_assert(SC % PF == 0, "ring slots must align with chunk boundaries");
  static_assert(NB % 2 == 0 || EPI != MEDUSA_EPI_SWIGLU, "SwiGLU pairs blocks within a wave");
  __shared__ __attribute__((aligned(16))) T xs[TM * LDX];

  const int g = blockIdx.z / ksplit, ks = blockIdx.z % ksplit;
  const int m0 = blockIdx.y * TM;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * (64 * NB) + wave * 16 * NB;
  const T* Xg = X + (int64_t)g * xbs;
  const T* Wg = W + (int64_t)g * Nw * Kd;
  const T* wrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = min(n0 + nb * 16 + lr, Nw - 1);
    wrow[nb] = Wg + (int64_t)r * Kd + lg * P16;
  }
  // this workgroup's share of the contraction: chunks [c_beg, c_end)
  const int total_chunks = Kd / XL_KC;   // Kd is a multiple of XL_KC here
  const int c_beg = (int)((int64_t)total_chunks * ks / ksplit);
  const int c_end = (int)((int64_t)total_chunks * (ks + 1) / ksplit);
  const int nchunks = c_end - c_beg;
  const int step0 = c_beg * SC;
  const int nsteps = nchunks * SC;

  // cooperative activation chunk: vector v of thread t covers row idx/(KC/P16)
  u32x4 xr[XV];
  auto xload = [&](int c) {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = threadIdx.x + i * 256;
      const int row = idx / (XL_KC / P16), col = idx % (XL_KC / P16);
      const int rr = min(m0 + row, M - 1);
      xr[i] = *reinterpret_cast<const u32x4*>(Xg + (int64_t)rr * Kd + (c_beg + c) * XL_KC + col * P16);
    }
  };
  auto xstore = [&]() {
#pragma unroll
    for (int i = 0; i < XV; ++i) {
      const int idx = threadIdx.x + i * 256;
      const int row = idx / (XL_KC / P16), col = idx % (XL_KC / P16);
      *reinterpret_cast<u32x4*>(&xs[row * LDX + col * P16]) = xr[i];
    }
  };

  f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 fb[PF][NB];
  auto wload = [&](int u, int st) {
    const int k = (step0 + min(st, nsteps - 1)) * KSTEP;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) fb[u][nb] = *reinterpret_cast<const u32x4*>(wrow[nb] + k);
  };

#pragma unroll
  for (int u = 0; u < PF; ++u) wload(u, u);
  xload(0);
  int s = 0;
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // everyone is done reading the previous chunk
    xstore();
    __syncthreads();
    if (c + 1 < nchunks) xload(c + 1);
    // SC steps of this chunk; the weight ring runs across chunk boundaries
    for (int s0 = 0; s0 < SC; s0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int sl = s0 + u;  // step within the chunk (SC is a multiple of PF)
        u32x4 xa[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xa[mb] = *reinterpret_cast<const u32x4*>(&xs[(mb * 16 + lr) * LDX + sl * KSTEP + lg * P16]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = TR::mma(xa[mb], fb[u][nb], acc[mb][nb]);
        wload(u, s + sl + PF);
      }
    }
    s += SC;
  }

  // epilogue straight from the accumulators: lane holds weight row
  // n0 + nb*16 + lr and activation rows m0 + mb*16 + 4*lg + r
  if (ksplit > 1) {  // fp32 partial of this contraction share; gemm_split_reduce finishes
    float* pg = part + ((int64_t)g * ksplit + ks) * M * Nw;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + mb * 16 + lg * 4 + r, n = n0 + nb * 16 + lr;
          if (m < M && n < Nw) pg[(int64_t)m * Nw + n] = acc[mb][nb][r];
        }
    return;
  }
  if (EPI == MEDUSA_EPI_SWIGLU) {
    // NB is even: block 2j is gate, 2j+1 the matching up rows
    const int F = Nw / 2;
    T* Yg = reinterpret_cast<T*>(Y) + (int64_t)g * M * F;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB / 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + mb * 16 + lg * 4 + r;
          const int f = (n0 >> 1) + j * 16 + lr;
          if (m < M && f < F) st<T>(Yg, (int64_t)m * F + f, silu_f(acc[mb][2 * j][r]) * acc[mb][2 * j + 1][r]);
        }
    return;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + mb * 16 + lg * 4 + r, n = n0 + nb * 16 + lr;
        if (m >= M || n >= Nw) continue;
        const float v = acc[mb][nb][r];
        const int64_t o = (int64_t)g * M * Nw + (int64_t)m * Nw + n;
        if (EPI == MEDUSA_EPI_NONE) {
          if (y_f32) reinterpret_cast<float*>(Y)[o] = v;
          else st<T>(reinterpret_cast<T*>(Y), o, v);
        } else if (EPI == MEDUSA_EPI_BIAS_SILU_RES) {
          const T* R = reinterpret_cast<const T*>(aux) + (int64_t)g * xbs;
          const float res = ld<T>(R, (int64_t)m * Nw + n);
          const float b = bias ? ld<T>(bias, (int64_t)g * Nw + n) : 0.f;
          st<T>(reinterpret_cast<T*>(Y), o, res + silu_f(v + b));
        } else {
          const float res = reinterpret_cast<const float*>(aux)[(int64_t)m * Nw + n];
          reinterpret_cast<float*>(Y)[(int64_t)m * Nw + n] = res + v;
        }
      }
}

// ---------------------------------------------------------------------------
// Block-range plan for M >= 2 rows (bf16): G workgroups of eight waves per
// (batch element, activation-row tile, contraction split), about one per
// compute unit, each owning a contiguous range of whole 16-row weight blocks
// (pairs of blocks for SwiGLU, whose gate and up rows interleave in 16-row
// blocks).  Wave w streams block w of the range (waves past the range only
// help stage activations).  Workgroup g starts its contraction at chunk
// g*nchunks/G and wraps round: at any moment the compute units read different
// column offsets of their rows (when all start at column 0 together the weight
// stream measured 20-35% slower).  The activation rows are staged through two
// LDS buffers, one 256-wide chunk at a time, with one barrier per chunk.  The
// epilogues with arithmetic go through LDS, so a gate block and its up block
// may sit in different waves and the output stores are coalesced; plain fp32
// results (split partials, fp32 outputs) are stored by each wave from its
// accumulators.  Each output is one
// wave's accumulation chain in step order from the workgroup's start chunk:
// results depend on (Kd, N) and the launch plan, itself a function of the
// shape.
constexpr int XB_KC = 256;
constexpr int XB_WAVES = 8;
constexpr int XB_MAXB = XB_WAVES;  // blocks per workgroup: one per wave

template <typename T, int EPI>
__device__ __forceinline__ void xb_store(int gi, int M, int Nw, int64_t xbs, const T* bias,
                                         const void* aux, void* Y, int y_f32, int m, int n, float v) {
  const int64_t o = (int64_t)gi * M * Nw + (int64_t)m * Nw + n;
  if (EPI == MEDUSA_EPI_NONE) {
    if (y_f32) reinterpret_cast<float*>(Y)[o] = v;
    else st<T>(reinterpret_cast<T*>(Y), o, v);
  } else if (EPI == MEDUSA_EPI_BIAS_SILU_RES) {
    const T* R = reinterpret_cast<const T*>(aux) + (int64_t)gi * xbs;
    const float res = ld<T>(R, (int64_t)m * Nw + n);
    const float b = bias ? ld<T>(bias, (int64_t)gi * Nw + n) : 0.f;
    st<T>(reinterpret_cast<T*>(Y), o, res + silu_f(v + b));
  } else {  // MEDUSA_EPI_RES_ADD_F32
    const float res = reinterpret_cast<const float*>(aux)[(int64_t)m * Nw + n];
    reinterpret_cast<float*>(Y)[(int64_t)m * Nw + n] = res + v;
  }
}


// The block-range kernel, with every operand brought in by LDS DMA (bf16).
// A register load of a weight step would read 64 bytes of each of 16 rows
// (the MFMA operand layout); here one DMA instruction reads 256 contiguous
// bytes of each of 4 rows (two whole 128-byte lines per row) into a per-wave
// LDS ring, and the MFMA operands are read back from LDS.  The activation chunk
// comes in by DMA too (no registers, no LDS store instructions), double
// buffered with one barrier per chunk.  Nothing is loaded into registers from
// global memory in the loop, so every wait is an explicit vmcnt immediate
// counted from the fixed issue order:
//   chunk head:  [wait: own DMA of chunk q landed] barrier, DMA chunk q+1
//   group g (4 steps, 2 per chunk): [wait: group g landed] 4 steps of MFMA,
//                lgkmcnt(0), DMA group g+2 into the slot just read
// In LDS both operands are XOR-swizzled in 16-byte units (slot ^ row) so
// that the 16 rows of one operand read fall in distinct banks; the swizzle is
// applied on the global side, since a DMA lane's LDS address is fixed.
// Internal epilogue of the QKV projection with rotary positions fused: W's q
// and k head rows are pair-interleaved (rows 2j, 2j+1 of a head = elements j,
// j + D/2), the accumulators are rounded to the model dtype (as the unfused
// projection stores them), rotated, and written to q, k, v [M, heads, D].
constexpr int EPI_ROPE_QKV = 16;
struct RopeArgs {
  const int32_t* pos;
  double log2_base;
  int Hq, Hkv, D;
  bf16_t* q;
  bf16_t* k;
  bf16_t* v;
};

#ifndef MEDUSA_GEMM_XD_WR
#define MEDUSA_GEMM_XD_WR 2  // weight groups in flight per wave (4 steps, 4 KB each)
#endif

template <int MB, int WR, int EPI>
__global__ __launch_bounds__(64 * XB_WAVES) void gemm_xdma_kernel(
    const bf16_t* __restrict__ X, int64_t xbs, int M, int Kd, const bf16_t* __restrict__ W, int Nw,
    const bf16_t* __restrict__ bias, const void* aux, void* Y, int y_f32, int G, int MT, int unit,
    float* __restrict__ part, int nsub, RopeArgs ra) {
  using T = bf16_t;
  constexpr int P16 = 8;                        // bf16 per 16 bytes
  constexpr int TM = 16 * MB;
  constexpr int XROWB = XB_KC * 2;              // bytes of one activation row per chunk
  constexpr int XBUFB = TM * XROWB;
  constexpr int XD = XBUFB / 1024 / XB_WAVES;   // activation DMAs per wave per chunk
  constexpr int WGB = 16 * 256;                 // one weight group: 16 rows x 256 bytes
  constexpr int WSLOTB = WR * WGB;
  constexpr int LDE = TM + 1;
  constexpr int SMEM = 2 * XBUFB + XB_WAVES * WSLOTB;
  static_assert(XD >= 1 && XD * XB_WAVES * 1024 == XBUFB, "activation chunk must split into whole DMAs");
  static_assert(XB_MAXB * 16 * LDE * 4 + XB_MAXB * 8 * 12 <= SMEM, "epilogue tile (and pair tables) must fit");
  static_assert(WR == 2 || WR == 3, "wait counts are worked out for rings of 2 and 3 groups");
  // Issue order per wave: prologue W(0) [.. W(WR-3)], X(0), W(WR-2), W(WR-1);
  // then per chunk q: X(q+1), group 2q, W(2q+WR), group 2q+1, W(2q+1+WR).
  // DMAs issued after the one awaited (4 per weight group, XD per chunk):
  constexpr int WAIT_CHUNK = waitcnt_vm(2 * 4);  // X(q): W(2q+WR-2), W(2q+WR-1)
  constexpr int WAIT_G0 = waitcnt_vm(WR == 2 ? 4 + XD : 8 + 2 * XD);  // W(2q): ..., X(q+1)
  constexpr int WAIT_G1 = waitcnt_vm(WR == 2 ? 4 + XD : 8 + XD);      // W(2q+1): ..., W(2q+WR)
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  float* ep = reinterpret_cast<float*>(smem);  // after the contraction

  const int g = blockIdx.x, slice = blockIdx.y;
  const int gi = slice / MT, m0 = (slice % MT) * TM;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int nunits = (Nw / 16) / unit;
  const int u0 = (int)((int64_t)g * nunits / G), u1 = (int)((int64_t)(g + 1) * nunits / G);
  const int b0 = u0 * unit, nb = (u1 - u0) * unit;  // this workgroup's blocks (<= XB_MAXB)
  // contraction split sp of S: chunks [cb, cb + nchunks)
  const int sp = blockIdx.z, S = gridDim.z;
  const int cb = (int)((int64_t)sp * (Kd / XB_KC) / S);
  const int nchunks = (int)((int64_t)(sp + 1) * (Kd / XB_KC) / S) - cb;
  const int ngroups = 2 * nchunks;
  const int c0 = (int)((int64_t)g * nchunks / G);  // start chunk within the split (< nchunks)
  const T* Xg = X + (int64_t)gi * xbs;
  const T* Wg = W + (int64_t)gi * Nw * Kd;

  // chunk q of this workgroup's order -> buffer q&1; DMA j covers rows 2j, 2j+1
  auto xissue = [&](int q) {
    int c = c0 + min(q, nchunks - 1);
    if (c >= nchunks) c -= nchunks;
    c += cb;
    const uint32_t base = lds0 + (q & 1) * XBUFB;
#pragma unroll
    for (int i = 0; i < XD; ++i) {
      const int j = wave * XD + i;
      const int row = 2 * j + (lane >> 5), slot = lane & 31;
      const int rr = min(m0 + row, M - 1);
      lds_dma16(Xg + (int64_t)rr * Kd + c * XB_KC + (slot ^ (row & 15)) * P16, base + j * 1024);
    }
  };
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](auto activec) {
    constexpr bool ACT = decltype(activec)::value;
    const T* wblk = Wg + (int64_t)min(b0 + wave, Nw / 16 - 1) * 16 * Kd;
    const uint32_t wring = lds0 + 2 * XBUFB + wave * WSLOTB;
    // weight group gq of this workgroup's order -> ring slot gq % WR;
    // DMA qq covers rows 4qq..4qq+3, 256 bytes each
    auto wissue = [&](int gq) {
      int pg = c0 * 2 + min(gq, ngroups - 1);
      if (pg >= ngroups) pg -= ngroups;
      pg += 2 * cb;
      const uint32_t base = wring + (gq % WR) * WGB;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int row = 4 * qq + (lane >> 4), slot = lane & 15;
        lds_dma16(wblk + (int64_t)row * Kd + pg * 128 + (slot ^ row) * P16, base + qq * 1024);
      }
    };
    if constexpr (ACT && WR == 3) wissue(0);
    xissue(0);
    if constexpr (ACT) {
      wissue(WR - 2);
      wissue(WR - 1);
    }
    for (int q = 0; q < nchunks; ++q) {
      __builtin_amdgcn_s_waitcnt(ACT ? WAIT_CHUNK : waitcnt_vm(0));  // own DMA of chunk q landed
      __builtin_amdgcn_s_barrier();  // every wave's, and chunk q-1 is no longer read
      asm volatile("" ::: "memory");
      xissue(q + 1);  // after the last chunk: a clamped copy nobody reads
      if constexpr (ACT) {
        const unsigned char* xb = smem + (q & 1) * XBUFB;
        auto group = [&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const int gq = 2 * q + h;
          __builtin_amdgcn_s_waitcnt(h == 0 ? WAIT_G0 : WAIT_G1);  // group gq landed
          asm volatile("" ::: "memory");
          const unsigned char* wb = smem + 2 * XBUFB + wave * WSLOTB + (gq % WR) * WGB;
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) {
            const u32x4 bw = *reinterpret_cast<const u32x4*>(wb + lr * 256 + (((sl * 4 + lg) ^ lr) * 16));
            u32x4 xa[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              xa[mb] = *reinterpret_cast<const u32x4*>(
                  xb + (mb * 16 + lr) * XROWB + ((((h * 4 + sl) * 4 + lg) ^ lr) * 16));
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_bf16_16x16x32(xa[mb], bw, acc[mb]);
          }
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);  // this slot's LDS reads are done
          asm volatile("" ::: "memory");
          wissue(gq + WR);
        };
        group(std::integral_constant<int, 0>());
        group(std::integral_constant<int, 1>());
      }
    }
  };
  if (wave < nb) run(std::true_type());
  else run(std::false_type());
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the clamped refills
  // fp32 results with no epilogue arithmetic (split partials [batch][S][M][N],
  // plain fp32 outputs): each wave stores its own accumulators, lane (lr, lg)
  // holding column lr of its block for rows 4 lg .. 4 lg + 3 of each 16-row
  // block (64-byte row pieces), without the LDS round trip and its barriers
  if constexpr (EPI != EPI_ROPE_QKV) {
    if (S > 1 || (EPI == MEDUSA_EPI_NONE && y_f32 && nsub == Nw)) {
      if (wave < nb) {
        float* dst = S > 1 ? part + ((int64_t)gi * S + sp) * M * Nw
                           : reinterpret_cast<float*>(Y) + (int64_t)gi * M * Nw;
        dst += (b0 + wave) * 16 + lr;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + mb * 16 + lg * 4 + r;
            if (m < M) dst[(int64_t)m * Nw] = acc[mb][r];
          }
      }
      return;
    }
  }
  __syncthreads();  // the operand buffers become the epilogue tile
  if (wave < nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) ep[(wave * 16 + lr) * LDE + mb * 16 + lg * 4 + r] = acc[mb][r];
  }
  __syncthreads();

  constexpr int NT = 64 * XB_WAVES;
  if constexpr (EPI == EPI_ROPE_QKV) {
    // pairs of adjacent columns: per pair of this range its frequency and
    // its output (q, k or v, and the column in that row) first
    const int np = nb * 8;
    const int qw = ra.Hq * ra.D, kw = ra.Hkv * ra.D, half = ra.D / 2;
    double* invt = reinterpret_cast<double*>(smem + XB_MAXB * 16 * LDE * 4);
    int* ptab = reinterpret_cast<int*>(invt + XB_MAXB * 8);
    if (threadIdx.x < np) {
      const int n = b0 * 16 + 2 * threadIdx.x;  // even column of qkv
      const int kind = n < qw ? 0 : n < qw + kw ? 1 : 2;
      const int nh = kind == 0 ? n : n - qw;
      // q and k rows 2j, 2j + 1 of a head are its elements j, j + D/2
      const int col = kind == 2 ? n - qw - kw : (nh / ra.D) * ra.D + (nh % ra.D) / 2;
      invt[threadIdx.x] = rope_inv_freq((n % ra.D) / 2, ra.D, ra.log2_base);
      ptab[threadIdx.x] = col * 4 + kind;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < np * TM; e += NT) {
      const int m = e / np, pl = e % np;
      if (m0 + m >= M) continue;
      const float x1 = bf2f(f2bf(ep[(2 * pl) * LDE + m]));
      const float x2 = bf2f(f2bf(ep[(2 * pl + 1) * LDE + m]));
      const int64_t row = m0 + m;
      const int info = ptab[pl], kind = info & 3, col = info >> 2;
      if (kind < 2) {
        T* dst = (kind == 0 ? ra.q + row * qw : ra.k + row * kw) + col;
        float c, sn, y1, y2;
        rope_cs(ra.pos[row], invt[pl], c, sn);
        rope_rot(x1, x2, c, sn, y1, y2);
        dst[0] = f2bf(y1);
        dst[half] = f2bf(y2);
      } else {
        T* dst = ra.v + row * kw + col;
        dst[0] = f2bf(x1);
        dst[1] = f2bf(x2);
      }
    }
    return;
  }
  if (EPI == MEDUSA_EPI_SWIGLU) {
    const int F = Nw / 2, f0 = b0 / 2 * 16, nf = nb / 2 * 16;
    T* Yg = reinterpret_cast<T*>(Y) + (int64_t)gi * M * F;
    for (int e = threadIdx.x; e < nf * TM; e += NT) {
      const int m = e / nf, fl = e % nf;
      const int gr = (fl / 16) * 32 + fl % 16;  // gate row in the range; up is 16 further
      if (m0 + m < M) st<T>(Yg, (int64_t)(m0 + m) * F + f0 + fl, silu_f(ep[gr * LDE + m]) * ep[(gr + 16) * LDE + m]);
    }
    return;
  }
  // nsub < Nw: a batch sharing its activation rows planned as one projection
  // onto its stacked weights; output column n is column n % nsub of element n / nsub
  const int nn = nb * 16;
  if (nsub == Nw) {
    for (int e = threadIdx.x; e < nn * TM; e += NT) {
      const int m = e / nn, nl = e % nn;
      if (m0 + m < M) xb_store<T, EPI>(gi, M, Nw, xbs, bias, aux, Y, y_f32, m0 + m, b0 * 16 + nl, ep[nl * LDE + m]);
    }
  } else {
    for (int e = threadIdx.x; e < nn * TM; e += NT) {
      const int m = e / nn, nl = e % nn, n = b0 * 16 + nl;
      if (m0 + m < M) xb_store<T, EPI>(n / nsub, M, nsub, xbs, bias, aux, Y, y_f32, m0 + m, n % nsub, ep[nl * LDE + m]);
    }
  }
}

// Large-row projection (M >= 256 rows: batched serving, heads over many
// rows), where the product is MFMA-bound rather than weight-stream bound.
//   * A workgroup computes a TN x TM tile of Y^T (TN weight rows by TM
//     activation rows) with WGN x WGM waves, each a WN x WM sub-tile of FN x FM
//     16x16 MFMA blocks.  The weight rows are the A operand and the
//     activation rows the B operand, so a lane's four results are four
//     consecutive output columns of one output row (vector stores).
//   * The contraction advances in stages of BK elements: a stage holds the
//     TN + TM rows' 2*BK-byte pieces, brought in by LDS-DMA (each lane's
//     source row and chunk are fixed, only the contraction offset moves) into
//     a ring of R stages: the first R stages are issued together, a slot is
//     refilled as soon as every wave has read it, and the wait before stage
//     t counts exactly the later stages already issued (one barrier per
//     stage, no fence).
//   * Inside a stage, row r keeps its 16-byte chunk c at position
//     c ^ ((r / L) % C), with L = 256 / (2*BK) rows per 64-bank line and C
//     chunks per row: the 16 rows of one operand read then fall in 16
//     distinct bank groups.
//   * Workgroup ids are remapped so that the ids one XCD receives (the
//     dispatcher deals them out round robin) walk the activation tiles of one
//     weight tile: the weight tile is read from memory once per XCD.
//   * Accumulation runs over the contraction in stage order, the same for
//     every shape of this plan: results depend on (M, Kd, N) only.
constexpr int GB_KALIGN = 64;  // contraction multiple the plan requires
// Wave priority while a wave issues its MFMAs (PRIO > 0: raised, so that of
// the waves ready to issue, those with their operands in registers go first
// and the MFMA pipe stays fed).  Measured at 1024 rows: the heads' W2 on
// 256 x 256 tiles -2%, their W1 on 192 x 256 tiles -4.6%, QKV and gate/up
// unchanged, the 128 x 128 tiles (8 waves of 64 x 32) 1-2% slower.
#ifndef MEDUSA_GEMM_BIG_PRIO
#define MEDUSA_GEMM_BIG_PRIO 1
#endif
template <int TN, int TM, int WGN, int WGM, int BK, int R, int EPI, int PRIO>
__global__ __launch_bounds__(64 * WGN * WGM) void gemm_big_kernel(
    const bf16_t* __restrict__ X, int64_t xbs, int M, int Kd, const bf16_t* __restrict__ W, int Nw,
    const bf16_t* __restrict__ bias, const void* aux, void* Y, int y_f32, int tilesN, int tilesM) {
  using T = bf16_t;
  constexpr int NW = WGN * WGM;
  constexpr int WN = TN / WGN, WM = TM / WGM;
  constexpr int FN = WN / 16, FM = WM / 16;
  constexpr int ROWB = BK * 2;               // bytes of one row in a stage
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int LPR = 256 / ROWB;            // rows sharing one 64-bank line
  constexpr int KSTEPS = BK / 32;            // MFMA contraction steps per stage
  constexpr int STAGEB = (TN + TM) * ROWB;
  constexpr int RPD = 1024 / ROWB;           // rows per DMA instruction
  constexpr int DPW = (TN + TM) / RPD / NW;  // DMA instructions per wave per stage
  static_assert(BK == 32 || BK == 64, "stage of 32 or 64 contraction elements");
  static_assert(GB_KALIGN % BK == 0, "the plan's contraction multiple covers a stage");
  static_assert(DPW >= 1 && DPW * NW * RPD == TN + TM, "a stage splits into whole DMAs per wave");
  static_assert(R >= 2 && R <= 4 && (R - 1) * DPW < 64, "ring of 2..4 stages, vmcnt range");
  static_assert(EPI != MEDUSA_EPI_SWIGLU || WN % 32 == 0, "gate/up block pairs inside a wave");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[R * STAGEB];

  const int tiles = tilesN * tilesM;
  const int g = blockIdx.y;  // batch element
  int id = blockIdx.x;
  const int q8 = tiles / 8;
  if (id < 8 * q8) id = (id % 8) * q8 + id / 8;  // XCD-aware: a bijection of [0, 8*q8)
  const int nt = id / tilesM, mt = id % tilesM;
  const int n0 = nt * TN, m0 = mt * TM;
  const T* Wg = W + (int64_t)g * Nw * Kd;
  const T* Xg = X + (int64_t)g * xbs;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wn = wave % WGN, wm = wave / WGN;

  // DMA sources of this lane (rows past the matrix edge re-read its last row;
  // their results are not stored)
  const T* src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int r = (wave * DPW + i) * RPD + lane / CPR;      // stage row this lane fills
    const int c = (lane % CPR) ^ ((r / LPR) % CPR);          // chunk fetched for its position
    src[i] = r < TN ? Wg + (int64_t)min(n0 + r, Nw - 1) * Kd + c * 8
                    : Xg + (int64_t)min(m0 + r - TN, M - 1) * Kd + c * 8;
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  auto issue = [&](int t, int slot) {
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      lds_dma16(src[i] + t * BK, lds_base + slot * STAGEB + (wave * DPW + i) * 1024);
  };
  auto wait_stages = [&](int n) {  // at most n stages of this wave's DMA in flight
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(1 * DPW)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * DPW)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * DPW)); break;
    }
  };

  // operand offsets inside a stage (A: weight rows first, B: activation
  // rows), per contraction step ks (chunk 4*ks + lg).  Every fragment's first
  // row is a multiple of 16, so a row's chunk position depends on lr only
  // ((r / LPR) % CPR = (lr / LPR) % CPR): fragment fn sits a constant
  // fn * 16 rows after fragment 0, and one base register per step serves all
  // fragments of an operand.
  static_assert(TN % 16 == 0 && WN % 16 == 0 && WM % 16 == 0 && 16 % LPR == 0, "fragment rows start at multiples of 16");
  int abase[KSTEPS], bbase[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int c = ((4 * ks + lg) ^ ((lr / LPR) % CPR)) * 16;
    abase[ks] = (wn * WN + lr) * ROWB + c;
    bbase[ks] = (TN + wm * WM + lr) * ROWB + c;
  }

  f32x4 acc[FN][FM];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = Kd / BK;
  const int first = min(nk, R);
  for (int t = 0; t < first; ++t) issue(t, t);
  for (int t = 0; t < nk; ++t) {
    // stages issued before this point: min(nk, R + max(t - 1, 0))
    wait_stages(t == 0 ? first - 1 : min(nk - 1 - t, R - 2));  // stage t has landed
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);  // ... and this wave's reads of stage t-1
    __builtin_amdgcn_s_barrier();               // ... and every other wave's
    asm volatile("" ::: "memory");
    if (t >= 1 && t - 1 + R < nk) issue(t - 1 + R, (t - 1) % R);
    const unsigned char* sb = lds + (t % R) * STAGEB;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 af[FN], bfr[FM];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) af[fn] = *reinterpret_cast<const u32x4*>(sb + abase[ks] + fn * 16 * ROWB);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) bfr[fm] = *reinterpret_cast<const u32x4*>(sb + bbase[ks] + fm * 16 * ROWB);
      if constexpr (PRIO > 0) __builtin_amdgcn_s_setprio(PRIO);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fn][fm] = mfma_bf16_16x16x32(af[fn], bfr[fm], acc[fn][fm]);
      if constexpr (PRIO > 0) __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("" ::: "memory");
  }

  // epilogue: lane holds Y[m][n .. n+3], m = m0 + wm*WM + fm*16 + lr,
  // n = n0 + wn*WN + fn*16 + 4*lg
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * WM + fm * 16 + lr;
    if (m >= M) continue;
    if constexpr (EPI == MEDUSA_EPI_SWIGLU) {
      const int F = Nw / 2;
      T* Yg = reinterpret_cast<T*>(Y) + (int64_t)g * M * F;
#pragma unroll
      for (int fp = 0; fp < FN; fp += 2) {  // gate block fp, up block fp + 1
        const int nb = n0 + wn * WN + fp * 16;
        if (nb >= Nw) continue;
        const int f = nb / 2 + 4 * lg;
        const f32x4 gt = acc[fp][fm], up = acc[fp + 1][fm];
        *reinterpret_cast<u32x2*>(Yg + (int64_t)m * F + f) =
            u32x2{pack_bf2(silu_f(gt[0]) * up[0], silu_f(gt[1]) * up[1]),
                  pack_bf2(silu_f(gt[2]) * up[2], silu_f(gt[3]) * up[3])};
      }
    } else {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int n = n0 + wn * WN + fn * 16 + 4 * lg;
        if (n >= Nw) continue;
        const f32x4 v = acc[fn][fm];
        // four consecutive outputs per lane: one vector access each (the
        // entry point requires Y, aux and bias 16-byte aligned, Nw % 16 == 0)
        const int64_t o = (int64_t)g * M * Nw + (int64_t)m * Nw + n;
        if (EPI == MEDUSA_EPI_NONE) {
          if (y_f32) *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + o) = v;
          else *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(Y) + o) = u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
        } else if (EPI == MEDUSA_EPI_RES_ADD_F32) {  // batch 1: Y, aux [M][Nw] float
          const int64_t r = (int64_t)m * Nw + n;
          const f32x4 res = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(aux) + r);
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + r) =
              f32x4{res[0] + v[0], res[1] + v[1], res[2] + v[2], res[3] + v[3]};
        } else {  // MEDUSA_EPI_BIAS_SILU_RES
          const u32x2 rr = *reinterpret_cast<const u32x2*>(reinterpret_cast<const T*>(aux) + (int64_t)g * xbs +
                                                           (int64_t)m * Nw + n);
          float bb[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const u32x2 bv = *reinterpret_cast<const u32x2*>(bias + (int64_t)g * Nw + n);
#pragma unroll
            for (int q = 0; q < 4; ++q) bb[q] = bf2f((bf16_t)(bv[q / 2] >> (16 * (q % 2))));
          }
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = bf2f((bf16_t)(rr[q / 2] >> (16 * (q % 2)))) + silu_f(v[q] + bb[q]);
          *reinterpret_cast<u32x2*>(reinterpret_cast<T*>(Y) + o) = u32x2{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
        }
      }
    }
  }
}

// 16-row blocks per workgroup of the small-row kernel (SwiGLU needs its
// gate/up pair of blocks in one tile, so it always takes at least 2)
#ifndef MEDUSA_GEMM_NB
#define MEDUSA_GEMM_NB 1
#endif
#ifndef MEDUSA_GEMM_KS
#define MEDUSA_GEMM_KS 4
#endif

// Sum of the split-contraction partials in split order, then the epilogue.
// One thread per output element.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(const float* __restrict__ part,
                                                                int ksplit, int M, int Nw,
                                                                int64_t xbs, const T* __restrict__ bias,
                                                                const void* aux, void* Y, int y_f32) {
  const int g = blockIdx.y;
  const int cols = EPI == MEDUSA_EPI_SWIGLU ? Nw / 2 : Nw;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)M * cols) return;
  const int m = (int)(e / cols), c = (int)(e % cols);
  const float* pg = part + (int64_t)g * ksplit * M * Nw;
  auto sum = [&](int n) {
    float v = pg[(int64_t)m * Nw + n];
    for (int q = 1; q < ksplit; ++q) v += pg[((int64_t)q * M + m) * Nw + n];
    return v;
  };
  if (EPI == MEDUSA_EPI_SWIGLU) {
    const int ncol = (c >> 4) * 32 + (c & 15);  // gate column; up is 16 further
    T* Yg = reinterpret_cast<T*>(Y) + (int64_t)g * M * cols;
    st<T>(Yg, (int64_t)m * cols + c, silu_f(sum(ncol)) * sum(ncol + 16));
    return;
  }
  const float v = sum(c);
  const int64_t o = (int64_t)g * M * Nw + (int64_t)m * Nw + c;
  if (EPI == MEDUSA_EPI_NONE) {
    if (y_f32) reinterpret_cast<float*>(Y)[o] = v;
    else st<T>(reinterpret_cast<T*>(Y), o, v);
  } else if (EPI == MEDUSA_EPI_BIAS_SILU_RES) {
    const T* R = reinterpret_cast<const T*>(aux) + (int64_t)g * xbs;
    const float res = ld<T>(R, (int64_t)m * Nw + c);
    const float b = bias ? ld<T>(bias, (int64_t)g * Nw + c) : 0.f;
    st<T>(reinterpret_cast<T*>(Y), o, res + silu_f(v + b));
  } else {
    const float res = reinterpret_cast<const float*>(aux)[(int64_t)m * Nw + c];
    reinterpret_cast<float*>(Y)[(int64_t)m * Nw + c] = res + v;
  }
}

// Split sum + residual add + RMSNorm, one workgroup per row (N <= 8192):
// x[m] += sum of the partials in split order (the same sums and the same
// final add as gemm_split_reduce_kernel's residual epilogue), then
// out[m] = RMSNorm(x[m]) * gain with the plain RMSNorm's own reduction.
template <typename T, int QB>
__global__ __launch_bounds__(256) void split_reduce_rmsnorm_kernel(const float* __restrict__ part,
                                                                   int ksplit, int M, int N,
                                                                   float* __restrict__ x,
                                                                   const T* __restrict__ gain,
                                                                   float eps, T* __restrict__ out) {
  const int m = blockIdx.x;
  const int N4 = N / 4;
  f32x4* xr = reinterpret_cast<f32x4*>(x + (int64_t)m * N);
  const f32x4* p0 = reinterpret_cast<const f32x4*>(part + (int64_t)m * N);
  const int64_t pstride = (int64_t)M * N4;  // one split's partials, in f32x4
  // Every load is unconditional (indices clamped; lanes past the row only
  // carry unused copies), so a batch of splits costs one memory round trip;
  // the adds keep split order.
  // (the first batch of up to QB splits is loaded together with the
  // residual row and the gain: one round trip for splits <= QB; the launch
  // takes QB = 2 for two splits, else 4, which changes no sum)
  f32x4 g[RMS_V4], v[RMS_V4], acc[RMS_V4];
  int ec[RMS_V4];
  rms_row_gain<T>(gain, N, g);
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    const int e = threadIdx.x + i * 256;
    ec[i] = e < N4 ? e : 0;
    v[i] = xr[ec[i]];
  }
  for (int q0 = 0; q0 < ksplit; q0 += QB) {
    f32x4 t[QB][RMS_V4];
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int i = 0; i < RMS_V4; ++i) t[j][i] = p0[min(q0 + j, ksplit - 1) * pstride + ec[i]];
#pragma unroll
    for (int j = 0; j < QB; ++j)
      if (q0 + j < ksplit)
#pragma unroll
        for (int i = 0; i < RMS_V4; ++i) acc[i] = (q0 + j == 0) ? t[j][i] : acc[i] + t[j][i];
  }
#pragma unroll
  for (int i = 0; i < RMS_V4; ++i) {
    v[i] = v[i] + acc[i];
    if (threadIdx.x + i * 256 < N4) xr[threadIdx.x + i * 256] = v[i];
  }
  const float rs = rms_row_scale(v, N, eps);
  rms_row_store<T>(v, N, rs, g, out + (int64_t)m * N);
}

#ifndef MEDUSA_GEMM_XL_NB
#define MEDUSA_GEMM_XL_NB 2
#endif
#ifndef MEDUSA_GEMM_XL_TARGET_WGS
#define MEDUSA_GEMM_XL_TARGET_WGS 384
#endif
#ifndef MEDUSA_GEMM_XL_MIN_N
#define MEDUSA_GEMM_XL_MIN_N 0
#endif

}  // namespace medusa

namespace medusa_host {
// Launch plan for one projection; a function of (M, Kd, N, dtype) only, never
// of the batch, so that equal shapes always take the same arithmetic path.
struct GemmPlan {
  bool xl;
  int ksplit;
  bool xb;      // block-range variant
  int xb_unit;  // blocks per unit (2: SwiGLU gate/up pairs)
  int xb_G;     // workgroups per (batch element, row tile, contraction split)
  int MT;       // activation-row tiles
  int xb_S;     // contraction splits of the block-range variant (partials when > 1)
  int big;      // large-row MFMA tiling (1; 0 off)
};
#ifndef MEDUSA_GEMM_XB_MIN_BLOCKS
#define MEDUSA_GEMM_XB_MIN_BLOCKS 512
#endif
#ifndef MEDUSA_GEMM_XB_WGS
#define MEDUSA_GEMM_XB_WGS 256
#endif
// narrower outputs (MEDUSA_GEMM_XD_MIN_BLOCKS <= N/16 < MEDUSA_GEMM_XB_MIN_BLOCKS)
// take the DMA block-range kernel with the contraction split this many ways
#ifndef MEDUSA_GEMM_XD_MIN_BLOCKS
#define MEDUSA_GEMM_XD_MIN_BLOCKS 128
#endif
#ifndef MEDUSA_GEMM_XD_SPLIT
#define MEDUSA_GEMM_XD_SPLIT 4
#endif
#ifndef MEDUSA_GEMM_XD_MIN_M
// fewest rows the block-range plan takes (one row keeps the one-block-per-
// workgroup kernel, which streams its weights at 6.2 TB/s there); at 16 rows
// (the heads of a 16-sequence batch) the block ranges took 275 us against
// 434 us for the five heads
#define MEDUSA_GEMM_XD_MIN_M 2
#endif
#ifndef MEDUSA_GEMM_XD_CPS
#define MEDUSA_GEMM_XD_CPS 8  // contraction chunks per split, at least
#endif
#ifndef MEDUSA_GEMM_BIG_MIN_M
#define MEDUSA_GEMM_BIG_MIN_M 256
#endif
// stage depth and ring of the 256- and 128-wide large-row tilings (measured
// at 1024 rows x 4096: 64-deep stages beat 32-deep ones by 6-12%; the ring
// depth beyond two stages changed little)
#ifndef MEDUSA_GEMM_BIG_BK1
#define MEDUSA_GEMM_BIG_BK1 64
#endif
// 256 x 256 tiles: 4 x 4 waves of 64 x 64 (each stage's operand reads from
// LDS: 16 KB per wave against 20 KB for 2 x 8 waves of 128 x 32, which
// measured 2% slower: the heads' vocabulary projection at 1024 rows 1157-1163
// against 1184-1189 us)
#ifndef MEDUSA_GEMM_BIG_WM1
#define MEDUSA_GEMM_BIG_WM1 4  // waves along the activation rows of a 256-wide tile
#endif
#ifndef MEDUSA_GEMM_BIG_WN1
#define MEDUSA_GEMM_BIG_WN1 4  // waves along the weight rows of a 256-wide tile
#endif
#ifndef MEDUSA_GEMM_BIG_R1
#define MEDUSA_GEMM_BIG_R1 2
#endif
#ifndef MEDUSA_GEMM_BIG_BK2
#define MEDUSA_GEMM_BIG_BK2 64
#endif
#ifndef MEDUSA_GEMM_BIG_R2
#define MEDUSA_GEMM_BIG_R2 3
#endif
#ifndef MEDUSA_GEMM_BIG_R3
#define MEDUSA_GEMM_BIG_R3 3  // stages in the ring of the 128 x 256 tiles (3: -2% with weights cold in HBM)
#endif
#ifndef MEDUSA_GEMM_BIG_WM2
#define MEDUSA_GEMM_BIG_WM2 4  // waves along the activation rows of a 128 x 128 tile (x 2 along the weight rows)
#endif
#ifndef MEDUSA_GEMM_BIG_WM3
#define MEDUSA_GEMM_BIG_WM3 8  // the same for 128 weight rows x 256 activation rows
#endif
#ifndef MEDUSA_GEMM_BIG_WM4
#define MEDUSA_GEMM_BIG_WM4 4  // the same for 192 weight rows x 256 activation rows
#endif
#ifndef MEDUSA_GEMM_BIG_R4
#define MEDUSA_GEMM_BIG_R4 2
#endif
#ifndef MEDUSA_GEMM_BIG_WN4
#define MEDUSA_GEMM_BIG_WN4 2  // waves along the weight rows of a 192-row tile
#endif

GemmPlan gemm_plan(int64_t M, int64_t Kd, int64_t Nw, int dt, int epi) {
  using namespace medusa;
  constexpr int XNB = MEDUSA_GEMM_XL_NB;
  GemmPlan p{false, 1, false, 1, 0, 1, 1, 0};
  const int unit = epi == MEDUSA_EPI_SWIGLU ? 2 : 1;
  // enough rows for the product to be MFMA-bound: the large-row tilings
  if (dt == MEDUSA_BF16 && M >= MEDUSA_GEMM_BIG_MIN_M && Kd % GB_KALIGN == 0 && Nw % (16 * unit) == 0 &&
      Nw <= INT32_MAX / 2) {
    p.big = 1;  // the launch picks the tiling, the batch counted (big_tiling)
    return p;
  }
  const bool narrow = Nw / 16 >= MEDUSA_GEMM_XD_MIN_BLOCKS;
  if (dt == MEDUSA_BF16 && M >= MEDUSA_GEMM_XD_MIN_M && Kd % XB_KC == 0 && Nw % (16 * unit) == 0 &&
      (Nw / 16 >= MEDUSA_GEMM_XB_MIN_BLOCKS || narrow) && Nw / 16 <= (1 << 24)) {
    const int nunits = (int)(Nw / 16 / unit);
    p.xb = true;
    p.xb_unit = unit;
    // a split contraction gives every compute unit's workgroup several blocks
    // (one split per ~8 chunks, at most MEDUSA_GEMM_XD_SPLIT: measured at 64 rows,
    // 4096 x 4096 is fastest split 2 ways and 4096 x 11008 4 ways)
    p.xb_S = Nw / 16 >= MEDUSA_GEMM_XB_MIN_BLOCKS
                 ? 1
                 : (int)std::max<int64_t>(1, std::min<int64_t>(MEDUSA_GEMM_XD_SPLIT, Kd / XB_KC / MEDUSA_GEMM_XD_CPS));
    // about one workgroup per compute unit, at most XB_MAXB blocks each
    p.xb_G = std::max(std::min(MEDUSA_GEMM_XB_WGS / p.xb_S, nunits), (nunits + XB_MAXB / unit - 1) / (XB_MAXB / unit));
    p.MT = (int)((M + (M <= 32 ? 32 : 64) - 1) / (M <= 32 ? 32 : 64));
    return p;
  }
  p.xl = dt == MEDUSA_BF16 && M > 16 && Kd % XL_KC == 0 && Nw >= MEDUSA_GEMM_XL_MIN_N &&
         Nw % (64 * XNB) == 0;
  if (!p.xl) return p;
  // Split the contraction only when the output tiles alone leave the chip
  // under-filled: each workgroup streams about 16-19 GB/s (latency bound), so
  // ~384 of them are needed, while a split costs M*N*4 bytes of partials per
  // share (measured: splitting 172+ tiles is a loss, 32-96 tiles a large win).
  const int64_t tiles = (Nw / (64 * XNB)) * ((M + 63) / 64);
  int64_t ks = 1;
  if (tiles > 0 && tiles < 160) ks = (MEDUSA_GEMM_XL_TARGET_WGS + tiles - 1) / tiles;
  ks = std::min<int64_t>(ks, Kd / XL_KC);
  ks = std::min<int64_t>(ks, 8);
  p.ksplit = (int)std::max<int64_t>(ks, 1);
  return p;
}

// Tiling of the large-row plan for M rows x Nw outputs x batch: 1 = 256 x 256
// tiles (16 waves of 64 x 64), 3 = 128 weight rows x 256 activation rows (16
// waves of 64 x 32), 2 = 128 x 128 (8 waves of 64 x 32).  Four waves per SIMD
// hide the operand reads' latency better than two (at 1024 rows: QKV 114.5
// -> 108 us, gate/up 212 -> 204 us, the heads' W2 stage -2.5%); the 128 x 128
// tiles gain nothing from 16 waves, and with 4 waves the O and down
// projections measured 4-5% slower.  Per unit of work the
// 256-wide tiles are the fastest (measured at 1024 rows: ≈ 1.4x the 128 x 256
// tiles and ≈ 1.6x the 128 x 128 ones), so they are taken when their last
// round over the 256 compute units is at least three quarters full or there
// are many rounds; otherwise the 128 x 256 tiles when they fill at least one
// round, else 128 x 128.  At 1024 rows: QKV (-> 12288) 136 -> 112 us with the
// 256-wide tiles, gate/up (-> 2 x 11008) 221 -> 212 us and the five heads' W1
// stage 283 -> 239 us with the 128 x 256 tiles; O and down keep 128 x 128.  All
// three run the contraction in the same order, so the choice changes no bit
// of the result and may count the tiles of every batch element.
int big_tiling(int64_t M, int64_t Nw, int batch) {
#ifdef MEDUSA_GEMM_BIG_FORCE
  return MEDUSA_GEMM_BIG_FORCE;  // one tiling for every shape (to time the tilings against each other)
#endif
  // Estimated time = rounds of tiles over the compute units x the time of
  // one round of that tile shape (a round of partly idle units costs about
  // as much as a full one).  Round costs relative to the 256 x 256 tiles,
  // measured at 1024 rows x 4096 (gate/up, QKV, the heads): 192 x 256: 0.92,
  // 128 x 256: 0.667, 128 x 128: 0.40.  Ties go to the larger tiles.
  constexpr int64_t CUS = 256;
  struct Tiling {
    int id, tn, tm, cost;
  };
  constexpr Tiling cand[4] = {{1, 256, 256, 1000}, {4, 192, 256, 920}, {3, 128, 256, 667}, {2, 128, 128, 400}};
  int best = 1;
  int64_t best_t = -1;
  for (const Tiling& c : cand) {
    const int64_t tiles = ((Nw + c.tn - 1) / c.tn) * ((M + c.tm - 1) / c.tm) * batch;
    const int64_t t = (tiles + CUS - 1) / CUS * c.cost;
    if (best_t < 0 || t < best_t) {
      best = c.id;
      best_t = t;
    }
  }
  return best;
}
size_t gemm_ws_bytes(int64_t M, int64_t Kd, int64_t Nw, int batch, int dt) {
  // the larger of the two plan families (SwiGLU plans in gate/up pairs);
  // only the split-contraction path uses scratch
  size_t need = 0;
  for (int epi : {(int)MEDUSA_EPI_NONE, (int)MEDUSA_EPI_SWIGLU}) {
    const GemmPlan p = gemm_plan(M, Kd, Nw, dt, epi);
    if (!p.xb && p.xl && p.ksplit > 1)
      need = std::max(need, align_up((size_t)batch * p.ksplit * M * Nw * sizeof(float), 256));
    if (p.xb && p.xb_S > 1)
      need = std::max(need, align_up((size_t)batch * p.xb_S * M * Nw * sizeof(float), 256));
  }
  return need;
}
}  // namespace medusa_host

namespace medusa {
// RMSNorm fused behind a residual projection whose contraction is split
struct SplitNorm {
  const void* gain;
  float eps;
  void* out;
};
template <typename T>
static void launch_split_reduce_rmsnorm(const float* part, int ksplit, int64_t M, int64_t Nw, void* Y,
                                        const SplitNorm* norm, hipStream_t st) {
  auto go = [&](auto qb) {
    hipLaunchKernelGGL((split_reduce_rmsnorm_kernel<T, decltype(qb)::value>), dim3((unsigned)M), dim3(256), 0, st,
                       part, ksplit, (int)M, (int)Nw, reinterpret_cast<float*>(Y),
                       reinterpret_cast<const T*>(norm->gain), norm->eps, reinterpret_cast<T*>(norm->out));
  };
  if (ksplit <= 2) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 4>{});
}
// Launches the projection; returns whether `norm` (residual epilogue only)
// was applied, fused into the reduction of a split contraction.
template <typename T, int EPI>
static bool launch_gemm_t(const void* X, int64_t xbs, int64_t M, int64_t Kd, const void* W,
                          int64_t Nw, int batch, const void* bias, const void* aux, void* Y,
                          int y_f32, void* ws, hipStream_t st, const SplitNorm* norm = nullptr) {
  constexpr int NB = (EPI == MEDUSA_EPI_SWIGLU && MEDUSA_GEMM_NB < 2) ? 2 : MEDUSA_GEMM_NB;
  constexpr int KS = MEDUSA_GEMM_KS;
  constexpr int TN = 16 * NB;
  constexpr int XNB = MEDUSA_GEMM_XL_NB;
  constexpr int DT = sizeof(T) == 2 ? MEDUSA_BF16 : MEDUSA_F32;
  medusa_host::GemmPlan plan = medusa_host::gemm_plan(M, Kd, Nw, DT, EPI);
  // A batch that shares its activation rows (xbs == 0) is one projection onto
  // its stacked weights [batch * Nw, Kd].  It is planned that way when each
  // element alone would split the contraction (the heads' first layer at
  // 64 rows: five 4096-wide outputs), so that every compute unit streams
  // whole blocks over the full contraction and no reduce launch follows.
  int64_t Nf = Nw;  // output columns of the launch
  int bf = batch;   // batch elements of the launch
  if ((EPI == MEDUSA_EPI_NONE || EPI == MEDUSA_EPI_BIAS_SILU_RES) && batch > 1 && xbs == 0 && !norm &&
      plan.xb && plan.xb_S > 1 && Nw * batch <= INT32_MAX / 2) {
    const medusa_host::GemmPlan pf = medusa_host::gemm_plan(M, Kd, Nw * batch, DT, EPI);
    if (pf.xb && pf.xb_S == 1) {
      plan = pf;
      Nf = Nw * batch;
      bf = 1;
    }
  }
  if constexpr (sizeof(T) == 2) {  // planned for bf16 only
    if (plan.big) {
      const T* Xt = reinterpret_cast<const T*>(X);
      const T* Wt = reinterpret_cast<const T*>(W);
      const T* Bt = reinterpret_cast<const T*>(bias);
      // Both tilings run the contraction in the same order (64-deep stages,
      // two 32-deep MFMA steps each), so their results are bit-identical and
      // the choice may count the tiles of every batch element.
      const int tiling = medusa_host::big_tiling(M, Nw, batch);
      if (tiling == 1) {
        const int tN = (int)((Nw + 255) / 256), tM = (int)((M + 255) / 256);
        hipLaunchKernelGGL((gemm_big_kernel<256, 256, MEDUSA_GEMM_BIG_WN1, MEDUSA_GEMM_BIG_WM1, MEDUSA_GEMM_BIG_BK1, MEDUSA_GEMM_BIG_R1, EPI, MEDUSA_GEMM_BIG_PRIO>),
                           dim3((unsigned)(tN * tM), (unsigned)batch),
                           dim3(64 * MEDUSA_GEMM_BIG_WN1 * MEDUSA_GEMM_BIG_WM1), 0, st, Xt, xbs, (int)M, (int)Kd, Wt, (int)Nw, Bt, aux, Y, y_f32, tN, tM);
      } else if (tiling == 4) {
        const int tN = (int)((Nw + 191) / 192), tM = (int)((M + 255) / 256);
        hipLaunchKernelGGL((gemm_big_kernel<192, 256, MEDUSA_GEMM_BIG_WN4, MEDUSA_GEMM_BIG_WM4, 64, MEDUSA_GEMM_BIG_R4, EPI, MEDUSA_GEMM_BIG_PRIO>),
                           dim3((unsigned)(tN * tM), (unsigned)batch),
                           dim3(64 * MEDUSA_GEMM_BIG_WN4 * MEDUSA_GEMM_BIG_WM4), 0, st, Xt, xbs, (int)M, (int)Kd, Wt, (int)Nw, Bt, aux, Y, y_f32, tN, tM);
      } else if (tiling == 3) {
        const int tN = (int)((Nw + 127) / 128), tM = (int)((M + 255) / 256);
        hipLaunchKernelGGL((gemm_big_kernel<128, 256, 2, MEDUSA_GEMM_BIG_WM3, 64, MEDUSA_GEMM_BIG_R3, EPI, MEDUSA_GEMM_BIG_PRIO>),
                           dim3((unsigned)(tN * tM), (unsigned)batch),
                           dim3(128 * MEDUSA_GEMM_BIG_WM3), 0, st, Xt, xbs, (int)M, (int)Kd, Wt, (int)Nw, Bt, aux, Y, y_f32, tN, tM);
      } else {
        const int tN = (int)((Nw + 127) / 128), tM = (int)((M + 127) / 128);
        hipLaunchKernelGGL((gemm_big_kernel<128, 128, 2, MEDUSA_GEMM_BIG_WM2, MEDUSA_GEMM_BIG_BK2, MEDUSA_GEMM_BIG_R2, EPI, 0>),
                           dim3((unsigned)(tN * tM), (unsigned)batch),
                           dim3(128 * MEDUSA_GEMM_BIG_WM2), 0, st, Xt, xbs, (int)M, (int)Kd, Wt, (int)Nw, Bt, aux, Y, y_f32, tN, tM);
      }
      return false;
    }
    if (plan.xb) {
      const dim3 grid((unsigned)plan.xb_G, (unsigned)(bf * plan.MT), (unsigned)plan.xb_S);
      const T* Xt = reinterpret_cast<const T*>(X);
      const T* Wt = reinterpret_cast<const T*>(W);
      const T* Bt = reinterpret_cast<const T*>(bias);
      float* part = reinterpret_cast<float*>(ws);
      if (M <= 32)
        hipLaunchKernelGGL((gemm_xdma_kernel<2, MEDUSA_GEMM_XD_WR, EPI>), grid, dim3(64 * XB_WAVES), 0, st, Xt, xbs,
                           (int)M, (int)Kd, Wt, (int)Nf, Bt, aux, Y, y_f32, plan.xb_G, plan.MT, plan.xb_unit, part,
                           (int)Nw, RopeArgs{});
      else
        hipLaunchKernelGGL((gemm_xdma_kernel<4, MEDUSA_GEMM_XD_WR, EPI>), grid, dim3(64 * XB_WAVES), 0, st, Xt, xbs,
                           (int)M, (int)Kd, Wt, (int)Nf, Bt, aux, Y, y_f32, plan.xb_G, plan.MT, plan.xb_unit, part,
                           (int)Nw, RopeArgs{});
      if (plan.xb_S > 1) {
        if (EPI == MEDUSA_EPI_RES_ADD_F32 && norm) {
          launch_split_reduce_rmsnorm<T>(part, plan.xb_S, M, Nw, Y, norm, st);
          return true;
        }
        const int64_t cols = EPI == MEDUSA_EPI_SWIGLU ? Nw / 2 : Nw;
        dim3 rgrid((unsigned)((M * cols + 255) / 256), (unsigned)batch);
        hipLaunchKernelGGL((gemm_split_reduce_kernel<T, EPI>), rgrid, dim3(256), 0, st, part, plan.xb_S,
                           (int)M, (int)Nw, xbs, Bt, aux, Y, y_f32);
      }
      return false;
    }
  }
  bool normed = false;
  auto go = [&](auto mbc) {
    constexpr int MB = decltype(mbc)::value;
    const unsigned gy = (unsigned)((M + 16 * MB - 1) / (16 * MB));
    if (plan.xl) {
      dim3 grid((unsigned)(Nw / (64 * XNB)), gy, (unsigned)(batch * plan.ksplit));
      hipLaunchKernelGGL((gemm_xlds_kernel<T, MB, XNB, EPI>), grid, dim3(256), 0, st,
                         reinterpret_cast<const T*>(X), xbs, (int)M, (int)Kd,
                         reinterpret_cast<const T*>(W), (int)Nw, reinterpret_cast<const T*>(bias),
                         aux, Y, y_f32, plan.ksplit, reinterpret_cast<float*>(ws));
      if (plan.ksplit > 1 && EPI == MEDUSA_EPI_RES_ADD_F32 && norm) {
        launch_split_reduce_rmsnorm<T>(reinterpret_cast<const float*>(ws), plan.ksplit, M, Nw, Y, norm, st);
        normed = true;
      } else if (plan.ksplit > 1) {
        const int64_t cols = EPI == MEDUSA_EPI_SWIGLU ? Nw / 2 : Nw;
        dim3 rgrid((unsigned)((M * cols + 255) / 256), (unsigned)batch);
        hipLaunchKernelGGL((gemm_split_reduce_kernel<T, EPI>), rgrid, dim3(256), 0, st,
                           reinterpret_cast<const float*>(ws), plan.ksplit, (int)M, (int)Nw, xbs,
                           reinterpret_cast<const T*>(bias), aux, Y, y_f32);
      }
      return;
    }
    dim3 grid((unsigned)((Nw + TN - 1) / TN), gy, (unsigned)batch);
    hipLaunchKernelGGL((gemm_kernel<T, MB, NB, KS, EPI>), grid, dim3(64 * KS), 0, st,
                       reinterpret_cast<const T*>(X), xbs, (int)M, (int)Kd,
                       reinterpret_cast<const T*>(W), (int)Nw, reinterpret_cast<const T*>(bias),
                       aux, Y, y_f32);
  };
  if (M <= 16) go(std::integral_constant<int, 1>());
  else if (M <= 32) go(std::integral_constant<int, 2>());
  else go(std::integral_constant<int, 4>());
  return normed;
}

}  // namespace medusa

namespace medusa_host {
// Internal launcher shared with medusa_heads (arguments already validated).
void launch_gemm(const void* X, int64_t xbs, int64_t M, int64_t Kd, const void* W, int64_t Nw,
                 int batch, int dt, int epi, const void* bias, const void* aux, void* Y,
                 int y_f32, void* ws, hipStream_t st) {
  using namespace medusa;
#define MEDUSA_GEMM_CASE(T, E)                                                              \
  launch_gemm_t<T, E>(X, xbs, M, Kd, W, Nw, batch, bias, aux, Y, y_f32, ws, st)
#define MEDUSA_GEMM_EPI(T)                                                                  \
  switch (epi) {                                                                            \
    case MEDUSA_EPI_NONE: MEDUSA_GEMM_CASE(T, MEDUSA_EPI_NONE); break;                      \
    case MEDUSA_EPI_BIAS_SILU_RES: MEDUSA_GEMM_CASE(T, MEDUSA_EPI_BIAS_SILU_RES); break;    \
    case MEDUSA_EPI_RES_ADD_F32: MEDUSA_GEMM_CASE(T, MEDUSA_EPI_RES_ADD_F32); break;        \
    default: MEDUSA_GEMM_CASE(T, MEDUSA_EPI_SWIGLU); break;                                 \
  }
  if (dt == MEDUSA_BF16) { MEDUSA_GEMM_EPI(bf16_t) } else { MEDUSA_GEMM_EPI(float) }
#undef MEDUSA_GEMM_EPI
#undef MEDUSA_GEMM_CASE
}
}  // namespace medusa_host

extern "C" size_t medusa_linear_ws(int64_t M, int64_t Kd, int64_t N, int32_t batch, int32_t dt) {
  // shapes medusa_linear rejects need nothing (and stay out of the planner's arithmetic)
  if (M <= 0 || Kd <= 0 || N <= 0 || batch <= 0) return 0;
  if (M > INT32_MAX || Kd > INT32_MAX || N > INT32_MAX || (dt != MEDUSA_F32 && dt != MEDUSA_BF16))
    return 0;
  return medusa_host::gemm_ws_bytes(M, Kd, N, batch, dt);
}

extern "C" int32_t medusa_linear(const void* X, int64_t x_bstride, int64_t M, int64_t Kd,
                                 const void* W, int64_t N, int32_t batch, int32_t dt,
                                 int32_t epilogue, const void* bias, const void* aux, void* Y,
                                 int32_t y_f32, void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear: unknown dtype %d", dt);
  MEDUSA_REQUIRE(epilogue >= MEDUSA_EPI_NONE && epilogue <= MEDUSA_EPI_SWIGLU,
                 MEDUSA_ERR_INVALID_ARG, "medusa_linear: unknown epilogue %d", epilogue);
  MEDUSA_REQUIRE(M >= 0 && Kd > 0 && N > 0 && batch >= 1 && x_bstride >= 0,
                 MEDUSA_ERR_INVALID_ARG, "medusa_linear: bad sizes M=%lld Kd=%lld N=%lld batch=%d",
                 (long long)M, (long long)Kd, (long long)N, batch);
  MEDUSA_REQUIRE(M <= INT32_MAX && Kd <= INT32_MAX && N <= INT32_MAX, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear: sizes above 2^31");
  const int p16 = dt == MEDUSA_BF16 ? 8 : 4;
  MEDUSA_REQUIRE(Kd % p16 == 0 && x_bstride % p16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear: Kd and x_bstride must be multiples of %d", p16);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(X && W && Y, MEDUSA_ERR_INVALID_ARG, "medusa_linear: NULL X, W or Y");
  MEDUSA_REQUIRE(((uintptr_t)X | (uintptr_t)W | (uintptr_t)Y | (uintptr_t)aux | (uintptr_t)bias) % 16 == 0,
                 MEDUSA_ERR_INVALID_ARG, "medusa_linear: X, W, Y, aux and bias must be 16-byte aligned");
  if (epilogue == MEDUSA_EPI_BIAS_SILU_RES)
    MEDUSA_REQUIRE(aux != NULL, MEDUSA_ERR_INVALID_ARG, "medusa_linear: residual (aux) is NULL");
  if (epilogue == MEDUSA_EPI_RES_ADD_F32)
    MEDUSA_REQUIRE(aux != NULL && batch == 1, MEDUSA_ERR_INVALID_ARG,
                   "medusa_linear: residual add needs aux and batch == 1");
  if (epilogue == MEDUSA_EPI_SWIGLU)
    MEDUSA_REQUIRE(N % 32 == 0, MEDUSA_ERR_INVALID_ARG,
                   "medusa_linear: SwiGLU needs N (gate+up rows) to be a multiple of 32");
  const size_t need = gemm_ws_bytes(M, Kd, N, batch, dt);
  MEDUSA_REQUIRE(need == 0 || (ws != NULL && ws_bytes >= need), MEDUSA_ERR_WORKSPACE,
                 "medusa_linear: workspace %zu < %zu bytes", ws_bytes, need);
  launch_gemm(X, x_bstride, M, Kd, W, N, batch, dt, epilogue, bias, aux, Y, y_f32, ws,
              (hipStream_t)stream);
  return check_launch("medusa_linear");
}

extern "C" int32_t medusa_linear_rmsnorm(const void* X, int64_t M, int64_t Kd, const void* W,
                                         int64_t N, int32_t dt, float* x, const void* gain,
                                         float eps, void* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_rmsnorm: unknown dtype %d", dt);
  MEDUSA_REQUIRE(M >= 0 && Kd > 0 && N > 0 && eps >= 0.f, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_rmsnorm: bad sizes M=%lld Kd=%lld N=%lld", (long long)M,
                 (long long)Kd, (long long)N);
  MEDUSA_REQUIRE(M <= INT32_MAX && Kd <= INT32_MAX, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_rmsnorm: sizes above 2^31");
  const int p16 = dt == MEDUSA_BF16 ? 8 : 4;
  MEDUSA_REQUIRE(Kd % p16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_rmsnorm: Kd must be a multiple of %d", p16);
  MEDUSA_REQUIRE(N % 4 == 0 && N <= 4 * 256 * medusa::RMS_V4, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_rmsnorm: N must be a multiple of 4 and at most %d",
                 4 * 256 * medusa::RMS_V4);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(X && W && x && out, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_rmsnorm: NULL X, W, x or out");
  MEDUSA_REQUIRE(((uintptr_t)X | (uintptr_t)W | (uintptr_t)x) % 16 == 0, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_rmsnorm: X, W and x must be 16-byte aligned");
  const int a4 = dt == MEDUSA_BF16 ? 8 : 16;  // four elements of gain and out
  MEDUSA_REQUIRE(((uintptr_t)gain | (uintptr_t)out) % a4 == 0, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_rmsnorm: gain and out must be %d-byte aligned", a4);
  const size_t need = gemm_ws_bytes(M, Kd, N, 1, dt);
  MEDUSA_REQUIRE(need == 0 || (ws != NULL && ws_bytes >= need), MEDUSA_ERR_WORKSPACE,
                 "medusa_linear_rmsnorm: workspace %zu < %zu bytes", ws_bytes, need);
  const medusa::SplitNorm norm{gain, eps, out};
  hipStream_t st = (hipStream_t)stream;
  const bool normed =
      dt == MEDUSA_BF16
          ? medusa::launch_gemm_t<medusa::bf16_t, MEDUSA_EPI_RES_ADD_F32>(X, 0, M, Kd, W, N, 1, nullptr, x, x, 0, ws, st, &norm)
          : medusa::launch_gemm_t<float, MEDUSA_EPI_RES_ADD_F32>(X, 0, M, Kd, W, N, 1, nullptr, x, x, 0, ws, st, &norm);
  if (!normed) {
    const int32_t rc = check_launch("medusa_linear_rmsnorm");
    if (rc != MEDUSA_OK) return rc;
    return medusa_rmsnorm(x, M, N, gain, eps, dt, out, stream);
  }
  return check_launch("medusa_linear_rmsnorm");
}

namespace medusa_host {
void launch_qkv_rope_pairs(const void* qkv, int64_t M, int Hq, int Hkv, int D, const int32_t* pos,
                           double log2_base, int dt, void* q, void* k, void* v, hipStream_t st);
// the fused epilogue runs where the projection takes the unsplit DMA block-range kernel
static bool qkv_rope_fused(int64_t M, int64_t Kd, int64_t N, int dt) {
  const GemmPlan p = gemm_plan(M, Kd, N, dt, MEDUSA_EPI_NONE);
  return dt == MEDUSA_BF16 && p.xb && p.xb_S == 1;
}
}  // namespace medusa_host

extern "C" size_t medusa_linear_qkv_rope_ws(int64_t M, int64_t Kd, int32_t Hq, int32_t Hkv,
                                            int32_t D, int32_t dt) {
  using namespace medusa_host;
  // shapes medusa_linear_qkv_rope rejects need nothing
  if (M <= 0 || Kd <= 0 || Hq <= 0 || Hkv <= 0 || D < 8 || D > 128 || M > INT32_MAX ||
      Kd > INT32_MAX || (dt != MEDUSA_F32 && dt != MEDUSA_BF16))
    return 0;
  const int64_t N = ((int64_t)Hq + 2 * (int64_t)Hkv) * D;
  if (N > INT32_MAX) return 0;
  if (qkv_rope_fused(M, Kd, N, dt)) return 0;
  const size_t es = dt == MEDUSA_BF16 ? 2 : 4;
  return align_up((size_t)M * N * es, 256) + gemm_ws_bytes(M, Kd, N, 1, dt);
}

extern "C" int32_t medusa_linear_qkv_rope(const void* X, int64_t M, int64_t Kd, const void* W,
                                          int32_t Hq, int32_t Hkv, int32_t D, const int32_t* pos,
                                          float base, int32_t dt, void* q, void* k, void* v,
                                          void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_qkv_rope: unknown dtype %d", dt);
  MEDUSA_REQUIRE(M >= 0 && Kd > 0 && M <= INT32_MAX && Kd <= INT32_MAX && Hq >= 1 && Hkv >= 1 &&
                     base > 1.f,
                 MEDUSA_ERR_INVALID_ARG, "medusa_linear_qkv_rope: bad sizes or base");
  MEDUSA_REQUIRE(D >= 8 && D <= 128 && D % 8 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_qkv_rope: head dim %d (multiple of 8 up to 128)", D);
  const int p16 = dt == MEDUSA_BF16 ? 8 : 4;
  MEDUSA_REQUIRE(Kd % p16 == 0, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_qkv_rope: Kd must be a multiple of %d", p16);
  if (M == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(X && W && pos && q && k && v, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_qkv_rope: NULL pointer");
  MEDUSA_REQUIRE(((uintptr_t)X | (uintptr_t)W | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) % 16 == 0,
                 MEDUSA_ERR_INVALID_ARG, "medusa_linear_qkv_rope: X, W, q, k and v must be 16-byte aligned");
  const int64_t N = ((int64_t)Hq + 2 * (int64_t)Hkv) * D;
  MEDUSA_REQUIRE(N <= INT32_MAX, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_linear_qkv_rope: (Hq + 2 Hkv) D = %lld above 2^31 - 1", (long long)N);
  const size_t need = medusa_linear_qkv_rope_ws(M, Kd, Hq, Hkv, D, dt);
  MEDUSA_REQUIRE(need == 0 || (ws != NULL && ws_bytes >= need), MEDUSA_ERR_WORKSPACE,
                 "medusa_linear_qkv_rope: workspace %zu < %zu bytes", ws_bytes, need);
  MEDUSA_REQUIRE(need == 0 || (uintptr_t)ws % 256 == 0, MEDUSA_ERR_INVALID_ARG,
                 "medusa_linear_qkv_rope: ws must be 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  const double lb = log2((double)base);
  if (qkv_rope_fused(M, Kd, N, dt)) {
    using namespace medusa;
    const GemmPlan plan = gemm_plan(M, Kd, N, dt, MEDUSA_EPI_NONE);
    const dim3 grid((unsigned)plan.xb_G, (unsigned)plan.MT, 1u);
    const RopeArgs ra{pos, lb, Hq, Hkv, D, (bf16_t*)q, (bf16_t*)k, (bf16_t*)v};
    const bf16_t* Xt = (const bf16_t*)X;
    const bf16_t* Wt = (const bf16_t*)W;
    if (M <= 32)
      hipLaunchKernelGGL((gemm_xdma_kernel<2, MEDUSA_GEMM_XD_WR, EPI_ROPE_QKV>), grid, dim3(64 * XB_WAVES), 0, st,
                         Xt, (int64_t)0, (int)M, (int)Kd, Wt, (int)N, (const bf16_t*)nullptr, nullptr, nullptr, 0,
                         plan.xb_G, plan.MT, 1, (float*)nullptr, (int)N, ra);
    else
      hipLaunchKernelGGL((gemm_xdma_kernel<4, MEDUSA_GEMM_XD_WR, EPI_ROPE_QKV>), grid, dim3(64 * XB_WAVES), 0, st,
                         Xt, (int64_t)0, (int)M, (int)Kd, Wt, (int)N, (const bf16_t*)nullptr, nullptr, nullptr, 0,
                         plan.xb_G, plan.MT, 1, (float*)nullptr, (int)N, ra);
    return check_launch("medusa_linear_qkv_rope");
  }
  // projection into scratch (pair layout), then the rotary pass over it
  const size_t es = dt == MEDUSA_BF16 ? 2 : 4;
  char* qkv = (char*)ws;
  void* gws = qkv + align_up((size_t)M * N * es, 256);
  launch_gemm(X, 0, M, Kd, W, N, 1, dt, MEDUSA_EPI_NONE, nullptr, nullptr, qkv, 0, gws, st);
  launch_qkv_rope_pairs(qkv, M, Hq, Hkv, D, pos, lb, dt, q, k, v, st);
  return check_launch("medusa_linear_qkv_rope");
}
