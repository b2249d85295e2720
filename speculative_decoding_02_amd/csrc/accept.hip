// medusa_accept: the longest branch the model accepts ("Medusa Heads",
// section "Attenzione sull'albero e accettazione": greedy decoding keeps a
// candidate equal to the model's top choice; typical acceptance keeps one
// whose base-model probability exceeds a threshold tied to the entropy; the
// longest accepted branch is kept).
//
// Kernel 1, one workgroup per (node, sequence): a coalesced sweep of the
// node's logits row gives argmax (lowest id on ties) and, in typical mode,
// the softmax statistics max m, log-sum log(s) and entropy H of z / T.
// Kernel 2, one wave per sequence: lane i decides whether node i passes its
// parent's test; a ballot gives the pass mask and one lane sweeps the tree in
// index order (parents precede children) to AND it along every branch.
//
// medusa_accept_sample: sampled verification, the rejection sampling against
// the base model that keeps Medusa-1 lossless ("Têtes de décodage Medusa",
// section "Plongée profonde" and its "Questions fréquemment posées" entry on
// lossless acceleration).  The candidates are fixed top-k tokens, so
// rejection-testing them one by one against p (renormalised over the tokens
// not yet rejected) selects child c with probability p(token c) and otherwise
// ends the branch with a draw from the rest: the law of one draw z ~ p per
// visited node, following the child whose token is z.  Kernel 1 (sampling
// variant) draws z for every node at once by Gumbel-max: argmax over v of
// z_v / T + G_v, G_v = -log(-log(u_v)), u_v from Philox4x64-10 (Salmon et
// al., SC 2011) with key (seed, step) and counter (v / 4, node, b, 0), word
// v % 4, u = (top 23 bits + 1/2) / 2^23.  Kernel 2 is the greedy sweep with
// the draws in place of the argmax, and advances the step counter.
#include <algorithm>

#include "common.h"

namespace medusa {

struct RowStats {
  int argmax;
  float m;      // max of z/T
  float logs;   // log sum exp(z/T - m)
  float ent;    // natural-log entropy of softmax(z/T)
};

__device__ __forceinline__ void arg_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

__global__ __launch_bounds__(256) void accept_stats_kernel(const float* __restrict__ logits,
                                                           int64_t V, int N, int typical,
                                                           float inv_t,
                                                           RowStats* __restrict__ stats) {
  const int n = blockIdx.x, b = blockIdx.y;
  const float* z = logits + ((int64_t)b * N + n) * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ float s2[4], s3[4];

  float bv = -INFINITY;
  int bi = 0x7fffffff;
  // 16-byte loads, four in flight per thread before any comparison
  const bool vec = (V % 4 == 0) && (((uintptr_t)z) % 16 == 0);
  const int64_t V4 = vec ? V / 4 : 0;
  for (int64_t e0 = tid; e0 < V4; e0 += 4 * 256) {
    f32x4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = min(e0 + u * 256, V4 - 1);
      q[u] = reinterpret_cast<const f32x4*>(z)[e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e0 + u * 256 < V4)
#pragma unroll
        for (int r = 0; r < 4; ++r) arg_better(bv, bi, q[u][r], (int)((e0 + u * 256) * 4 + r));
  }
  for (int64_t e = V4 * 4 + tid; e < V; e += 256) arg_better(bv, bi, z[e], (int)e);
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    arg_better(bv, bi, ov, oi);
  }
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  for (int w = 1; w < 4; ++w) arg_better(bv, bi, sv[w], si[w]);

  RowStats rs;
  rs.argmax = bi;
  rs.m = bv * inv_t;
  rs.logs = 0.f;
  rs.ent = 0.f;
  if (typical) {
    // m = max(z/T) = max(z)/T for T > 0
    const float m = rs.m;
    float s = 0.f, e1 = 0.f;
    for (int64_t e0 = tid; e0 < V4; e0 += 4 * 256) {
      f32x4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = reinterpret_cast<const f32x4*>(z)[min(e0 + u * 256, V4 - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * 256 < V4)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float y = q[u][r] * inv_t - m;
            const float p = expf(y);
            s += p;
            e1 += p * y;
          }
    }
    for (int64_t e = V4 * 4 + tid; e < V; e += 256) {
      const float y = z[e] * inv_t - m;
      const float p = expf(y);
      s += p;
      e1 += p * y;
    }
    s = wave_sum(s);
    e1 = wave_sum(e1);
    if (lane == 0) { s2[wave] = s; s3[wave] = e1; }
    __syncthreads();
    s = (s2[0] + s2[1]) + (s2[2] + s2[3]);
    e1 = (s3[0] + s3[1]) + (s3[2] + s3[3]);
    rs.logs = logf(s);
    rs.ent = rs.logs - e1 / s;  // H = log s - sum(p*y)/s with y = z/T - m
  }
  if (tid == 0) stats[(int64_t)b * N + n] = rs;
}

// ---- counter-based generator: Philox4x64 with 10 rounds ----
struct U64x4 {
  uint64_t w[4];
};
__device__ __forceinline__ U64x4 philox4x64_10(U64x4 c, uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;  // round multipliers
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;  // key increments
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(M0, c.w[0]), lo0 = M0 * c.w[0];
    const uint64_t hi1 = __umul64hi(M1, c.w[2]), lo1 = M1 * c.w[2];
    c = U64x4{{hi1 ^ c.w[1] ^ k0, lo1, hi0 ^ c.w[3] ^ k1, lo0}};
    k0 += W0;
    k1 += W1;
  }
  return c;
}
// Gumbel-max score of one vocabulary entry: z / T + G, rounded after the
// product and after the sum (no fused multiply-add).
__device__ __forceinline__ float gumbel_score(float z, float inv_t, uint64_t w) {
  const float u = ((float)(uint32_t)(w >> 41) + 0.5f) * 0x1p-23f;  // exact, in (0, 1)
  const float g = -logf(-logf(u));
  return __fadd_rn(__fmul_rn(z, inv_t), g);
}

// Draws from softmax(z / T), one per (node, sequence) row: split `s` of the
// row's S contiguous ranges of 4-entry blocks finds its Gumbel-max
// (score, entry) (lowest entry on a tie); the sweep kernel takes the best of
// the S partials.  One generator block serves 4 entries; the row is split so
// that the grid covers the chip (the 64-bit multiplies of the generator make
// this the costly part).
struct Draw {
  float score;
  int idx;
};
__global__ __launch_bounds__(256) void accept_draw_kernel(const float* __restrict__ logits,
                                                          int64_t V, int N, float inv_t,
                                                          const uint64_t* __restrict__ rng,
                                                          Draw* __restrict__ part) {
  const int n = blockIdx.x, b = blockIdx.y, sp = blockIdx.z, S = gridDim.z;
  const float* z = logits + ((int64_t)b * N + n) * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sv[4];
  __shared__ int si[4];
  const uint64_t seed = rng[0], step = rng[1];

  const int64_t nblk = (V + 3) / 4;
  const int64_t e0 = nblk * sp / S, e1 = nblk * (sp + 1) / S;
  const bool vec = (V % 4 == 0) && (((uintptr_t)z) % 16 == 0);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int64_t e = e0 + tid; e < e1; e += 256) {
    f32x4 q;
    if (vec) {
      q = reinterpret_cast<const f32x4*>(z)[e];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) q[r] = z[min(e * 4 + r, V - 1)];
    }
    const U64x4 w = philox4x64_10(U64x4{{(uint64_t)e, (uint64_t)n, (uint64_t)b, 0ull}}, seed, step);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e * 4 + r < V) arg_better(bv, bi, gumbel_score(q[r], inv_t, w.w[r]), (int)(e * 4 + r));
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    arg_better(bv, bi, ov, oi);
  }
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    bv = sv[0];
    bi = si[0];
    for (int w = 1; w < 4; ++w) arg_better(bv, bi, sv[w], si[w]);
    part[((int64_t)b * N + n) * S + sp] = Draw{bv, bi};
  }
}

__global__ __launch_bounds__(64) void accept_sweep_kernel(
    const float* __restrict__ logits, int64_t V, const int* __restrict__ tokens,
    const int* __restrict__ parent, int N, int K, int typical, float inv_t, float epsilon,
    float delta, const RowStats* __restrict__ stats, int* __restrict__ accept_len,
    int* __restrict__ path, int* __restrict__ next_token, const Draw* __restrict__ draws,
    int S, uint64_t* __restrict__ rng) {
  const int b = blockIdx.x, i = threadIdx.x;
  const int64_t base = (int64_t)b * N;
  // sampled mode: node i's draw = the best of its S partials
  __shared__ int zs[MEDUSA_MAX_NODES];
  if (draws != nullptr) {
    if (i < N) {
      Draw d = draws[(base + i) * S];
      for (int q = 1; q < S; ++q) {
        const Draw o = draws[(base + i) * S + q];
        arg_better(d.score, d.idx, o.score, o.idx);
      }
      zs[i] = d.idx;
    }
    __syncthreads();
  }
  bool ok = false;
  if (i >= 1 && i < N) {
    const int p = parent[base + i];
    const int tok = tokens[base + i];
    if (draws != nullptr) {
      ok = tok == zs[p];
    } else if (!typical) {
      ok = tok == stats[base + p].argmax;
    } else {
      const RowStats rp = stats[base + p];
      const float lp = logits[(base + p) * V + tok] * inv_t - rp.m - rp.logs;
      const float thr = fminf(epsilon, delta * expf(-rp.ent));
      ok = expf(lp) > thr;
    }
  }
  const uint64_t pass = __ballot(ok);
  __shared__ int depth[MEDUSA_MAX_NODES];
  if (i != 0) return;
  uint64_t acc = 1ull;
  depth[0] = 0;
  int best = 0;
  for (int j = 1; j < N; ++j) {
    const int p = parent[base + j];
    depth[j] = depth[p] + 1;
    if (((acc >> p) & 1ull) && ((pass >> j) & 1ull)) {
      acc |= 1ull << j;
      if (depth[j] > depth[best]) best = j;
    }
  }
  const int a = depth[best];
  accept_len[b] = a;
  int* pth = path + (int64_t)b * (K + 1);
  for (int d = a + 1; d <= K; ++d) pth[d] = -1;
  int j = best;
  for (int d = a; d >= 0; --d) {  // depth <= K for validated templates
    if (d <= K) pth[d] = j;
    j = parent[base + j];
  }
  next_token[b] = draws != nullptr ? zs[best] : stats[base + best].argmax;
  // sampled mode: the next call draws with fresh noise (every sequence's draw
  // kernel has read the step before any sweep runs: stream order)
  if (rng != nullptr && b == 0) rng[1] += 1;
}

}  // namespace medusa

namespace {
// splits of a row for the sampled draws: enough workgroups for the chip
// (about 512), at least 1024 vocabulary entries each, at most 16
int draw_splits(int B, int N, int64_t V) {
  int s = (512 + B * N - 1) / (B * N);
  s = std::min<int64_t>(s, std::max<int64_t>(V / 1024, 1));
  return std::max(1, std::min(s, 16));
}
}  // namespace

extern "C" size_t medusa_accept_ws(int32_t B, int32_t N) {
  if (B < 0 || N < 0) return 0;
  // greedy / typical row statistics, or up to 16 sampled partials per row
  return medusa_host::align_up((size_t)B * N * std::max(sizeof(medusa::RowStats),
                                                        16 * sizeof(medusa::Draw)), 256);
}

extern "C" int32_t medusa_accept(const float* logits, int64_t V, const int32_t* tokens,
                                 const int32_t* parent, int32_t B, int32_t N, int32_t K,
                                 int32_t mode, float temperature, float epsilon, float delta,
                                 int32_t* accept_len, int32_t* path, int32_t* next_token,
                                 void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(V >= 1 && V <= INT32_MAX, MEDUSA_ERR_INVALID_ARG, "medusa_accept: bad V");
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_accept: B=%d N=%d (N must be in [1, 64])", B, N);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_NODES - 1, MEDUSA_ERR_INVALID_ARG,
                 "medusa_accept: K=%d", K);
  MEDUSA_REQUIRE(mode == 0 || mode == 1, MEDUSA_ERR_INVALID_ARG,
                 "medusa_accept: mode %d (0 greedy, 1 typical)", mode);
  if (mode == 1)
    MEDUSA_REQUIRE(temperature > 0.f && epsilon >= 0.f && delta >= 0.f, MEDUSA_ERR_INVALID_ARG,
                   "medusa_accept: typical needs temperature > 0, epsilon >= 0, delta >= 0");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && tokens && parent && accept_len && path && next_token,
                 MEDUSA_ERR_INVALID_ARG, "medusa_accept: NULL pointer");
  const size_t need = medusa_accept_ws(B, N);
  MEDUSA_REQUIRE(ws != NULL && ws_bytes >= need, MEDUSA_ERR_WORKSPACE,
                 "medusa_accept: workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const float inv_t = mode == 1 ? 1.f / temperature : 1.f;
  medusa::RowStats* stats = (medusa::RowStats*)ws;
  hipLaunchKernelGGL(medusa::accept_stats_kernel, dim3(N, B), dim3(256), 0, st, logits, V, N,
                     mode, inv_t, stats);
  hipLaunchKernelGGL(medusa::accept_sweep_kernel, dim3(B), dim3(64), 0, st, logits, V, tokens,
                     parent, N, K, mode, inv_t, epsilon, delta, stats, accept_len, path,
                     next_token, (const medusa::Draw*)nullptr, 0, (uint64_t*)nullptr);
  return check_launch("medusa_accept");
}

extern "C" int32_t medusa_accept_sample(const float* logits, int64_t V, const int32_t* tokens,
                                        const int32_t* parent, int32_t B, int32_t N, int32_t K,
                                        float temperature, uint64_t* rng, int32_t* accept_len,
                                        int32_t* path, int32_t* next_token, void* ws,
                                        size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(V >= 1 && V <= INT32_MAX, MEDUSA_ERR_INVALID_ARG, "medusa_accept_sample: bad V");
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_UNSUPPORTED,
                 "medusa_accept_sample: B=%d N=%d (N must be in [1, 64])", B, N);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_NODES - 1, MEDUSA_ERR_INVALID_ARG,
                 "medusa_accept_sample: K=%d", K);
  MEDUSA_REQUIRE(temperature > 0.f && temperature < 1e30f, MEDUSA_ERR_INVALID_ARG,
                 "medusa_accept_sample: temperature must be positive and finite");
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && tokens && parent && rng && accept_len && path && next_token,
                 MEDUSA_ERR_INVALID_ARG, "medusa_accept_sample: NULL pointer");
  MEDUSA_REQUIRE((uintptr_t)rng % 8 == 0, MEDUSA_ERR_INVALID_ARG,
                 "medusa_accept_sample: rng must be 8-byte aligned");
  const size_t need = medusa_accept_ws(B, N);
  MEDUSA_REQUIRE(ws != NULL && ws_bytes >= need, MEDUSA_ERR_WORKSPACE,
                 "medusa_accept_sample: workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  const float inv_t = 1.f / temperature;
  medusa::Draw* draws = (medusa::Draw*)ws;
  const int S = draw_splits(B, N, V);
  hipLaunchKernelGGL(medusa::accept_draw_kernel, dim3(N, B, S), dim3(256), 0, st, logits, V, N,
                     inv_t, rng, draws);
  hipLaunchKernelGGL(medusa::accept_sweep_kernel, dim3(B), dim3(64), 0, st, logits, V, tokens,
                     parent, N, K, 0, inv_t, 0.f, 0.f, (const medusa::RowStats*)nullptr,
                     accept_len, path, next_token, draws, S, rng);
  return check_launch("medusa_accept_sample");
}
