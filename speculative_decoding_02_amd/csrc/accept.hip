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

__global__ __launch_bounds__(64) void accept_sweep_kernel(
    const float* __restrict__ logits, int64_t V, const int* __restrict__ tokens,
    const int* __restrict__ parent, int N, int K, int typical, float inv_t, float epsilon,
    float delta, const RowStats* __restrict__ stats, int* __restrict__ accept_len,
    int* __restrict__ path, int* __restrict__ next_token) {
  const int b = blockIdx.x, i = threadIdx.x;
  const int64_t base = (int64_t)b * N;
  bool ok = false;
  if (i >= 1 && i < N) {
    const int p = parent[base + i];
    const RowStats rp = stats[base + p];
    const int tok = tokens[base + i];
    if (!typical) {
      ok = tok == rp.argmax;
    } else {
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
  next_token[b] = stats[base + best].argmax;
}

}  // namespace medusa

extern "C" size_t medusa_accept_ws(int32_t B, int32_t N) {
  if (B < 0 || N < 0) return 0;
  return medusa_host::align_up((size_t)B * N * sizeof(medusa::RowStats), 256);
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
                     next_token);
  return check_launch("medusa_accept");
}
