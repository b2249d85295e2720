// medusa_accept: the longest branch the model accepts ("Medusa Heads",
// section "Attenzione sull'albero e accettazione": greedy decoding keeps a
// candidate equal to the model's top choice; typical acceptance keeps one
// whose base-model probability exceeds a threshold tied to the entropy; the
// longest accepted branch is kept).
//
// Kernel 1, S workgroups per (node, sequence), each over a contiguous range
// of the node's logits row: the range's argmax (lowest id on ties) and, in
// typical mode, its softmax partial sums relative to its own maximum.
// Kernel 2, one wave per sequence: lane i merges node i's S partials (max m,
// log-sum log(s) and entropy H of z / T), decides whether node i passes its
// parent's test (the parent's statistics come by lane shuffle), and the
// accepted set follows from the pass mask and the nodes' ancestor masks.
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

__device__ __forceinline__ void arg_better(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}

// Statistics of one range of a logits row: its maximum z and where it is
// (lowest index on a tie) and, in typical mode, with y = z / T - v / T:
// s = sum of exp(y), e = sum of exp(y) * y over the range.
struct StatPart {
  float v;
  int i;
  float s;
  float e;
};

// Splits of a row: enough workgroups for the chip (about 512), at least 1024
// vocabulary entries each, at most 16.
__host__ __device__ inline int row_splits(int B, int N, int64_t V) {
  int s = (512 + B * N - 1) / (B * N);
  s = (int)(s < V / 1024 ? s : V / 1024);
  return s < 1 ? 1 : (s > 16 ? 16 : s);
}

__global__ __launch_bounds__(256) void accept_stats_kernel(const float* __restrict__ logits,
                                                           int64_t V, int N, int typical,
                                                           float inv_t,
                                                           StatPart* __restrict__ part) {
  const int n = blockIdx.x, b = blockIdx.y, sp = blockIdx.z, S = gridDim.z;
  const float* z = logits + ((int64_t)b * N + n) * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sv[4], s2[4], s3[4];
  __shared__ int si[4];
  // blocks of 4 entries; this split's range [e0, e1)
  const int64_t nblk = (V + 3) / 4;
  const int64_t e0 = nblk * sp / S, e1 = nblk * (sp + 1) / S;
  const bool vec = (V % 4 == 0) && (((uintptr_t)z) % 16 == 0);
  auto load = [&](int64_t e) -> f32x4 {
    f32x4 q;
    if (vec) {
      q = reinterpret_cast<const f32x4*>(z)[e];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) q[r] = z[min(e * 4 + r, V - 1)];
    }
    return q;
  };
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int64_t e = e0 + tid; e < e1; e += 256) {
    const f32x4 q = load(e);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e * 4 + r < V) arg_better(bv, bi, q[r], (int)(e * 4 + r));
  }
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
  StatPart ps{bv, bi, 0.f, 0.f};
  if (typical) {
    const float m = bv * inv_t;  // max of z / T over the range, T > 0
    float sm = 0.f, e1s = 0.f;
    for (int64_t e = e0 + tid; e < e1; e += 256) {
      const f32x4 q = load(e);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (e * 4 + r < V) {
          const float y = q[r] * inv_t - m;
          const float p = expf(y);
          sm += p;
          e1s += p * y;
        }
    }
    sm = wave_sum(sm);
    e1s = wave_sum(e1s);
    if (lane == 0) { s2[wave] = sm; s3[wave] = e1s; }
    __syncthreads();
    ps.s = (s2[0] + s2[1]) + (s2[2] + s2[3]);
    ps.e = (s3[0] + s3[1]) + (s3[2] + s3[3]);
  }
  if (tid == 0) part[((int64_t)b * N + n) * S + sp] = ps;
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

// The accepted branch of sequence b, decided by one wave (lane i = node i).
// Lane i first merges node i's S row partials: its draw (sampled), or its
// argmax and, in typical mode, max m, log-sum log(s) and entropy H of z / T.
// Node i passes when its token is its parent's choice (argmax, the typical
// threshold, or the parent's draw); the parent's values come by shuffle.  A
// node is accepted when it and every ancestor below the root pass: its
// ancestor-or-self mask, built by walking the parent links through lane
// shuffles (one step per tree level), must lie inside the pass mask.  The
// kept node is the deepest accepted one, the lowest index among equally deep
// ones; the path is read off its ancestor mask (the ancestor at depth d sits
// at path[d]).  Lanes write path[0..K] (-1 past the kept depth) to `pth`
// (global or LDS).
struct Sweep {
  int a;     // accept length (depth of the kept node)
  int best;  // kept node
  int next;  // next root token
};
__device__ __forceinline__ Sweep wave_sweep(int b, int lane, const float* __restrict__ logits,
                                            int64_t V, const int* __restrict__ tokens,
                                            const int* __restrict__ parent, int N, int K,
                                            int typical, float inv_t, float epsilon, float delta,
                                            const StatPart* __restrict__ stats,
                                            const Draw* __restrict__ draws, int S, int* pth) {
  const int64_t base = (int64_t)b * N;
  const bool live = lane < N;
  const int par = live ? min(parent[base + lane], MEDUSA_MAX_NODES - 1) : -1;
  const int tok = live ? tokens[base + lane] : 0;
  // node lane's choice z (draw or argmax) and, typical, its softmax statistics
  int z = 0;
  float m = 0.f, logs = 0.f, ent = 0.f;
  if (draws != nullptr) {
    if (live) {
      Draw d = draws[(base + lane) * S];
      for (int q = 1; q < S; ++q) {
        const Draw o = draws[(base + lane) * S + q];
        arg_better(d.score, d.idx, o.score, o.idx);
      }
      z = d.idx;
    }
  } else if (live) {
    const StatPart* ps = stats + (base + lane) * S;
    float bv = ps[0].v;
    int bi = ps[0].i;
    for (int q = 1; q < S; ++q) arg_better(bv, bi, ps[q].v, ps[q].i);
    z = bi;
    if (typical) {
      m = bv * inv_t;
      float sm = 0.f, e1 = 0.f;
      for (int q = 0; q < S; ++q) {
        const float mq = ps[q].v * inv_t - m;  // <= 0
        const float sc = expf(mq);
        sm += ps[q].s * sc;
        e1 += sc * (ps[q].e + ps[q].s * mq);
      }
      logs = logf(sm);
      ent = logs - e1 / sm;  // H = log s - sum(p*y)/s with y = z/T - m
    }
  }
  const int pp = max(par, 0);
  const int zpar = __shfl(z, pp, 64);
  bool ok = false;
  if (!typical || draws != nullptr) {
    ok = live && lane >= 1 && par >= 0 && tok == zpar;
  } else {
    const float mp = __shfl(m, pp, 64), lsp = __shfl(logs, pp, 64), hp = __shfl(ent, pp, 64);
    if (live && lane >= 1 && par >= 0) {
      const float lp = logits[(base + par) * V + tok] * inv_t - mp - lsp;
      const float thr = fminf(epsilon, delta * expf(-hp));
      ok = expf(lp) > thr;
    }
  }
  const uint64_t pass = __ballot(ok) | 1ull;  // the root is always kept
  uint64_t anc = live ? 1ull << lane : 0ull;
  int j = par;
  for (int it = 0; it < MEDUSA_MAX_NODES && __ballot(j >= 0) != 0; ++it) {
    const int jn = __shfl(par, max(j, 0), 64);
    if (j >= 0) {
      anc |= 1ull << j;
      j = jn;
    }
  }
  const bool accepted = live && (anc & ~pass) == 0ull;
  const int depth = __popcll(anc) - 1;
  int key = accepted ? (depth << 6) | (63 - lane) : -1;
  for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, 64));
  Sweep r;
  r.a = key >> 6;
  r.best = 63 - (key & 63);
  const uint32_t lo = __shfl((uint32_t)anc, r.best, 64);
  const uint32_t hi = __shfl((uint32_t)(anc >> 32), r.best, 64);
  const uint64_t on_path = ((uint64_t)hi << 32) | lo;
  if (((on_path >> lane) & 1ull) && depth <= K) pth[depth] = lane;
  if (lane > r.a && lane <= K) pth[lane] = -1;
  r.next = __shfl(z, r.best, 64);
  return r;
}

__global__ __launch_bounds__(64) void accept_sweep_kernel(
    const float* __restrict__ logits, int64_t V, const int* __restrict__ tokens,
    const int* __restrict__ parent, int N, int K, int typical, float inv_t, float epsilon,
    float delta, const StatPart* __restrict__ stats, int* __restrict__ accept_len,
    int* __restrict__ path, int* __restrict__ next_token, const Draw* __restrict__ draws,
    int S, uint64_t* __restrict__ rng) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const Sweep r = wave_sweep(b, lane, logits, V, tokens, parent, N, K, typical, inv_t, epsilon,
                             delta, stats, draws, S, path + (int64_t)b * (K + 1));
  if (lane != 0) return;
  accept_len[b] = r.a;
  next_token[b] = r.next;
  // sampled mode: the next call draws with fresh noise (every sequence's draw
  // kernel has read the step before any sweep runs: stream order)
  if (rng != nullptr && b == 0) rng[1] += 1;
}

// The tail of a decode step in one launch, after the row partials (or the
// draws): one workgroup per (group of kv heads, layer, sequence).  Wave 0 of
// every workgroup decides its sequence's accepted branch (wave_sweep: the
// same result in every workgroup) while wave 1 stages the page-table entries
// of slots ctx..ctx+N-1; then the workgroup moves its kv heads' kept rows in
// its layer's cache (read all, barrier, write all, as kv_compact).  The
// workgroup of (group 0, layer 0) also writes the accept outputs, the kept
// branch's last hidden state, the next root token and the decode log.  The
// context length is read by every workgroup, so it is advanced by the last
// one to arrive (a per-sequence counter, reset by that workgroup): a
// workgroup arrives only after its read of the length has been used (its
// cache addresses depend on it), so none can read the new value.
struct TailArgs {
  const float* logits;
  int64_t V;
  const int* tokens;
  const int* parent;
  int N, K, typical;
  float inv_t, epsilon, delta;
  const StatPart* stats;
  const Draw* draws;
  int S;
  uint64_t* rng;
  LayerPtrs lp;
  int Hkv, P;
  const int* page_table;
  int max_pages;
  const void* hidden;
  int64_t H;  // elements of a hidden row
  void* h_best;
  int* ctx;
  int* root;
  int* accept_len;
  int* path;
  int* next_token;
  int* log;
  int cap;
  unsigned* arrive;
};

template <int D, int ES>
constexpr int tail_heads() { return 128 / (D * ES / 16); }  // kv heads per workgroup

template <int D, int ES>
__global__ __launch_bounds__(256) void decode_tail_kernel(const TailArgs t) {
  constexpr int CPR = D * ES / 16;  // 16-byte chunks per cache row
  constexpr int G = tail_heads<D, ES>();
  __shared__ uint4 buf[2 * (MEDUSA_MAX_HEADS + 1) * G * CPR];
  __shared__ int s_path[MEDUSA_MAX_NODES];
  __shared__ int s_pt[MEDUSA_MAX_NODES + 1];
  __shared__ int s_a, s_best, s_next, s_n0, s_steps;
  const int HG = (t.Hkv + G - 1) / G;
  const int hg = blockIdx.x % HG, l = blockIdx.x / HG, b = blockIdx.y;
  const int tid = threadIdx.x;
  const bool lead = blockIdx.x == 0;
  const int64_t lrow = (int64_t)b * (2 + 2 * (int64_t)t.cap);
  const int c = t.ctx[b];
  const int pg0 = c / t.P;
  const int npg = (c + t.N - 1) / t.P - pg0 + 1;  // pages of slots c..c+N-1 (<= N+1)
  if (tid < 64) {
    const Sweep r = wave_sweep(b, tid, t.logits, t.V, t.tokens, t.parent, t.N, t.K, t.typical,
                               t.inv_t, t.epsilon, t.delta, t.stats, t.draws, t.S, s_path);
    if (tid == 0) {
      s_a = r.a;
      s_best = r.best;
      s_next = r.next;
    }
  } else if (tid - 64 < npg) {
    s_pt[tid - 64] = t.page_table[(int64_t)b * t.max_pages + min(pg0 + tid - 64, t.max_pages - 1)];
  } else if (lead && tid == 255) {
    s_n0 = t.log[lrow];
    s_steps = t.log[lrow + 1];
  }
  __syncthreads();
  const int a = min(s_a, t.K);

  // the kept rows of this layer's kv heads h0 .. h0+gh-1
  const int h0 = hg * G, gh = min(G, t.Hkv - h0);
  auto row_ptr = [&](char* pool, int h, int slot) -> uint4* {
    const int page = s_pt[slot / t.P - pg0];
    return reinterpret_cast<uint4*>(pool + ((((int64_t)page * t.Hkv + h) * t.P + slot % t.P) * D) * ES);
  };
  char* pools[2] = {(char*)t.lp.k[l], (char*)t.lp.v[l]};
  const int per = (a + 1) * CPR;  // chunks per (pool, head)
  const int items = 2 * gh * per;
  for (int e = tid; e < items; e += 256) {
    const int which = e / (gh * per), rem = e % (gh * per), h = rem / per, r2 = rem % per;
    buf[e] = row_ptr(pools[which], h0 + h, c + s_path[r2 / CPR])[r2 % CPR];
  }
  __syncthreads();
  for (int e = tid; e < items; e += 256) {
    const int which = e / (gh * per), rem = e % (gh * per), h = rem / per, r2 = rem % per;
    const int d = r2 / CPR;
    if (s_path[d] != d) row_ptr(pools[which], h0 + h, c + d)[r2 % CPR] = buf[e];
  }

  if (lead) {
    int* lg = t.log + lrow;
    if (tid <= t.K) t.path[(int64_t)b * (t.K + 1) + tid] = s_path[tid];
    if (tid <= a && s_n0 + tid < t.cap) lg[2 + s_n0 + tid] = t.tokens[(int64_t)b * t.N + s_path[tid]];
    if (tid == 0) {
      t.accept_len[b] = s_a;
      t.next_token[b] = s_next;
      t.root[b] = s_next;
      if (s_steps < t.cap) lg[2 + t.cap + s_steps] = s_a;
      lg[0] = s_n0 + a + 1;
      lg[1] = s_steps + 1;
      if (t.rng != nullptr && b == 0) t.rng[1] += 1;  // fresh noise for the next draws
    }
    const int64_t chunks = t.H * ES / 16;
    const uint4* src = reinterpret_cast<const uint4*>(t.hidden) + ((int64_t)b * t.N + s_best) * chunks;
    uint4* dst = reinterpret_cast<uint4*>(t.h_best) + (int64_t)b * chunks;
    for (int64_t e = tid; e < chunks; e += 256) dst[e] = src[e];
  }
  __syncthreads();
  if (tid == 0) {
    const unsigned total = gridDim.x;
    const unsigned prev = __hip_atomic_fetch_add(t.arrive + b, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == total - 1) {
      t.ctx[b] = c + a + 1;
      __hip_atomic_store(t.arrive + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace medusa

extern "C" size_t medusa_accept_ws(int32_t B, int32_t N) {
  if (B < 0 || N < 0) return 0;
  // up to 16 row partials (statistics or draws) per row
  return medusa_host::align_up((size_t)B * N * 16 * std::max(sizeof(medusa::StatPart),
                                                             sizeof(medusa::Draw)), 256);
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
  medusa::StatPart* stats = (medusa::StatPart*)ws;
  const int S = medusa::row_splits(B, N, V);
  hipLaunchKernelGGL(medusa::accept_stats_kernel, dim3(N, B, S), dim3(256), 0, st, logits, V, N,
                     mode, inv_t, stats);
  hipLaunchKernelGGL(medusa::accept_sweep_kernel, dim3(B), dim3(64), 0, st, logits, V, tokens,
                     parent, N, K, mode, inv_t, epsilon, delta, stats, accept_len, path,
                     next_token, (const medusa::Draw*)nullptr, S, (uint64_t*)nullptr);
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
  const int S = medusa::row_splits(B, N, V);
  hipLaunchKernelGGL(medusa::accept_draw_kernel, dim3(N, B, S), dim3(256), 0, st, logits, V, N,
                     inv_t, rng, draws);
  hipLaunchKernelGGL(medusa::accept_sweep_kernel, dim3(B), dim3(64), 0, st, logits, V, tokens,
                     parent, N, K, 0, inv_t, 0.f, 0.f, (const medusa::StatPart*)nullptr,
                     accept_len, path, next_token, draws, S, rng);
  return check_launch("medusa_accept_sample");
}

// The arrival counters sit after the statistics of the largest tree (N = 64),
// at an offset that depends on B only, so one workspace serves calls of any
// N (the counters of one call are never another call's statistics).
static size_t tail_counter_offset(int32_t B) { return medusa_accept_ws(B, MEDUSA_MAX_NODES); }

extern "C" size_t medusa_decode_tail_ws(int32_t B, int32_t N) {
  if (B < 0 || N < 0) return 0;
  // the accept statistics or draws, then one arrival counter per sequence
  return tail_counter_offset(B) + medusa_host::align_up((size_t)B * sizeof(unsigned), 256);
}

extern "C" int32_t medusa_decode_tail(
    const float* logits, int64_t V, const int32_t* tokens, const int32_t* parent, int32_t B,
    int32_t N, int32_t K, int32_t mode, float temperature, float epsilon, float delta,
    uint64_t* rng, void* const* Kc, void* const* Vc, int32_t L, const int32_t* page_table,
    int32_t max_pages, int32_t P, int32_t Hkv, int32_t D, int32_t dt, const void* hidden,
    int64_t H, void* h_best, int32_t* ctx, int32_t* root, int32_t* accept_len, int32_t* path,
    int32_t* next_token, int32_t* log, int32_t cap, void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  const char* fn = "medusa_decode_tail";
  MEDUSA_REQUIRE(V >= 1 && V <= INT32_MAX, MEDUSA_ERR_INVALID_ARG, "%s: bad V", fn);
  MEDUSA_REQUIRE(B >= 0 && N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_UNSUPPORTED,
                 "%s: B=%d N=%d (N must be in [1, 64])", fn, B, N);
  MEDUSA_REQUIRE(K >= 0 && K <= MEDUSA_MAX_HEADS, MEDUSA_ERR_UNSUPPORTED, "%s: K=%d outside [0, %d]",
                 fn, K, MEDUSA_MAX_HEADS);
  MEDUSA_REQUIRE(mode >= 0 && mode <= 2, MEDUSA_ERR_INVALID_ARG,
                 "%s: mode %d (0 greedy, 1 typical, 2 sampled)", fn, mode);
  if (mode >= 1)
    MEDUSA_REQUIRE(temperature > 0.f && temperature < 1e30f && epsilon >= 0.f && delta >= 0.f,
                   MEDUSA_ERR_INVALID_ARG,
                   "%s: needs a positive finite temperature and epsilon, delta >= 0", fn);
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dt);
  MEDUSA_REQUIRE(D == 64 || D == 128, MEDUSA_ERR_UNSUPPORTED, "%s: head dim %d", fn, D);
  MEDUSA_REQUIRE(L >= 1 && L <= MEDUSA_MAX_LAYERS, MEDUSA_ERR_UNSUPPORTED, "%s: L=%d outside [1, %d]",
                 fn, L, MEDUSA_MAX_LAYERS);
  MEDUSA_REQUIRE(Hkv >= 1 && Hkv <= 65535 && P >= 1 && max_pages >= 1 && cap >= 0,
                 MEDUSA_ERR_INVALID_ARG, "%s: Hkv=%d P=%d max_pages=%d cap=%d", fn, Hkv, P,
                 max_pages, cap);
  const int es = dt == MEDUSA_BF16 ? 2 : 4;
  MEDUSA_REQUIRE(H >= 1 && (H * es) % 16 == 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: hidden rows must be whole 16-byte chunks (H=%lld)", fn, (long long)H);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(logits && tokens && parent && Kc && Vc && page_table && hidden && h_best && ctx &&
                     root && accept_len && path && next_token && log && (rng || mode != 2),
                 MEDUSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  MEDUSA_REQUIRE(((uintptr_t)hidden | (uintptr_t)h_best) % 16 == 0 && (uintptr_t)rng % 8 == 0,
                 MEDUSA_ERR_INVALID_ARG, "%s: hidden and h_best must be 16-byte aligned, rng 8", fn);
  const size_t need = medusa_decode_tail_ws(B, N);
  MEDUSA_REQUIRE(ws != NULL && ws_bytes >= need, MEDUSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes",
                 fn, ws_bytes, need);
  medusa::TailArgs t{};
  for (int l = 0; l < L; ++l) {
    MEDUSA_REQUIRE(Kc[l] && Vc[l], MEDUSA_ERR_INVALID_ARG, "%s: NULL pool for layer %d", fn, l);
    MEDUSA_REQUIRE(((uintptr_t)Kc[l] | (uintptr_t)Vc[l]) % 16 == 0, MEDUSA_ERR_INVALID_ARG,
                   "%s: pools must be 16-byte aligned", fn);
    t.lp.k[l] = Kc[l];
    t.lp.v[l] = Vc[l];
  }
  hipStream_t st = (hipStream_t)stream;
  const float inv_t = mode >= 1 ? 1.f / temperature : 1.f;
  t.logits = logits;
  t.V = V;
  t.tokens = tokens;
  t.parent = parent;
  t.N = N;
  t.K = K;
  t.typical = mode == 1;
  t.inv_t = inv_t;
  t.epsilon = epsilon;
  t.delta = delta;
  t.Hkv = Hkv;
  t.P = P;
  t.page_table = page_table;
  t.max_pages = max_pages;
  t.hidden = hidden;
  t.H = H;
  t.h_best = h_best;
  t.ctx = ctx;
  t.root = root;
  t.accept_len = accept_len;
  t.path = path;
  t.next_token = next_token;
  t.log = log;
  t.cap = cap;
  t.arrive = (unsigned*)((char*)ws + tail_counter_offset(B));
  if (mode == 2) {
    t.draws = (medusa::Draw*)ws;
    t.S = medusa::row_splits(B, N, V);
    t.rng = rng;
    hipLaunchKernelGGL(medusa::accept_draw_kernel, dim3(N, B, t.S), dim3(256), 0, st, logits, V, N,
                       inv_t, rng, (medusa::Draw*)ws);
  } else {
    t.stats = (medusa::StatPart*)ws;
    t.S = medusa::row_splits(B, N, V);
    hipLaunchKernelGGL(medusa::accept_stats_kernel, dim3(N, B, t.S), dim3(256), 0, st, logits, V, N,
                       mode, inv_t, (medusa::StatPart*)ws);
  }
#define MEDUSA_TAIL(DD, ES)                                                                   \
  hipLaunchKernelGGL((medusa::decode_tail_kernel<DD, ES>),                                     \
                     dim3((unsigned)(L * ((Hkv + medusa::tail_heads<DD, ES>() - 1) /            \
                                          medusa::tail_heads<DD, ES>())),                      \
                          (unsigned)B),                                                        \
                     dim3(256), 0, st, t)
  if (dt == MEDUSA_BF16) { if (D == 128) MEDUSA_TAIL(128, 2); else MEDUSA_TAIL(64, 2); }
  else { if (D == 128) MEDUSA_TAIL(128, 4); else MEDUSA_TAIL(64, 4); }
#undef MEDUSA_TAIL
  return check_launch(fn);
}
