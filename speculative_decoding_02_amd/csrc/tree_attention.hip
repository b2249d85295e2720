// medusa_tree_attention: one tree-masked attention pass over a paged KV cache
// plus the tree's own keys ("Medusa Heads", section "Attenzione sull'albero e
// accettazione": every candidate token is appended at once and the mask lets
// each token see only its ancestors, so all branches are verified in one pass;
// arXiv abstract page: tree-based attention).
//
// Work decomposition (gfx950, 64-wide waves):
//   grid = (splits, Hq, B); a workgroup owns one contiguous key range of one
//   (sequence, query head): cached keys 0..ctx-1 followed by the N tree keys.
//   Its 4 waves each own 16 tree nodes (query rows) and sweep the range in
//   tiles of 64 keys.
//   * K tile [64 x D] and the TRANSPOSED V tile [D x 64] are staged in LDS
//     (16-byte global loads; the next tile is prefetched into registers while
//     the current one is computed).
//   * S^T = K Q^T on MFMA: the result lands with lane l holding node l%16 and
//     keys 4*(l/16)+r, which is exactly the operand layout of P^T in
//     O^T += V^T P^T, so probabilities never leave registers.
//   * online softmax in fp32 (base-2 exponent), per node; tree keys are
//     kept iff their bit is set in the node's uint64 ancestor mask.
//   * the tree keys' K/V are stored into cache slots ctx..ctx+N-1 by the
//     workgroup whose split covers them (first query head of each kv group),
//     after its tile loop.
//   * a (sequence, head) whose key range needs one split writes O directly;
//     otherwise every split writes (max, sum, unnormalised O) partials and a
//     second, small launch merges them in fixed split order.  Deterministic;
//     no cross-workgroup synchronisation inside a launch.
//   * the tile loads run PF tiles ahead through a ring of register stages
//     (unrolled, so every stage index is static), keeping a workgroup's whole
//     key range in flight for the short ranges of decode-time splits.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace medusa {

constexpr int ATT_TILE = 64;
constexpr int ATT_THREADS = 256;
constexpr int ATT_MAX_SPLIT_PAGES = 256;  // page-table window of one split (LDS)

template <typename T, int D>
struct AttnCfg {
  static constexpr int P16 = 16 / (int)sizeof(T);       // elements per 16-byte vector
  static constexpr int LDK = D + P16;                    // K row, padded by 16 B
  static constexpr int LDV = ATT_TILE + 4;               // V^T row, padded
  static constexpr int QSTEPS = D / (4 * P16);           // MFMA steps over the head dim
  static constexpr int KCHUNKS = ATT_TILE * D / P16;     // 16-byte chunks per K tile
  static constexpr int KPT = KCHUNKS / ATT_THREADS;      // chunks per thread
  static constexpr int VGROUPS = (ATT_TILE / 4) * (D / P16);  // (4 keys x P16 dims) groups
  static constexpr int VPT = (VGROUPS + ATT_THREADS - 1) / ATT_THREADS;
  static_assert(KCHUNKS % ATT_THREADS == 0, "K tile chunks");
};

// Element type of the split partials: fp16 for bf16 attention, fp32 for fp32
// attention.  A split's partial is its normalised output, a convex
// combination of V rows.  In fp16 it is stored block-scaled: each (split,
// node) row is multiplied by 2^-s, with s chosen from the row's largest
// magnitude so that it lands in [2^14, 2^15), and s is kept with the row's
// (max, sum).  fp16's 11-bit significand then covers the row's large
// entries (relative rounding 2^-11, far inside bf16's 2^-8) whatever the
// magnitude of V, which bf16 allows up to 3.4e38, while fp16 alone would
// overflow above 65504.  The scaling by a power of two is exact.
template <typename T> struct PartT { using type = float; };
template <> struct PartT<bf16_t> { using type = _Float16; };

// (running max in log2 units, sum, scale exponent s of the stored row, pad)
struct PartStat {
  float m, l;
  int s, pad;
};
// the exponent s with mx * 2^-s in [2^14, 2^15) (0 for an all-zero row)
__device__ __forceinline__ int part_scale_exp(float mx) {
  int e = 0;
  (void)frexpf(mx, &e);  // mx = f * 2^e, f in [1/2, 1)
  return mx > 0.f ? e - 15 : 0;
}

// component i (compile-time after unrolling) of a 16-byte register vector
__device__ __forceinline__ uint32_t u4c(u32x4 v, int i) { return v[i]; }

template <typename T> struct AttnMma;
template <> struct AttnMma<bf16_t> {
  // scores: K rows (A) x Q rows (B), 8 dims per lane
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) { return mfma_bf16_16x16x32(a, b, c); }
};
template <> struct AttnMma<float> {
  static __device__ __forceinline__ f32x4 qk(u32x4 a, u32x4 b, f32x4 c) {
    c = mfma_f32_16x16x4(__uint_as_float(a.x), __uint_as_float(b.x), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.y), __uint_as_float(b.y), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.z), __uint_as_float(b.z), c);
    c = mfma_f32_16x16x4(__uint_as_float(a.w), __uint_as_float(b.w), c);
    return c;
  }
};

struct AttnArgs {
  const void* Q;
  const void* Kt;
  const void* Vt;
  void* Kc;
  void* Vc;
  const int* page_table;
  const int* ctx;
  const uint64_t* mask;
  void* O;
  PartStat* ml;      // [B*Hq*S*N]
  void* opart;       // [B*Hq*S*N*D] of PartT<T>: a split's output divided by its own sum
  int max_pages, P, B, N, Hq, Hkv, chunk;  // chunk = keys per split (multiple of 64)
  int max_ctx;
  int lp;            // log2(P) when P is a power of two, else -1 (page math by division)
  float scale_log2;
};

template <typename T, int D, int PF>
__global__ __launch_bounds__(ATT_THREADS) void tree_attention_kernel(AttnArgs a) {
  using C = AttnCfg<T, D>;
  constexpr int P16 = C::P16;
  __shared__ __attribute__((aligned(16))) T Ks[ATT_TILE * C::LDK];
  __shared__ __attribute__((aligned(16))) T Vs[D * C::LDV];
  __shared__ int spages[ATT_MAX_SPLIT_PAGES];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = gridDim.x;
  const int N = a.N;
  const int k_beg = s * a.chunk;
  const int group = a.Hq / a.Hkv;
  const int kvh = h / group;
  const bool appender = (h % group) == 0;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int node = wave * 16 + lr;
  const bool wave_active = wave * 16 < N;
  const int nodec = min(node, N - 1);

  const T* Qp = reinterpret_cast<const T*>(a.Q);
  const T* Ktp = reinterpret_cast<const T*>(a.Kt);
  const T* Vtp = reinterpret_cast<const T*>(a.Vt);
  T* Kcp = reinterpret_cast<T*>(a.Kc);
  T* Vcp = reinterpret_cast<T*>(a.Vc);
  const int* pt = a.page_table + (int64_t)b * a.max_pages;

  // One round trip before the tile loads: the sequence length, the split's
  // slice of the page table (sized from max_ctx + N, so it does not wait for
  // the length; it covers the cache slots and the tree slots the split may
  // touch), this wave's queries and its nodes' ancestor masks are all
  // loaded together.  The page slice goes to LDS, so that address
  // computation never waits on a global load (a wait there would also wait
  // for every tile load in flight).
  const int page0 = k_beg / a.P;
  const int slice_end = min(k_beg + a.chunk, a.max_ctx + N);
  const int npages = slice_end > k_beg ? (slice_end - 1) / a.P - page0 + 1 : 0;
  // (a length outside [0, max_ctx] breaks the caller's contract; it is
  // clamped so that every access stays inside the page slice)
  const int ctxb = min(max(a.ctx[b], 0), a.max_ctx);
  // npages <= ATT_MAX_SPLIT_PAGES == ATT_THREADS: one page per thread, held
  // in a register until the queries' loads are issued too
  static_assert(ATT_MAX_SPLIT_PAGES <= ATT_THREADS, "one page-table entry per thread");
  const int my_page = threadIdx.x < npages ? pt[page0 + threadIdx.x] : 0;

  // element offset of key j's row for kv head kvh (cache slot or tree node)
  // page of key j and its slot there (shifts when P is a power of two: the
  // address math runs per lane for every tile)
  auto cache_off = [&](int j) -> int64_t {
    const int pj = a.lp >= 0 ? (j >> a.lp) : j / a.P;
    const int sj = a.lp >= 0 ? (j & (a.P - 1)) : j - pj * a.P;
    const int page = spages[pj - page0];
    return (((int64_t)page * a.Hkv + kvh) * a.P + sj) * D;
  };
  auto tree_off = [&](int j) -> int64_t {
    return (((int64_t)b * N + max(j - ctxb, 0)) * a.Hkv + kvh) * D;
  };

  // ---- this wave's queries, B operand of S^T = K Q^T ----
  u32x4 qf[C::QSTEPS];
  {
    const T* qrow = Qp + (((int64_t)b * N + nodec) * a.Hq + h) * D;
#pragma unroll
    for (int st = 0; st < C::QSTEPS; ++st)
      qf[st] = *reinterpret_cast<const u32x4*>(qrow + st * 4 * P16 + lg * P16);
  }
  const uint64_t mrow = a.mask[(int64_t)b * N + nodec];
  // Everything above is in registers or LDS before any tile load is issued,
  // so the loop never waits on it (a wait there would also drain the tile
  // loads).
  __builtin_amdgcn_s_waitcnt(0);
  if (threadIdx.x < npages) spages[threadIdx.x] = my_page;
  __syncthreads();
  const int total = ctxb + N;
  if (k_beg >= total) return;  // uniform over the workgroup
  const int k_end = min(k_beg + a.chunk, total);

  // ---- tile loaders ----
  u32x4 kreg[PF][C::KPT];
  u32x4 vreg[PF][C::VPT][4];

  // Loads never feed a select (that would wait for them at once): keys past
  // the split's end read a valid row (clamped index) whose score is masked
  // to -inf later, so its probability is exactly 0 and its finite V adds 0.
  auto gload = [&](int u, int tile0) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int c = tid + i * ATT_THREADS;
      const int key = c / (D / P16), part = c % (D / P16);
      const int jj = min(tile0 + key, k_end - 1);
      const T* kc = Kcp + cache_off(jj);
      const T* kt = Ktp + tree_off(jj);
      const T* src = (jj < ctxb ? kc : kt) + part * P16;
      kreg[u][i] = *reinterpret_cast<const u32x4*>(src);
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int g = min(tid + i * ATT_THREADS, C::VGROUPS - 1);
      const int kg = g / (D / P16), dg = g % (D / P16);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = min(tile0 + kg * 4 + r, k_end - 1);
        const T* vc = Vcp + cache_off(jj);
        const T* vt = Vtp + tree_off(jj);
        const T* src = (jj < ctxb ? vc : vt) + dg * P16;
        vreg[u][i][r] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };

  auto lds_store = [&](int u, int tile0) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int c = tid + i * ATT_THREADS;
      const int key = c / (D / P16), part = c % (D / P16);
      *reinterpret_cast<u32x4*>(&Ks[key * C::LDK + part * P16]) = kreg[u][i];
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int g = tid + i * ATT_THREADS;
      if (g < C::VGROUPS) {
        const int kg = g / (D / P16), dg = g % (D / P16);
        const int key0 = kg * 4, d0 = dg * P16;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int sh = (e & 1) * 16, wi = e >> 1;
            u32x2 v;
            v.x = ((u4c(vreg[u][i][0], wi) >> sh) & 0xffffu) | (((u4c(vreg[u][i][1], wi) >> sh) & 0xffffu) << 16);
            v.y = ((u4c(vreg[u][i][2], wi) >> sh) & 0xffffu) | (((u4c(vreg[u][i][3], wi) >> sh) & 0xffffu) << 16);
            *reinterpret_cast<u32x2*>(&Vs[(d0 + e) * C::LDV + key0]) = v;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            u32x4 v = {u4c(vreg[u][i][0], e), u4c(vreg[u][i][1], e), u4c(vreg[u][i][2], e), u4c(vreg[u][i][3], e)};
            *reinterpret_cast<u32x4*>(&Vs[(d0 + e) * C::LDV + key0]) = v;
          }
        }
      }
    }
  };

  // ---- running softmax state: lane holds node lr; O^T rows d = db*16+4*lg+r ----
  constexpr int DB = D / 16;
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  // Prologue and refills load unconditionally (tile index clamped to the
  // split's last tile), so the waits before each tile count only later loads.
  const int ntiles = (k_end - k_beg + ATT_TILE - 1) / ATT_TILE;
  const int last_tile0 = k_beg + (ntiles - 1) * ATT_TILE;
#pragma unroll
  for (int u = 0; u < PF; ++u) gload(u, min(k_beg + u * ATT_TILE, last_tile0));
  for (int t0 = 0; t0 < ntiles; t0 += PF) {
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    const int t = t0 + u;
    if (t >= ntiles) break;
    const int tile0 = k_beg + t * ATT_TILE;
    lds_store(u, tile0);
    __syncthreads();
    gload(u, min(tile0 + PF * ATT_TILE, last_tile0));

    if (wave_active) {
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < C::QSTEPS; ++st) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(
              &Ks[(kb * 16 + lr) * C::LDK + st * 4 * P16 + lg * P16]);
          sacc[kb] = AttnMma<T>::qk(kf, qf[st], sacc[kb]);
        }
      }
      float x[4][4];
      float tmax = -INFINITY;
      // a tile wholly inside the cached keys needs no mask (wave-uniform)
      const bool plain = tile0 + ATT_TILE <= min(ctxb, k_end);
      if (plain) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[kb][r] = sacc[kb][r] * a.scale_log2;
            tmax = fmaxf(tmax, x[kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = tile0 + kb * 16 + lg * 4 + r;
            const uint32_t bit = (uint32_t)(mrow >> (uint32_t)min(max(j - ctxb, 0), 63)) & 1u;
            const bool ok = (j < k_end) & ((j < ctxb) | (bit != 0u));
            x[kb][r] = ok ? sacc[kb][r] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[kb][r]);
          }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(mrun, tmax);
      const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(mrun - mnew);
      float psum = 0.f;
      if (plain) {  // every score finite, so mnew is too
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[kb][r] = exp2f(x[kb][r] - mnew);
            psum += x[kb][r];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = (x[kb][r] == -INFINITY) ? 0.f : exp2f(x[kb][r] - mnew);
            x[kb][r] = p;
            psum += p;
          }
      }
      lrun = lrun * alpha + psum;
      mrun = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (sizeof(T) == 2) {
          u32x2 pb;
          pb.x = pack_bf2(x[kb][0], x[kb][1]);
          pb.y = pack_bf2(x[kb][2], x[kb][3]);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2 vf = *reinterpret_cast<const u32x2*>(
                &Vs[(db * 16 + lr) * C::LDV + kb * 16 + lg * 4]);
            oacc[db] = mfma_bf16_16x16x16(vf, pb, oacc[db]);
          }
        } else {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const f32x4 vf = *reinterpret_cast<const f32x4*>(
                &Vs[(db * 16 + lr) * C::LDV + kb * 16 + lg * 4]);
            oacc[db] = mfma_f32_16x16x4(vf.x, x[kb][0], oacc[db]);
            oacc[db] = mfma_f32_16x16x4(vf.y, x[kb][1], oacc[db]);
            oacc[db] = mfma_f32_16x16x4(vf.z, x[kb][2], oacc[db]);
            oacc[db] = mfma_f32_16x16x4(vf.w, x[kb][3], oacc[db]);
          }
        }
      }
    }
    __syncthreads();
  }
  }

  // Store the tree keys' K/V of this split into cache slots ctx..ctx+N-1
  // (after the tile loop, so these stores never sit between tile loads).
  if (appender && k_end > ctxb) {
    constexpr int CPR = D / P16;  // 16-byte chunks per row
    const int j0 = max(k_beg, ctxb);
    const int items = (k_end - j0) * CPR * 2;
    for (int e = tid; e < items; e += ATT_THREADS) {
      const int which = e / ((k_end - j0) * CPR), rem = e % ((k_end - j0) * CPR);
      const int j = j0 + rem / CPR, part = rem % CPR;
      const T* src = (which ? Vtp : Ktp) + tree_off(j) + part * P16;
      T* dst = (which ? Vcp : Kcp) + cache_off(j) + part * P16;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
  }

  float ltot = lrun + __shfl_xor(lrun, 16, 64);
  ltot = ltot + __shfl_xor(ltot, 32, 64);
  T* Op = reinterpret_cast<T*>(a.O);
  const bool node_ok = wave_active && node < N;

  // A one-split grid writes O directly; otherwise every split writes its
  // partials (a sequence whose range fits in one split included).
  if (S == 1) {
    if (node_ok) {
      const float inv = 1.f / ltot;
      T* orow = Op + (((int64_t)b * N + node) * a.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) st<T>(orow, db * 16 + lg * 4 + r, oacc[db][r] * inv);
    }
    return;
  }

  // ---- multi-split: partials; tree_attention_combine merges them ----
  const int64_t bh = (int64_t)b * a.Hq + h;
  if (node_ok) {
    using PT = typename PartT<T>::type;
    PT* op = reinterpret_cast<PT*>(a.opart) + ((bh * S + s) * N + node) * D;
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (sizeof(PT) == 2) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 v = {(_Float16)(oacc[db][0] * inv), (_Float16)(oacc[db][1] * inv), (_Float16)(oacc[db][2] * inv),
                (_Float16)(oacc[db][3] * inv)};
        *reinterpret_cast<h4*>(op + db * 16 + lg * 4) = v;
      } else {
        *reinterpret_cast<f32x4*>(op + db * 16 + lg * 4) = oacc[db] * inv;
      }
    }
    if (lg == 0) a.ml[(bh * S + s) * N + node] = PartStat{mrun, ltot, 0, 0};
  }
}

// bf16 kernel: the split's key/value tiles stream straight into LDS.
//   * 4*KQ waves: wave w owns tree nodes 16*(w%4) .. +15 and, in every
//     64-key tile, the 64/KQ keys of part w/4, with its own online-softmax
//     state; the parts are merged through LDS after the tile loop.  KQ waves
//     per SIMD keep the MFMA and vector pipes busy while the others wait on
//     their dependency chains (LDS reads, MFMA results, exponentials).
//   * Each wave issues LDS-DMA loads (16 bytes per lane, written at m0 +
//     16*lane) for its share of a tile's K and V rows into a ring of R LDS
//     slots.  The first R tiles are issued together right after the
//     page-table round trip; afterwards a slot is refilled as soon as every
//     wave is done reading it, so up to R-1 tiles stay in flight while one is
//     computed.  Only tiles of the split are loaded, and the wait before tile
//     t lets exactly the later tiles already issued remain in flight.
//   * Row r of a tile keeps its 16-byte chunk c at position c ^ (r & SW):
//     the lane that fills position p fetches chunk p ^ (r & SW).  The score
//     MFMA's operand reads (16 rows, one chunk column) then hit 16 distinct
//     bank groups.
//   * V stays row-major; the P.V MFMA's V^T operand comes from the gfx950
//     transposing LDS read: within a 16-lane block, lane i returns element
//     i%4 of the 4 values at source lane (i/4)+4r's address, so pointing lane
//     j of block g at V[key 4g + j/4][dim 4(j%4)] yields V[key 4g + r][dim i].
//   * One barrier per tile: at the start of tile t every wave has its own
//     DMA of tile t landed and its LDS reads of tile t-1 done, so after the
//     barrier tile t is readable everywhere and tile t-1's slot is free for
//     tile t-1+R.  s_barrier goes without a fence (a fenced barrier would
//     wait for every DMA in flight).
//   * Online softmax with a lazy reference: the running maximum m (log2
//     units) only moves, and the output and sum are only rescaled, when some
//     node of the wave sees a score above m + ATT_LAZY; otherwise the tile's
//     probabilities are taken against the old m (each at most 2^ATT_LAZY,
//     far inside fp32 and bf16 range).  Output, sum and m always refer to the
//     same m, so the normalised result is the same softmax.
//   * The DMA source addresses are computed without branches: the page
//     lookups of a wave's rows are read from LDS together, cached and tree
//     rows are chosen by selects, and P2 (page size a power of two) turns the
//     page/slot split into a shift and a mask.
constexpr float ATT_LAZY = 8.f;
template <int D, int R, int KQ, bool P2>
__global__ __launch_bounds__(256 * KQ) void tree_attention_stream_kernel(AttnArgs a) {
  using T = bf16_t;
  constexpr int NT = 256 * KQ;                 // threads
  constexpr int NW = NT / 64;                  // waves
  constexpr int KW = ATT_TILE / KQ;            // keys per wave and tile
  constexpr int KB = KW / 16;                  // 16-key MFMA blocks per wave and tile
  static_assert(KQ == 2 || KQ == 4, "two or four key parts");
  constexpr int P16 = 8;                       // bf16 per 16 bytes
  constexpr int ROWB = D * 2;                  // bytes per key row
  constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  constexpr int SW = CPR - 1;                  // swizzle mask
  // V rows are read 8 rows x 2 adjacent chunks per 32-lane pass of the
  // transposing read: with 16 chunks a row (D = 128) the chunk is XORed with
  // twice the row so that those 16 pieces land on 16 distinct bank groups
  // (XOR with the row would map chunks 2d, 2d+1 of rows r, r^1 together)
  auto vsw = [](int r) { return CPR == 16 ? ((2 * r) & SW) : (r & SW); };
  constexpr int TILEB = ATT_TILE * ROWB;       // bytes of one K (or V) tile
  constexpr int SLOTB = 2 * TILEB;
  constexpr int RPD = 1024 / ROWB;             // rows per DMA instruction (64 lanes x 16 B)
  constexpr int DPW = TILEB / 1024 / NW;       // DMA instructions per wave per tensor
  constexpr int OPS = 2 * DPW;                 // vector-memory ops per wave per tile
  constexpr int QSTEPS = D / 32;
  constexpr int DB = D / 16;
  static_assert(DPW >= 1 && DPW * NW * 1024 == TILEB, "tile must split into whole DMAs");
  static_assert(R >= 2 && R <= 8, "ring of 2..8 tiles");
  static_assert((R - 1) * OPS < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[R * SLOTB];
  __shared__ int spages[ATT_MAX_SPLIT_PAGES];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int S = gridDim.x;
  const int N = a.N;
  const int k_beg = s * a.chunk;
  const int group = a.Hq / a.Hkv;
  const int kvh = h / group;
  const bool appender = (h % group) == 0;
  const int tid = threadIdx.x;
  // wave index made provably uniform, so per-wave branches stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int nb = wave & 3, hf = wave >> 2;     // node block, key part
  const int node = nb * 16 + lr;
  const bool wave_active = nb * 16 < N;
  const int nodec = min(node, N - 1);

  const T* Qp = reinterpret_cast<const T*>(a.Q);
  const T* Ktp = reinterpret_cast<const T*>(a.Kt);
  const T* Vtp = reinterpret_cast<const T*>(a.Vt);
  T* Kcp = reinterpret_cast<T*>(a.Kc);
  T* Vcp = reinterpret_cast<T*>(a.Vc);
  const int* pt = a.page_table + (int64_t)b * a.max_pages;

  // One round trip before the tile stream: the sequence length, the split's
  // slice of the page table (sized from max_ctx + N, so it does not wait for
  // the length; it covers the cache slots and the tree slots the split may
  // touch), this wave's queries and its nodes' ancestor masks.  The page
  // slice goes to LDS, so that address computation never waits on a global
  // load (a wait there would also wait for every tile load in flight).
  const int page0 = k_beg / a.P;
  const int slice_end = min(k_beg + a.chunk, a.max_ctx + N);
  const int npages = slice_end > k_beg ? (slice_end - 1) / a.P - page0 + 1 : 0;
  // (a length outside [0, max_ctx] breaks the caller's contract; it is
  // clamped so that every access stays inside the page slice)
  const int ctxb = min(max(a.ctx[b], 0), a.max_ctx);
  static_assert(ATT_MAX_SPLIT_PAGES <= NT, "one page-table entry per thread");
  const int my_page = threadIdx.x < npages ? pt[page0 + threadIdx.x] : 0;
  u32x4 qf[QSTEPS];
  {
    const T* qrow = Qp + (((int64_t)b * N + nodec) * a.Hq + h) * D;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st)
      qf[st] = *reinterpret_cast<const u32x4*>(qrow + st * 4 * P16 + lg * P16);
  }
  const uint64_t mrow = a.mask[(int64_t)b * N + nodec];
  __builtin_amdgcn_s_waitcnt(0);
  if (threadIdx.x < npages) spages[threadIdx.x] = my_page;
  __syncthreads();
  const int total = ctxb + N;
  if (k_beg >= total) return;  // uniform over the workgroup
  const int k_end = min(k_beg + a.chunk, total);
  const int ntiles = (k_end - k_beg + ATT_TILE - 1) / ATT_TILE;

  // page of key j and its slot there
  const int64_t page_elems = (int64_t)a.Hkv * a.P * D;  // one page of the cache
  const int head_elems = kvh * a.P * D;                  // this head's rows in a page
  auto cache_off = [&](int j) -> int64_t {
    const int pj = P2 ? (j >> a.lp) : j / a.P;
    const int sj = P2 ? (j & (a.P - 1)) : j - pj * a.P;
    const int page = spages[pj - page0];
    return (int64_t)page * page_elems + (head_elems + sj * D);
  };
  const int64_t tree_base = ((int64_t)b * N * a.Hkv + kvh) * D;
  auto tree_off = [&](int j) -> int64_t {
    return tree_base + max(j - ctxb, 0) * (a.Hkv * D);
  };

  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds;
  // DMA of tile t (< ntiles) into ring slot `slot`.  Rows past the split's
  // end re-read its last key (their scores are masked).  Every key of
  // [k_beg, k_end) has its page in spages (the tree keys' too: they go to
  // cache slots ctx..ctx+N-1), so the lookup runs for every row and the
  // tree rows just ignore it.
  auto issue = [&](int t, int slot) {
    const int tile0 = k_beg + t * ATT_TILE;
    int jj[DPW], pg[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int r = (wave * DPW + i) * RPD + lane / CPR;  // tile row this lane fills
      jj[i] = min(tile0 + r, k_end - 1);
      pg[i] = spages[(P2 ? (jj[i] >> a.lp) : jj[i] / a.P) - page0];
    }
    if (tile0 + ATT_TILE <= ctxb) {  // (wave-uniform) every row of the tile is a cache row
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        const int q = wave * DPW + i;          // 1 KB block of the tile
        const int r = q * RPD + lane / CPR;
        const int c = (lane % CPR) ^ (r & SW); // chunk fetched for that position
        const int cv = (lane % CPR) ^ vsw(r);
        const int j = jj[i];
        const int sj = P2 ? (j & (a.P - 1)) : j - (j / a.P) * a.P;
        const int64_t row = (int64_t)(uint32_t)pg[i] * page_elems + (head_elems + sj * D);
        const uint32_t kd = lds_base + slot * SLOTB + q * 1024;
        lds_dma16(Kcp + row + c * P16, kd);
        lds_dma16(Vcp + row + cv * P16, kd + TILEB);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int q = wave * DPW + i;          // 1 KB block of the tile
      const int r = q * RPD + lane / CPR;
      const int c = (lane % CPR) ^ (r & SW); // chunk fetched for that position
      const int cv = (lane % CPR) ^ vsw(r);
      const int j = jj[i];
      const bool cached = j < ctxb;
      const int sj = P2 ? (j & (a.P - 1)) : j - (j / a.P) * a.P;
      const int64_t coff = (int64_t)(uint32_t)pg[i] * page_elems + (head_elems + sj * D);
      const int64_t off = cached ? coff : tree_off(j);
      const T* ksrc = (cached ? Kcp : Ktp) + off + c * P16;
      const T* vsrc = (cached ? Vcp : Vtp) + off + cv * P16;
      const uint32_t kd = lds_base + slot * SLOTB + q * 1024;
      lds_dma16(ksrc, kd);
      lds_dma16(vsrc, kd + TILEB);
    }
  };
  // wait until at most n tiles of this wave's DMA are in flight (n < R)
  auto wait_tiles = [&](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 1 ? 1 * OPS : 0)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 2 ? 2 * OPS : 0)); break;
      case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 3 ? 3 * OPS : 0)); break;
      case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 4 ? 4 * OPS : 0)); break;
      case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 5 ? 5 * OPS : 0)); break;
      case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 6 ? 6 * OPS : 0)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 7 ? 7 * OPS : 0)); break;
    }
  };

  // This lane's LDS byte offsets inside a ring slot (first 16-key block; the
  // next block is 16 rows further): K operand chunk of each contraction step,
  // and the transposing-read address of each 16-dim block of V.
  int kofs[QSTEPS], vofs[DB];
#pragma unroll
  for (int st = 0; st < QSTEPS; ++st)
    kofs[st] = (hf * KW + lr) * ROWB + (((st * 4 + lg) ^ (lr & SW)) * 16);
  {
    const int rr = hf * KW + 4 * lg + (lr >> 2);  // source row of this lane's address
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = db * 2 + ((lr & 3) >> 1);
      vofs[db] = rr * ROWB + ((c ^ vsw(rr)) * 16) + (lr & 1) * 8;
    }
  }

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  const int first = min(ntiles, R);
  for (int t = 0; t < first; ++t) issue(t, t);
  for (int t = 0; t < ntiles; ++t) {
    const int slot = t % R;
    // tiles issued before this point: min(ntiles, R + max(t - 1, 0))
    wait_tiles(t == 0 ? first - 1 : min(ntiles - 1 - t, R - 2));  // tile t has landed
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);  // ... and this wave's LDS reads of tile t-1
    __builtin_amdgcn_s_barrier();               // ... and every other wave's
    asm volatile("" ::: "memory");              // no LDS access moves across the barrier
    if (t >= 1 && t - 1 + R < ntiles) issue(t - 1 + R, (t - 1) % R);  // into tile t-1's slot
    const int key0 = k_beg + t * ATT_TILE + hf * KW;  // this wave's KW keys
    const unsigned char* ks = lds + slot * SLOTB;
    const unsigned char* vs = ks + TILEB;
    if (wave_active && key0 < k_end) {
      f32x4 sacc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < QSTEPS; ++st) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(ks + kofs[st] + kb * 16 * ROWB);
          sacc[kb] = mfma_bf16_16x16x32(kf, qf[st], sacc[kb]);
        }
      }
      // the V^T operands do not depend on the softmax: read them now, so the
      // LDS latency overlaps the score MFMAs and the exponentials
      typedef short s4 __attribute__((ext_vector_type(4)));
      u32x2 vf[KB][DB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          vf[kb][db] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s4*)(vs + vofs[db] + kb * 16 * ROWB)));
      // raw scores x (masked: -inf); the scale (> 0, in log2 units) is
      // applied to the maximum and inside the exponent's FMA
      float x[KB][4];
      float tmax = -INFINITY;
      // keys wholly inside the cached range need no mask (wave-uniform)
      const bool plain = key0 + KW <= min(ctxb, k_end);
      if (plain) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[kb][r] = sacc[kb][r];
            tmax = fmaxf(tmax, x[kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = key0 + kb * 16 + lg * 4 + r;
            const uint32_t bit = (uint32_t)(mrow >> (uint32_t)min(max(j - ctxb, 0), 63)) & 1u;
            const bool ok = (j < k_end) & ((j < ctxb) | (bit != 0u));
            x[kb][r] = ok ? sacc[kb][r] : -INFINITY;
            tmax = fmaxf(tmax, x[kb][r]);
          }
      }
      tmax = rows4_max(tmax) * a.scale_log2;
      // move the reference only when some node's scores outgrow it
      if (__builtin_amdgcn_ballot_w64(tmax > mrun + ATT_LAZY) != 0) {
        const float mnew = fmaxf(mrun, tmax);
        const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
        lrun *= alpha;
        mrun = mnew;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
      float psum = 0.f;
      if (plain) {  // every score finite, and mrun finite once a score was seen
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            x[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][r], a.scale_log2, -mrun));
            psum += x[kb][r];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = (x[kb][r] == -INFINITY)
                                ? 0.f
                                : __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][r], a.scale_log2, -mrun));
            x[kb][r] = p;
            psum += p;
          }
      }
      lrun += psum;
      // O^T += V^T P^T.  Lane l holds the probabilities of keys kb*16 +
      // 4*(l/16) + r; two 16-key blocks form the 8-element contraction slice
      // of one 16x16x32 step (element i = block i/4, r = i%4), and the two
      // transposing reads of those blocks give V^T in the same key order.
      auto vread = [&](int kb, int db) -> u32x2 { return vf[kb][db]; };
      if constexpr (KB % 2 == 0) {
#pragma unroll
        for (int kb = 0; kb < KB; kb += 2) {
          const u32x4 pb = {pack_bf2(x[kb][0], x[kb][1]), pack_bf2(x[kb][2], x[kb][3]),
                            pack_bf2(x[kb + 1][0], x[kb + 1][1]), pack_bf2(x[kb + 1][2], x[kb + 1][3])};
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2 v0 = vread(kb, db), v1 = vread(kb + 1, db);
            oacc[db] = mfma_bf16_16x16x32(u32x4{v0.x, v0.y, v1.x, v1.y}, pb, oacc[db]);
          }
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const u32x2 pb = {pack_bf2(x[kb][0], x[kb][1]), pack_bf2(x[kb][2], x[kb][3])};
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db] = mfma_bf16_16x16x16(vread(kb, db), pb, oacc[db]);
        }
      }
    }
    asm volatile("" ::: "memory");
  }
  // (every tile issued was waited for above: no DMA is left in flight)

  // Store the tree keys' K/V of this split into cache slots ctx..ctx+N-1.
  if (appender && k_end > ctxb) {
    constexpr int CPRT = D / P16;
    const int j0 = max(k_beg, ctxb);
    const int items = (k_end - j0) * CPRT * 2;
    for (int e = tid; e < items; e += NT) {
      const int which = e / ((k_end - j0) * CPRT), rem = e % ((k_end - j0) * CPRT);
      const int j = j0 + rem / CPRT, part = rem % CPRT;
      const T* src = (which ? Vtp : Ktp) + tree_off(j) + part * P16;
      T* dst = (which ? Vcp : Kcp) + cache_off(j) + part * P16;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
  }

  // merge key parts 1..KQ-1 into part 0, in part order (per node: max and
  // sum per lane; output dims db*16 + lg*4 + r of this lane)
  float ltot = rows4_sum(lrun);
  __syncthreads();                             // every wave is done with the ring
  float* xch = reinterpret_cast<float*>(lds);  // [KQ-1 parts][4 node blocks][64 lanes][DB*4 + 2]
  constexpr int XW = DB * 4 + 2;
  static_assert((KQ - 1) * 4 * 64 * XW * 4 <= R * SLOTB, "exchange fits in the ring");
  if (hf >= 1) {
    float* d = xch + (((hf - 1) * 4 + nb) * 64 + lane) * XW;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) d[db * 4 + r] = oacc[db][r];
    d[DB * 4] = mrun;
    d[DB * 4 + 1] = ltot;
  }
  __syncthreads();
  if (hf >= 1) return;
#pragma unroll
  for (int q = 1; q < KQ; ++q) {
    const float* d = xch + (((q - 1) * 4 + nb) * 64 + lane) * XW;
    const float m1 = d[DB * 4], l1 = d[DB * 4 + 1];
    const float mm = fmaxf(mrun, m1);
    const float w0 = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun - mm);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[db][r] = oacc[db][r] * w0 + d[db * 4 + r] * w1;
    ltot = ltot * w0 + l1 * w1;
    mrun = mm;
  }
  const bool node_ok = wave_active && node < N;
  if (S == 1) {
    if (node_ok) {
      const float inv = 1.f / ltot;
      T* orow = reinterpret_cast<T*>(a.O) + (((int64_t)b * N + node) * a.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) st<T>(orow, db * 16 + lg * 4 + r, oacc[db][r] * inv);
    }
    return;
  }
  const int64_t bh = (int64_t)b * a.Hq + h;
  // the row's block exponent: its largest magnitude over the four lanes that
  // hold node `node` (every lane of a wave takes part in the row swaps)
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  float amax = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(oacc[db][r] * inv));
  const int sexp = part_scale_exp(rows4_max(amax));
  if (node_ok) {
    _Float16* op = reinterpret_cast<_Float16*>(a.opart) + ((bh * S + s) * N + node) * D;
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      h4 v = {(_Float16)ldexpf(oacc[db][0] * inv, -sexp), (_Float16)ldexpf(oacc[db][1] * inv, -sexp),
              (_Float16)ldexpf(oacc[db][2] * inv, -sexp), (_Float16)ldexpf(oacc[db][3] * inv, -sexp)};
      *reinterpret_cast<h4*>(op + db * 16 + lg * 4) = v;
    }
    if (lg == 0) a.ml[(bh * S + s) * N + node] = PartStat{mrun, ltot, sexp, 0};
  }
}

// bf16 kernel without key splits, for launches with few (sequence, head)
// pairs, such as one sequence's decode step: one workgroup per (sequence,
// query head, block of 16 tree nodes) covers its head's whole key range, so
// no split partials are written and no merge launch follows.
//   * The 8 waves take the range's 16-key chunks in turn (chunk c goes to
//     wave c % 8), each with its own online softmax over its chunks; the
//     eight states of a node are merged through LDS in wave order after the
//     loop (a fixed order: the result does not depend on timing).
//   * Each wave streams its chunks' K and V rows by LDS-DMA into a ring of R
//     slots of its own, so inside the loop a wave waits only on its own
//     loads: eight independent chains per CU and no barrier per tile.  The
//     chunks' rows use the split kernel's 16-byte-chunk swizzles, so the
//     score operand reads and the transposing V reads are conflict-free.
//   * The workgroups that read the same kv head (its node blocks and the
//     query heads of its group) run on one XCD: workgroup i goes to XCD
//     i % 8, and the grid is ordered so that every workgroup of one
//     (sequence, kv head) shares i % 8.  Their K/V rows then come from HBM
//     once and from that XCD's L2 for the other readers.
//   * The workgroups of the first query head of a kv group store their
//     nodes' K/V rows into cache slots ctx + node (the rows are loaded in
//     the first round trip and stored after the loop, so the store adds no
//     dependent load at the end).  The other workgroups read tree keys from
//     Kt/Vt and cached keys from slots below ctx only, so those stores race
//     with no read.
//   * A workgroup's range is at most NBK_MAX_KEYS planned keys (max_ctx + N;
//     the host plans longer ranges on the split kernel), so its page table
//     fits a small LDS window.
constexpr int NBK_WAVES = 8;
constexpr int NBK_CHUNK = 16;
constexpr int NBK_MAX_KEYS = 1024;                  // planned keys per workgroup
constexpr int NBK_MAX_PAGES = NBK_MAX_KEYS / 4 + 1;  // page-table window (LDS): pages of >= 4 slots
template <int D, int R, bool P2>
__global__ __launch_bounds__(64 * NBK_WAVES) void tree_attention_nodes_kernel(AttnArgs a, int runs,
                                                                            int per_run) {
  using T = bf16_t;
  constexpr int NT = 64 * NBK_WAVES;
  constexpr int P16 = 8;                       // bf16 per 16 bytes
  constexpr int ROWB = D * 2;                  // bytes per key row
  constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  constexpr int SW = CPR - 1;                  // swizzle mask
  auto vsw = [](int r) { return CPR == 16 ? ((2 * r) & SW) : (r & SW); };
  constexpr int CHB = NBK_CHUNK * ROWB;        // bytes of one chunk's K (or V)
  constexpr int SLOTB = 2 * CHB;               // K then V
  constexpr int WAVEB = R * SLOTB;             // one wave's ring
  constexpr int RPD = 1024 / ROWB;             // rows per DMA instruction (64 lanes x 16 B)
  constexpr int DPC = CHB / 1024;              // DMA instructions per chunk and tensor
  constexpr int OPS = 2 * DPC;                 // vector-memory ops per chunk
  constexpr int QSTEPS = D / 32;
  constexpr int DB = D / 16;
  constexpr int XW = DB * 4 + 2;               // exchange words per lane
  static_assert(DPC >= 1 && DPC * 1024 == CHB, "a chunk must split into whole DMAs");
  static_assert(R >= 2 && R <= 8 && (R - 1) * OPS < 64, "ring depth / vmcnt range");
  static_assert(NBK_WAVES * 64 * XW * 4 <= NBK_WAVES * WAVEB, "exchange fits in the rings");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NBK_WAVES * WAVEB];
  __shared__ int spages[NBK_MAX_PAGES];

  // workgroup -> (sequence, kv head) run, then (query head in group, node block)
  const int wg = blockIdx.x;
  const int run = (wg >> 3) / per_run * 8 + (wg & 7);
  if (run >= runs) return;  // padding of the XCD-ordered grid (uniform)
  const int k = (wg >> 3) % per_run;
  const int N = a.N;
  const int NB = (N + 15) >> 4;
  const int group = a.Hq / a.Hkv;
  const int b = run / a.Hkv, kvh = run % a.Hkv;
  const int h = kvh * group + k / NB;
  const int nb = k % NB;
  const bool appender = (h % group) == 0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int node = nb * 16 + lr;
  const int nodec = min(node, N - 1);
  const int ntree = min(N, nb * 16 + 16);      // tree keys this block's nodes may see

  const T* Qp = reinterpret_cast<const T*>(a.Q);
  const T* Ktp = reinterpret_cast<const T*>(a.Kt);
  const T* Vtp = reinterpret_cast<const T*>(a.Vt);
  T* Kcp = reinterpret_cast<T*>(a.Kc);
  T* Vcp = reinterpret_cast<T*>(a.Vc);
  const int* pt = a.page_table + (int64_t)b * a.max_pages;

  // One round trip before the stream: the length, the page table of slots
  // 0 .. max_ctx + N - 1 (into LDS), this lane's query row, its node's
  // ancestor mask and, in appending workgroups, the block's tree rows.  (The
  // host checks max_ctx + N <= NBK_MAX_KEYS and <= max_pages * P.)
  const int npages = (a.max_ctx + N + a.P - 1) / a.P;
  const int ctxb = min(max(a.ctx[b], 0), a.max_ctx);
  u32x4 qf[QSTEPS];
  {
    const T* qrow = Qp + (((int64_t)b * N + nodec) * a.Hq + h) * D;
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st)
      qf[st] = *reinterpret_cast<const u32x4*>(qrow + st * 4 * P16 + lg * P16);
  }
  const uint64_t mrow = a.mask[(int64_t)b * N + nodec];
  // appending workgroups: this block's tree rows, stored at the end
  const int t0 = nb * 16;
  const int app_items = appender ? (ntree - t0) * (D / P16) * 2 : 0;
  constexpr int APP = (16 * (D / P16) * 2 + NT - 1) / NT;  // 16-byte pieces per thread
  u32x4 app[APP];
#pragma unroll
  for (int i = 0; i < APP; ++i) {
    const int e = min(tid + i * NT, max(app_items - 1, 0));
    const int which = e / ((ntree - t0) * (D / P16)), rem = e % ((ntree - t0) * (D / P16));
    const int64_t off = (((int64_t)b * N + t0 + rem / (D / P16)) * a.Hkv + kvh) * D + (rem % (D / P16)) * P16;
    app[i] = *reinterpret_cast<const u32x4*>((which ? Vtp : Ktp) + off);
  }
  for (int e = tid; e < npages; e += NT) spages[e] = pt[e];
  // every prologue load has landed: the loop's waits then count chunk DMA only
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int tot = ctxb + ntree;
  const int nchunks = (tot + NBK_CHUNK - 1) / NBK_CHUNK;
  const int nw = nchunks > wave ? (nchunks - wave + NBK_WAVES - 1) / NBK_WAVES : 0;

  const int64_t page_elems = (int64_t)a.Hkv * a.P * D;  // one page of the cache
  const int head_elems = kvh * a.P * D;                  // this head's rows in a page
  auto cache_off = [&](int j) -> int64_t {
    const int pj = P2 ? (j >> a.lp) : j / a.P;
    const int sj = P2 ? (j & (a.P - 1)) : j - pj * a.P;
    return (int64_t)(uint32_t)spages[pj] * page_elems + (head_elems + sj * D);
  };
  const int64_t tree_base = ((int64_t)b * N * a.Hkv + kvh) * D;
  auto tree_off = [&](int j) -> int64_t {
    return tree_base + max(j - ctxb, 0) * (a.Hkv * D);
  };

  const uint32_t wave_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds +
                            wave * WAVEB;
  const uintptr_t kc_u = reinterpret_cast<uintptr_t>(Kcp), kt_u = reinterpret_cast<uintptr_t>(Ktp);
  const uintptr_t vc_u = reinterpret_cast<uintptr_t>(Vcp), vt_u = reinterpret_cast<uintptr_t>(Vtp);
  // DMA of this wave's chunk ci into ring slot `slot`.  Rows past the range
  // re-read its last key (their scores are masked).
  auto issue = [&](int ci, int slot) {
    const int key0 = (wave + NBK_WAVES * ci) * NBK_CHUNK;
    const uint32_t kd = wave_lds + slot * SLOTB;
    // the rows' page lookups first, all together (a DMA's memory clobber
    // would otherwise keep each lookup behind the previous DMA); every key
    // below max_ctx + N has its page in spages, tree rows ignore theirs
    int jj[DPC], pg[DPC];
#pragma unroll
    for (int q = 0; q < DPC; ++q) {
      jj[q] = min(key0 + q * RPD + lane / CPR, tot - 1);
      pg[q] = spages[P2 ? (jj[q] >> a.lp) : jj[q] / a.P];
    }
#pragma unroll
    for (int q = 0; q < DPC; ++q) {
      const int r = q * RPD + lane / CPR;      // chunk row this lane fills
      const int c = (lane % CPR) ^ (r & SW);   // K chunk fetched for that position
      const int cv = (lane % CPR) ^ vsw(r);    // V chunk
      const int j = jj[q];
      const bool cached = j < ctxb;
      // both offsets, then selects on values (no branch, no pointer select
      // through memory)
      const int sj = P2 ? (j & (a.P - 1)) : j - (j / a.P) * a.P;
      const int64_t coff = (int64_t)(uint32_t)pg[q] * page_elems + (head_elems + sj * D);
      const int64_t toff = tree_off(j);
      const int64_t off = cached ? coff : toff;
      const uintptr_t kbase = cached ? kc_u : kt_u, vbase = cached ? vc_u : vt_u;
      lds_dma16(reinterpret_cast<const T*>(kbase) + off + c * P16, kd + q * 1024);
      lds_dma16(reinterpret_cast<const T*>(vbase) + off + cv * P16, kd + CHB + q * 1024);
    }
  };
  // wait until at most n chunks of this wave's DMA are in flight (n < R)
  auto wait_chunks = [&](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 1 ? 1 * OPS : 0)); break;
      case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 2 ? 2 * OPS : 0)); break;
      case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 3 ? 3 * OPS : 0)); break;
      case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 4 ? 4 * OPS : 0)); break;
      case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 5 ? 5 * OPS : 0)); break;
      case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 6 ? 6 * OPS : 0)); break;
      default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(R > 7 ? 7 * OPS : 0)); break;
    }
  };

  // this lane's LDS byte offsets inside a slot: the K operand chunk of each
  // contraction step (key row lr) and the transposing-read address of each
  // 16-dim block of V (key row 4*lg + lr/4)
  int kofs[QSTEPS], vofs[DB];
#pragma unroll
  for (int st = 0; st < QSTEPS; ++st) kofs[st] = lr * ROWB + (((st * 4 + lg) ^ (lr & SW)) * 16);
  {
    const int rr = 4 * lg + (lr >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = db * 2 + ((lr & 3) >> 1);
      vofs[db] = rr * ROWB + ((c ^ vsw(rr)) * 16) + (lr & 1) * 8;
    }
  }

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  const int first = min(nw, R);
  for (int ci = 0; ci < first; ++ci) issue(ci, ci);
  for (int ci = 0; ci < nw; ++ci) {
    const int slot = ci % R;
    // chunks issued so far: min(nw, R + ci); the ones after ci stay in flight
    wait_chunks(min(nw, R + ci) - ci - 1);
    asm volatile("" ::: "memory");
    const unsigned char* ks = lds + wave * WAVEB + slot * SLOTB;
    const unsigned char* vs = ks + CHB;
    u32x4 kf[QSTEPS];
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) kf[st] = *reinterpret_cast<const u32x4*>(ks + kofs[st]);
    typedef short s4 __attribute__((ext_vector_type(4)));
    u32x2 vf[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vf[db] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (__attribute__((address_space(3))) s4*)(vs + vofs[db])));
    // the slot's operands are in registers: refill it
    __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
    asm volatile("" ::: "memory");
    if (ci + R < nw) issue(ci + R, slot);

    const int key0 = (wave + NBK_WAVES * ci) * NBK_CHUNK;
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < QSTEPS; ++st) sacc = mfma_bf16_16x16x32(kf[st], qf[st], sacc);
    // raw scores (masked: -inf); lane l holds keys key0 + 4*lg + r of node lr
    float x[4];
    float tmax = -INFINITY;
    const bool plain = key0 + NBK_CHUNK <= ctxb;  // (wave-uniform) cached keys only: no mask
    if (plain) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = sacc[r];
        tmax = fmaxf(tmax, x[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = key0 + lg * 4 + r;
        const uint32_t bit = (uint32_t)(mrow >> (uint32_t)min(max(j - ctxb, 0), 63)) & 1u;
        const bool ok = (j < tot) & ((j < ctxb) | (bit != 0u));
        x[r] = ok ? sacc[r] : -INFINITY;
        tmax = fmaxf(tmax, x[r]);
      }
    }
    tmax = rows4_max(tmax) * a.scale_log2;
    // lazy reference, as in the split kernel
    if (__builtin_amdgcn_ballot_w64(tmax > mrun + ATT_LAZY) != 0) {
      const float mnew = fmaxf(mrun, tmax);
      const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(mrun - mnew);
      lrun *= alpha;
      mrun = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    float psum = 0.f;
    if (plain) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], a.scale_log2, -mrun));
        psum += x[r];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = (x[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(x[r], a.scale_log2, -mrun));
        x[r] = p;
        psum += p;
      }
    }
    lrun += psum;
    // O^T += V^T P^T over the chunk's 16 keys (contraction index 4*lg + r)
    const u32x2 pb = {pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])};
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = mfma_bf16_16x16x16(vf[db], pb, oacc[db]);
    asm volatile("" ::: "memory");
  }
  // (every chunk issued was waited for above: no DMA is left in flight)

  // this block's tree rows (loaded in the first round trip) into cache
  // slots ctx + t
#pragma unroll
  for (int i = 0; i < APP; ++i) {
    const int e = tid + i * NT;
    if (e < app_items) {
      const int which = e / ((ntree - t0) * (D / P16)), rem = e % ((ntree - t0) * (D / P16));
      const int j = ctxb + t0 + rem / (D / P16);
      T* dst = reinterpret_cast<T*>(which ? vc_u : kc_u) + cache_off(j) + (rem % (D / P16)) * P16;
      *reinterpret_cast<u32x4*>(dst) = app[i];
    }
  }

  // merge the waves' states per node, in wave order; wave w finishes the
  // 16-dim blocks db = w, w + 8, ...
  const float ltot = rows4_sum(lrun);
  __syncthreads();                             // every wave is done with its ring
  float* xch = reinterpret_cast<float*>(lds);  // [waves][64 lanes][XW]
  {
    float* d = xch + (wave * 64 + lane) * XW;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) d[db * 4 + r] = oacc[db][r];
    d[DB * 4] = mrun;
    d[DB * 4 + 1] = ltot;
  }
  __syncthreads();
  if (node >= N) return;
  T* orow = reinterpret_cast<T*>(a.O) + (((int64_t)b * N + node) * a.Hq + h) * D;
  for (int db = wave; db < DB; db += NBK_WAVES) {
    float mm = -INFINITY;
#pragma unroll
    for (int q = 0; q < NBK_WAVES; ++q) mm = fmaxf(mm, xch[(q * 64 + lane) * XW + DB * 4]);
    float l = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NBK_WAVES; ++q) {
      const float* d = xch + (q * 64 + lane) * XW;
      const float mq = d[DB * 4];
      const float w = mq == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mq - mm);
      l += w * d[DB * 4 + 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] += w * d[db * 4 + r];
    }
    const float inv = 1.f / l;
    const u32x2 v = {pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2*>(orow + db * 16 + lg * 4) = v;
  }
}

// Merge of the split partials of one (sequence, head): O = sum_s w_s l_s o_s
// / sum_s w_s l_s with w_s = 2^(m_s - max m) and o_s the split's normalised
// output, splits in index order.  One
// workgroup per (group of 8 nodes, head, sequence); 32 lanes per node (4
// head dims each), so the grid covers the chip even at batch 1.  Up to
// CMB_BATCH splits (the smallest of 4, 8, 16 that covers the plan's split
// count) are loaded in one go together with the sequence length (splits past
// the sequence's last one are read but weighted out), so a decode-time merge
// costs one round trip.  The batch size changes no arithmetic: the splits
// are added in index order either way.
constexpr int CMB_NODES = 8;
template <typename T, int D, int CMB_BATCH>
__global__ __launch_bounds__(ATT_THREADS) void tree_attention_combine_kernel(AttnArgs a, int S) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int N = a.N;
  constexpr int D4 = D / 4;                       // lanes per node
  const int n = blockIdx.x * CMB_NODES + threadIdx.x / D4;
  if (threadIdx.x / D4 >= CMB_NODES || n >= N) return;
  const int d0 = (threadIdx.x % D4) * 4;
  const int64_t bh = (int64_t)b * a.Hq + h;
  const int ctxb = min(max(a.ctx[b], 0), a.max_ctx);
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = 0; q0 < S; q0 += CMB_BATCH) {
    PartStat ml[CMB_BATCH];
    f32x4 op[CMB_BATCH];
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j) {
      const int q = min(q0 + j, S - 1);
      ml[j] = a.ml[(bh * S + q) * N + n];
      using PT = typename PartT<T>::type;
      const PT* src = reinterpret_cast<const PT*>(a.opart) + ((bh * S + q) * N + n) * D + d0;
      if constexpr (sizeof(PT) == 2) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        const h4 v = *reinterpret_cast<const h4*>(src);
        const int sx = ml[j].s;  // undo the row's block scaling (exact)
        op[j] = f32x4{ldexpf((float)v[0], sx), ldexpf((float)v[1], sx), ldexpf((float)v[2], sx),
                      ldexpf((float)v[3], sx)};
      } else {
        op[j] = *reinterpret_cast<const f32x4*>(src);
      }
    }
    const int nsplit = (ctxb + N + a.chunk - 1) / a.chunk;
    // this batch's maximum, then the running state rescaled to it
    float Mb = M;
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j)
      if (q0 + j < nsplit) Mb = fmaxf(Mb, ml[j].m);
    const float r = (M == -INFINITY) ? 0.f : exp2f(M - Mb);
    L *= r;
    acc *= r;
#pragma unroll
    for (int j = 0; j < CMB_BATCH; ++j) {
      if (q0 + j < nsplit && ml[j].m != -INFINITY) {
        const float wl = exp2f(ml[j].m - Mb) * ml[j].l;
        L += wl;
        acc += wl * op[j];
      }
    }
    M = Mb;
  }
  const float inv = 1.f / L;
  T* orow = reinterpret_cast<T*>(a.O) + (((int64_t)b * N + n) * a.Hq + h) * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) st<T>(orow, d0 + r, acc[r] * inv);
}

}  // namespace medusa

namespace {

// Keys per split and number of splits: a split is a whole number of 64-key
// tiles, sized so that B * Hq * splits is near MEDUSA_ATTN_TARGET_WGS
// workgroups (about one to two per compute unit).
#ifndef MEDUSA_ATTN_TARGET_WGS
#define MEDUSA_ATTN_TARGET_WGS 384
#endif
#ifndef MEDUSA_ATTN_PF
#define MEDUSA_ATTN_PF 2
#endif
struct SplitPlan {
  int chunk, splits;
};
#ifndef MEDUSA_ATTN_DMA_WGS
#define MEDUSA_ATTN_DMA_WGS 256
#endif
#ifndef MEDUSA_ATTN_DMA_R
#define MEDUSA_ATTN_DMA_R 4
#endif
#ifndef MEDUSA_ATTN_KQ
#define MEDUSA_ATTN_KQ 2
#endif
// A split holds at most MEDUSA_ATTN_MAX_CHUNK keys: with many (sequence,
// head) pairs one split each would do, but in a ragged batch a pair's
// workgroup then streams its whole context, and the longest ones finish far
// behind the rest.  Capped splits keep every workgroup's work within one
// chunk; the splits past a sequence's own length exit at once, so each
// sequence takes as many as its actual context needs.
#ifndef MEDUSA_ATTN_MAX_CHUNK
#define MEDUSA_ATTN_MAX_CHUNK 1536
#endif
SplitPlan plan_splits(int B, int Hq, int N, int max_ctx, int P, int target) {
  const int64_t total = (int64_t)max_ctx + N;
  const int64_t bh = (int64_t)B * Hq;
  const int64_t want = (target + bh - 1) / bh;
  int64_t chunk = (total + want - 1) / want;
  chunk = (chunk + medusa::ATT_TILE - 1) / medusa::ATT_TILE * medusa::ATT_TILE;
  if (chunk > MEDUSA_ATTN_MAX_CHUNK) chunk = MEDUSA_ATTN_MAX_CHUNK / medusa::ATT_TILE * medusa::ATT_TILE;
  // a split's keys must span at most ATT_MAX_SPLIT_PAGES pages
  const int64_t cap = ((medusa::ATT_MAX_SPLIT_PAGES - 1) * (int64_t)P) / medusa::ATT_TILE * medusa::ATT_TILE;
  if (cap >= medusa::ATT_TILE && chunk > cap) chunk = cap;
  return {(int)chunk, (int)((total + chunk - 1) / chunk)};
}

// bf16 calls whose (sequence, query head, 16-node block) workgroups fit in
// one round of one workgroup per CU, and whose page table (slots 0 ..
// max_ctx + N - 1) fits the LDS window, take the kernel without key splits;
// with more workgroups than that the split kernel's balance over the CUs
// wins (and its one workgroup per key range needs no L2 sharing).
// Every workgroup of that kernel streams its head's whole key range, so its
// time grows with the range about 2.7 times as fast as the split kernel's
// (measured at the 7B layer: 10.9 us at 595 keys, 24.1 us at 2112, against
// 13.5 and 18.3 us for the split kernel and its merge); it takes ranges of
// up to MEDUSA_ATTN_NODES_MAX_KEYS planned keys (max_ctx + N), near the
// crossing point.
#ifndef MEDUSA_ATTN_NODES_MAX_WGS
#define MEDUSA_ATTN_NODES_MAX_WGS 256
#endif
#ifndef MEDUSA_ATTN_NODES_MAX_KEYS
#define MEDUSA_ATTN_NODES_MAX_KEYS 1024
#endif
bool nodes_path(int B, int N, int Hq, int max_ctx, int P, int dt) {
  if (dt != MEDUSA_BF16) return false;
  const int64_t wgs = (int64_t)B * Hq * ((N + 15) / 16);
  const int64_t keys = (int64_t)max_ctx + N;
  // (keys <= NBK_MAX_KEYS and P >= 4 keep the page table inside the kernel's window)
  return wgs <= MEDUSA_ATTN_NODES_MAX_WGS && keys <= MEDUSA_ATTN_NODES_MAX_KEYS &&
         keys <= medusa::NBK_MAX_KEYS && (keys + P - 1) / P <= medusa::NBK_MAX_PAGES;
}

// largest B and Hq (grid dimensions of the attention launches)
#define MEDUSA_ATTN_MAX_GRID 65535
struct WsLayout {
  size_t ml, opart, total;
};
WsLayout ws_layout(int B, int Hq, int N, int D, int S, size_t part_elem) {
  using medusa_host::align_up;
  WsLayout w;
  w.ml = 0;
  w.opart = w.ml + align_up((size_t)B * Hq * S * N * sizeof(medusa::PartStat), 256);
  w.total = w.opart + align_up((size_t)B * Hq * S * N * D * part_elem, 256);
  return w;
}

}  // namespace

extern "C" size_t medusa_tree_attention_ws(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                           int32_t D, int32_t max_ctx, int32_t P) {
  // shapes medusa_tree_attention rejects need nothing
  if (B <= 0 || N < 1 || N > MEDUSA_MAX_NODES || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 ||
      (D != 64 && D != 128) || max_ctx < 0 || P < 4 || P > 4096 || max_ctx > INT32_MAX - N ||
      B > MEDUSA_ATTN_MAX_GRID || Hq > MEDUSA_ATTN_MAX_GRID)
    return 0;
  // either dtype's plan (fp32 partials are the larger element)
  const SplitPlan p1 = plan_splits(B, Hq, N, max_ctx, P, MEDUSA_ATTN_TARGET_WGS);
  const SplitPlan p2 = plan_splits(B, Hq, N, max_ctx, P, MEDUSA_ATTN_DMA_WGS);
  return ws_layout(B, Hq, N, D, std::max(p1.splits, p2.splits), sizeof(float)).total;
}

static int32_t tree_attention_impl(const char* fn, const void* Q, const void* Kt, const void* Vt,
                                   void* Kc, void* Vc, const int32_t* page_table, int32_t max_pages,
                                   int32_t P, const int32_t* ctx, int32_t max_ctx,
                                   const uint64_t* mask, int32_t B, int32_t N, int32_t Hq,
                                   int32_t Hkv, int32_t D, float scale, int32_t dt, void* O,
                                   void* ws, size_t ws_bytes, void* stream);

extern "C" int32_t medusa_tree_attention_splits(int32_t B, int32_t N, int32_t Hq, int32_t Hkv,
                                                int32_t D, int32_t max_ctx, int32_t P,
                                                int32_t dt) {
  if (medusa_tree_attention_ws(B, N, Hq, Hkv, D, max_ctx, P) == 0 ||
      (dt != MEDUSA_F32 && dt != MEDUSA_BF16))
    return -1;
  if (nodes_path(B, N, Hq, max_ctx, P, dt)) return 0;
  return plan_splits(B, Hq, N, max_ctx, P,
                     dt == MEDUSA_BF16 ? MEDUSA_ATTN_DMA_WGS : MEDUSA_ATTN_TARGET_WGS)
      .splits;
}

extern "C" int32_t medusa_tree_attention(const void* Q, const void* Kt, const void* Vt, void* Kc,
                                         void* Vc, const int32_t* page_table, int32_t max_pages,
                                         int32_t P, const int32_t* ctx, int32_t max_ctx,
                                         const uint64_t* mask, int32_t B, int32_t N, int32_t Hq,
                                         int32_t Hkv, int32_t D, float scale, int32_t dt,
                                         void* O, void* ws, size_t ws_bytes, void* stream) {
  return tree_attention_impl("medusa_tree_attention", Q, Kt, Vt, Kc, Vc, page_table, max_pages, P,
                             ctx, max_ctx, mask, B, N, Hq, Hkv, D, scale, dt, O, ws, ws_bytes,
                             stream);
}

// ---------------------------------------------------------------------------
// The variant that allocates nothing, for callers that cannot allocate (code
// under graph capture, tight serving loops): the split partials live in a
// file-scope device array of fixed size, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): the device address comes
// from hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
static constexpr size_t kAttnScratchBytes = MEDUSA_ATTN_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, or null

// the current device's address of `scratch` (taken on first use), or null
// with the error recorded
void* scratch_ptr(const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    medusa_host::fail(MEDUSA_ERR_HIP, "%s: no current device (or device id %d >= %d)", fn, dev,
                      kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      medusa_host::fail(MEDUSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn,
                        dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int32_t medusa_tree_attention_noalloc(const void* Q, const void* Kt, const void* Vt,
                                                 void* Kc, void* Vc, const int32_t* page_table,
                                                 int32_t max_pages, int32_t P, const int32_t* ctx,
                                                 int32_t max_ctx, const uint64_t* mask, int32_t B,
                                                 int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                                 float scale, int32_t dt, void* O, void* stream) {
  using namespace medusa_host;
  const char* fn = "medusa_tree_attention_noalloc";
  const size_t need = medusa_tree_attention_ws(B, N, Hq, Hkv, D, max_ctx, P);
  MEDUSA_REQUIRE(need <= kAttnScratchBytes, MEDUSA_ERR_UNSUPPORTED,
                 "%s: B=%d N=%d Hq=%d D=%d max_ctx=%d need %zu bytes of split partials, more "
                 "than the fixed %zu (use medusa_tree_attention with a workspace)",
                 fn, B, N, Hq, D, max_ctx, need, kAttnScratchBytes);
  void* ws = scratch_ptr(fn);
  if (ws == nullptr) return MEDUSA_ERR_HIP;
  return tree_attention_impl(fn, Q, Kt, Vt, Kc, Vc, page_table, max_pages, P, ctx, max_ctx, mask,
                             B, N, Hq, Hkv, D, scale, dt, O, ws, kAttnScratchBytes, stream);
}

static int32_t tree_attention_impl(const char* fn, const void* Q, const void* Kt, const void* Vt,
                                   void* Kc, void* Vc, const int32_t* page_table, int32_t max_pages,
                                   int32_t P, const int32_t* ctx, int32_t max_ctx,
                                   const uint64_t* mask, int32_t B, int32_t N, int32_t Hq,
                                   int32_t Hkv, int32_t D, float scale, int32_t dt, void* O,
                                   void* ws, size_t ws_bytes, void* stream) {
  using namespace medusa_host;
  MEDUSA_REQUIRE(dt == MEDUSA_F32 || dt == MEDUSA_BF16, MEDUSA_ERR_UNSUPPORTED,
                 "%s: unknown dtype %d", fn, dt);
  MEDUSA_REQUIRE(D == 64 || D == 128, MEDUSA_ERR_UNSUPPORTED,
                 "%s: head dim %d not in {64, 128}", fn, D);
  MEDUSA_REQUIRE(N >= 1 && N <= MEDUSA_MAX_NODES, MEDUSA_ERR_UNSUPPORTED,
                 "%s: N=%d outside [1, 64]", fn, N);
  MEDUSA_REQUIRE(B >= 0 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: B=%d Hq=%d Hkv=%d (Hq must be a multiple of Hkv)", fn, B, Hq,
                 Hkv);
  MEDUSA_REQUIRE(B <= MEDUSA_ATTN_MAX_GRID && Hq <= MEDUSA_ATTN_MAX_GRID && max_ctx <= INT32_MAX - N,
                 MEDUSA_ERR_UNSUPPORTED, "%s: B=%d or Hq=%d above %d, or max_ctx=%d too large", fn,
                 B, Hq, MEDUSA_ATTN_MAX_GRID, max_ctx);
  MEDUSA_REQUIRE(P >= 1 && max_pages >= 1 && max_ctx >= 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: P=%d max_pages=%d max_ctx=%d", fn, P, max_pages, max_ctx);
  MEDUSA_REQUIRE(P >= 4 && P <= 4096, MEDUSA_ERR_UNSUPPORTED,
                 "%s: page size %d outside [4, 4096]", fn, P);
  MEDUSA_REQUIRE((int64_t)max_ctx + N <= (int64_t)max_pages * P, MEDUSA_ERR_INVALID_ARG,
                 "%s: max_ctx + N = %d exceeds max_pages * P = %lld", fn,
                 max_ctx + N, (long long)max_pages * P);
  MEDUSA_REQUIRE(scale > 0.f && scale < 1e30f, MEDUSA_ERR_INVALID_ARG,
                 "%s: scale must be positive and finite", fn);
  if (B == 0) return MEDUSA_OK;
  MEDUSA_REQUIRE(Q && Kt && Vt && Kc && Vc && page_table && ctx && mask && O,
                 MEDUSA_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  MEDUSA_REQUIRE(((uintptr_t)Q | (uintptr_t)Kt | (uintptr_t)Vt | (uintptr_t)Kc | (uintptr_t)Vc) %
                         16 == 0,
                 MEDUSA_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  const SplitPlan p = plan_splits(B, Hq, N, max_ctx, P,
                                  dt == MEDUSA_BF16 ? MEDUSA_ATTN_DMA_WGS : MEDUSA_ATTN_TARGET_WGS);
  const WsLayout L = ws_layout(B, Hq, N, D, p.splits, sizeof(float));
  MEDUSA_REQUIRE(ws != NULL && ws_bytes >= L.total, MEDUSA_ERR_WORKSPACE,
                 "%s: workspace %zu < %zu bytes", fn, ws_bytes, L.total);
  MEDUSA_REQUIRE((uintptr_t)ws % 256 == 0, MEDUSA_ERR_INVALID_ARG,
                 "%s: ws must be 256-byte aligned", fn);

  medusa::AttnArgs a;
  a.Q = Q; a.Kt = Kt; a.Vt = Vt; a.Kc = Kc; a.Vc = Vc;
  a.page_table = page_table; a.ctx = ctx; a.mask = mask; a.O = O;
  a.ml = (medusa::PartStat*)((char*)ws + L.ml);
  a.opart = (char*)ws + L.opart;
  a.max_pages = max_pages; a.P = P; a.B = B; a.N = N; a.Hq = Hq; a.Hkv = Hkv;
  a.lp = (P & (P - 1)) == 0 ? __builtin_ctz((unsigned)P) : -1;
  a.chunk = p.chunk;
  a.max_ctx = max_ctx;
  a.scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)p.splits, (unsigned)Hq, (unsigned)B);
  dim3 cgrid((unsigned)((N + medusa::CMB_NODES - 1) / medusa::CMB_NODES), (unsigned)Hq, (unsigned)B);
  hipStream_t st = (hipStream_t)stream;
  const dim3 blk(medusa::ATT_THREADS);
  constexpr int PF = MEDUSA_ATTN_PF;
  // split batch of the merge: 4, 8 or 16 (at 7 splits a batch of 8 measured
  // faster than 16: fewer registers and no clamped re-reads)
#define MEDUSA_ATT_COMBINE(T, DD)                                                            \
  do {                                                                                       \
    if (p.splits <= 4)                                                                       \
      hipLaunchKernelGGL((medusa::tree_attention_combine_kernel<T, DD, 4>), cgrid, blk, 0, st, a, p.splits); \
    else if (p.splits <= 8)                                                                  \
      hipLaunchKernelGGL((medusa::tree_attention_combine_kernel<T, DD, 8>), cgrid, blk, 0, st, a, p.splits); \
    else                                                                                     \
      hipLaunchKernelGGL((medusa::tree_attention_combine_kernel<T, DD, 16>), cgrid, blk, 0, st, a, p.splits); \
  } while (0)
#define MEDUSA_ATT_LAUNCH(KERNEL, T, DD)                                                     \
  do {                                                                                       \
    hipLaunchKernelGGL((KERNEL), grid, blk, 0, st, a);                                       \
    if (p.splits > 1) MEDUSA_ATT_COMBINE(T, DD);                                             \
  } while (0)
  constexpr int RD = MEDUSA_ATTN_DMA_R;
  if (nodes_path(B, N, Hq, max_ctx, P, dt)) {
    // XCD-ordered grid: runs of (sequence, kv head), each of group * NB
    // workgroups, dealt to the 8 XCDs in turn (padding exits at once)
    const int NB = (N + 15) / 16;
    const int runs = B * Hkv, per_run = (Hq / Hkv) * NB;
    const dim3 ngrid((unsigned)(((runs + 7) / 8) * 8 * per_run));
    const dim3 nblk(64 * medusa::NBK_WAVES);
    const bool p2 = a.lp >= 0;
    if (D == 128 && p2)
      hipLaunchKernelGGL((medusa::tree_attention_nodes_kernel<128, 2, true>), ngrid, nblk, 0, st, a, runs, per_run);
    else if (D == 128)
      hipLaunchKernelGGL((medusa::tree_attention_nodes_kernel<128, 2, false>), ngrid, nblk, 0, st, a, runs, per_run);
    else if (p2)
      hipLaunchKernelGGL((medusa::tree_attention_nodes_kernel<64, 4, true>), ngrid, nblk, 0, st, a, runs, per_run);
    else
      hipLaunchKernelGGL((medusa::tree_attention_nodes_kernel<64, 4, false>), ngrid, nblk, 0, st, a, runs, per_run);
    return check_launch(fn);
  }
  if (dt == MEDUSA_BF16) {
    const bool p2 = a.lp >= 0;
    // two key parts per tile (8 waves); four parts (16 waves) measured slower
    constexpr int KQ = MEDUSA_ATTN_KQ;
    constexpr int KQ64 = KQ < 2 ? KQ : 2;  // a 64-wide tile is 8 DMA blocks: at most 8 waves
    const dim3 blk8(256 * (D == 128 ? KQ : KQ64));
#define MEDUSA_ATT_LAUNCH_S(KERNEL, DD)                                                      \
  do {                                                                                       \
    hipLaunchKernelGGL((KERNEL), grid, blk8, 0, st, a);                                      \
    if (p.splits > 1) MEDUSA_ATT_COMBINE(medusa::bf16_t, DD);                                \
  } while (0)
    if (D == 128 && p2) MEDUSA_ATT_LAUNCH_S((medusa::tree_attention_stream_kernel<128, RD, KQ, true>), 128);
    else if (D == 128) MEDUSA_ATT_LAUNCH_S((medusa::tree_attention_stream_kernel<128, RD, KQ, false>), 128);
    else if (p2) MEDUSA_ATT_LAUNCH_S((medusa::tree_attention_stream_kernel<64, 2 * RD, KQ64, true>), 64);
    else MEDUSA_ATT_LAUNCH_S((medusa::tree_attention_stream_kernel<64, 2 * RD, KQ64, false>), 64);
#undef MEDUSA_ATT_LAUNCH_S
  } else {
    if (D == 128) MEDUSA_ATT_LAUNCH((medusa::tree_attention_kernel<float, 128, PF>), float, 128);
    else MEDUSA_ATT_LAUNCH((medusa::tree_attention_kernel<float, 64, PF>), float, 64);
  }
#undef MEDUSA_ATT_LAUNCH
#undef MEDUSA_ATT_COMBINE
  return check_launch(fn);
}
