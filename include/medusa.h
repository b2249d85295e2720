/*
 * libmedusa: the Medusa decode step on one AMD Instinct MI355X (gfx950).
 *
 * The step (page "Medusa Heads", Ultralytics glossary; page "Têtes de
 * décodage Medusa", section "Plongée profonde"; arXiv abstract page "Medusa:
 * Simple LLM Inference Acceleration Framework with Multiple Decoding Heads"):
 *   1. K extra heads read the final hidden state; head k scores the token at
 *      t+k+1 (medusa_heads, medusa_topk).
 *   2. The per-head top-k lists are combined as a Cartesian product into a
 *      candidate tree whose nodes share prefixes (medusa_build_tree).
 *   3. One forward pass verifies every tree node at once; an attention mask
 *      lets each node see only its ancestors (medusa_tree_attention, plus
 *      the backbone calls medusa_embed ... medusa_linear).
 *   4. The longest branch the model agrees with is kept, greedy or typical
 *      (medusa_accept), and only that branch stays in the KV cache
 *      (kv_compact); its last hidden state feeds the heads next round
 *      (medusa_gather_rows).  medusa_decode_tail does all of step 4 and
 *      the step's bookkeeping in two launches.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers are DEVICE pointers unless a parameter says "host".  Tensors are
 *   dense row-major in the layout given in brackets, innermost last.
 * - dtype: MEDUSA_F32 tensors hold float; MEDUSA_BF16 tensors hold bfloat16
 *   bit patterns (uint16).  Logits, top-k values, softmax statistics and the
 *   residual stream are always float.  Arithmetic is fp32 in both modes.
 * - Ownership: the caller allocates and frees every buffer, workspaces
 *   included; the library never allocates and keeps no state between calls.
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = default
 *   stream).  Every call only enqueues work and returns; nothing blocks the
 *   host.  Buffers must stay alive until the stream has passed the call.
 * - Errors: every call returns a medusa_status.  Arguments are validated on
 *   the host before any launch; on failure nothing is enqueued and
 *   medusa_last_error() (thread-local) describes the problem.  Values read
 *   on the device (token ids, ctx, page tables, templates, paths) are not
 *   checked: out-of-range device data is undefined behaviour.
 * - Limits: tree nodes N <= 64 (one uint64 mask per node), heads K <= 8,
 *   top-k <= 64, head dim D in {64, 128}, Hq a multiple of Hkv.
 */
#ifndef MEDUSA_H_
#define MEDUSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_INVALID_ARG = 1,   /* NULL pointer, negative size, bad template ... */
  MEDUSA_ERR_UNSUPPORTED = 2,   /* dtype, head dim or size outside the limits     */
  MEDUSA_ERR_WORKSPACE = 3,     /* workspace smaller than the *_ws query          */
  MEDUSA_ERR_HIP = 4            /* a HIP launch failed                            */
} medusa_status;

#define MEDUSA_MAX_NODES 64
#define MEDUSA_MAX_HEADS 8
#define MEDUSA_MAX_TOPK 64
#define MEDUSA_MAX_TOPK_LISTS 64   /* per-chunk top-k lists per row (vocabulary <= 64 x 4096) */
#define MEDUSA_MAX_LAYERS 128

const char* medusa_status_string(int32_t status);
const char* medusa_last_error(void);
int32_t medusa_abi_version(void);

/* ------------------------------------------------------------------------
 * Tree template check (host only).
 * The tree is the Cartesian product of per-head top-k ("Medusa Heads",
 * section "Attenzione sull'albero e accettazione").  A template fixes its
 * shape: node 0 is the root (parent -1); node i > 0 has parent[i] < i and
 * uses rank[i] of the top-k list of head depth(i).
 * parent, rank: HOST arrays [N].  Checks N in [1, 64], parent[0] == -1,
 * 0 <= parent[i] < i, depth(i) <= K, 0 <= rank[i] < topk, and distinct ranks
 * among siblings.  Returns MEDUSA_OK or MEDUSA_ERR_INVALID_ARG.
 * ---------------------------------------------------------------------- */
int32_t medusa_tree_validate(const int32_t* parent, const int32_t* rank, int32_t N,
                             int32_t K, int32_t topk);

/* ------------------------------------------------------------------------
 * medusa_tree_from_accuracy (host): the sparse tree of the most accurate
 * head combinations ("Medusa Heads", tree section: a sparse 64-node tree
 * built from the most accurate combinations beat a dense 256-node tree).
 *   accuracy [K, topk] float (host), in [0, 1]: the chance that head k+1's
 *     rank-r candidate is the right token (measured on the caller's data).
 * A combination (r1..rd), d <= K, has accuracy prod_j accuracy[j][r_j]; the
 * tree keeps the root and the N-1 most accurate combinations (ties: the
 * shallower, then the lexicographically smaller rank tuple), a prefix-closed
 * set.  Outputs (host): parent [N], rank [N] in canonical order (by depth,
 * then rank tuple; the form medusa_tree_validate accepts) and, if expected is
 * not NULL, the sum of the kept accuracies (expected accepted candidates per
 * step when the heads are independent).
 * ---------------------------------------------------------------------- */
int32_t medusa_tree_from_accuracy(const float* accuracy, int32_t K, int32_t topk, int32_t N,
                                  int32_t* parent, int32_t* rank, double* expected);

/* ------------------------------------------------------------------------
 * Generic projection  Y = epilogue(X W^T)   (nn.Linear orientation).
 * The backbone's projections and the heads' two layers ("Medusa Heads",
 * section "Come le teste prevedono i token successivi": a feed-forward layer
 * with SiLU and a residual connection, then a vocabulary projection).
 *   X [batch][M, Kd] (dtype dt, row stride Kd, batch stride x_bstride
 *     elements, 0 = shared), W [batch][N, Kd] (dt), Y [batch][M, N].
 *   epilogue:
 *     MEDUSA_EPI_NONE        Y = acc                          (Y dtype: y_f32 ? float : dt)
 *     MEDUSA_EPI_BIAS_SILU_RES  Y = R + SiLU(acc + bias)      (R = aux [batch][M, N] dt,
 *                                bias [batch][N] dt; needs N == Kd when R is X)
 *     MEDUSA_EPI_RES_ADD_F32 Y = aux + acc, Y and aux float [M, N] (may alias)
 *     MEDUSA_EPI_SWIGLU      W holds gate and up rows interleaved in blocks of
 *                            16 (block j: gate rows 16j..16j+15 then up rows);
 *                            Y [M, N/2] = SiLU(gate) * up   (dt)
 *   Every reduction runs in a fixed order: equal inputs, shapes and batch
 *   give bitwise equal outputs.  The launch plan is a function of (M, Kd, N,
 *   dt), and of the batch only where a batch that shares its activation rows
 *   (x_bstride 0) is planned as one projection onto its stacked weights; the
 *   large-row tilings (bf16, M >= 256) all accumulate in the same order, so
 *   there a batch element's outputs do not depend on the batch.
 * Kd must be a multiple of 8 (bf16) or 4 (f32); X, W, Y, aux and bias
 * 16-byte aligned (MEDUSA_ERR_INVALID_ARG otherwise).
 * ws: medusa_linear_ws(M, Kd, N, batch, dt) bytes of scratch for contraction
 * split partials (0 for shapes that do not split; then ws may be NULL).
 * ---------------------------------------------------------------------- */
typedef enum {
  MEDUSA_EPI_NONE = 0,
  MEDUSA_EPI_BIAS_SILU_RES = 1,
  MEDUSA_EPI_RES_ADD_F32 = 2,
  MEDUSA_EPI_SWIGLU = 3
} medusa_epilogue;

size_t medusa_linear_ws(int64_t M, int64_t Kd, int64_t N, int32_t batch, int32_t dt);
int32_t medusa_linear(const void* X, int64_t x_bstride, int64_t M, int64_t Kd, const void* W,
                      int64_t N, int32_t batch, int32_t dt, int32_t epilogue, const void* bias,
                      const void* aux, void* Y, int32_t y_f32, void* ws, size_t ws_bytes,
                      void* stream);

/* ------------------------------------------------------------------------
 * medusa_heads: K Medusa heads on M hidden rows, plus per-head top-k.
 * ("Medusa Heads", section "Come le teste prevedono i token successivi":
 *  head k reads the final hidden state h that lm_head reads and scores the
 *  token at t+k+1 as  logits_k = W2_k (h + SiLU(W1_k h + b1_k)).)
 *   X [M, H] (dt), W1 [K, H, H] (row = output feature), b1 [K, H] (dt),
 *   W2 [K, V, H] (dt, no bias).
 *   logits: [K, M, V] float, or NULL to keep them internal.
 *   topk (0..64): if > 0, topk_ids [K, M, topk] int32 and topk_vals
 *   [K, M, topk] float receive each row's largest logits, value descending,
 *   equal values ordered by lower token id.
 *   ws: device workspace of at least medusa_heads_ws(...) bytes.
 * With W1 = 0, b1 = 0 and W2_k = lm_head the logits equal
 * medusa_linear(X, lm_head) bit for bit.
 * ---------------------------------------------------------------------- */
size_t medusa_heads_ws(int64_t M, int64_t H, int32_t K, int64_t V, int32_t topk, int32_t dt);
/* medusa_heads_lists: medusa_heads with the top-k's first stage only, for a
 * consumer that merges the lists itself (medusa_tree_embed with lists > 1):
 * list_ids [K, M, S, topk] int32 and list_vals [K, M, S, topk] float, S =
 * medusa_topk_lists(V), hold each 4096-wide vocabulary chunk's top-k of each
 * row (value descending, ties by lower token id); the row's top-k is the
 * top-k of its S lists.  1 <= topk <= min(64, V); the rest as medusa_heads
 * (its workspace query included). */
int32_t medusa_heads_lists(const void* X, int64_t M, int64_t H, int32_t K, const void* W1,
                           const void* b1, const void* W2, int64_t V, int32_t dt, int32_t topk,
                           int32_t* list_ids, float* list_vals, void* ws, size_t ws_bytes,
                           void* stream);
int32_t medusa_heads(const void* X, int64_t M, int64_t H, int32_t K, const void* W1,
                     const void* b1, const void* W2, int64_t V, int32_t dt, float* logits,
                     int32_t topk, int32_t* topk_ids, float* topk_vals, void* ws,
                     size_t ws_bytes, void* stream);

/* medusa_topk: top-k of each float row ("Medusa Heads", tree section: the
 * heads' best guesses).  logits [R, V] float -> ids [R, k] int32, vals [R, k]
 * float; order value descending, ties by lower index; 1 <= k <= 64, k <= V.
 * ws: medusa_topk_ws(R, V, k) bytes (0 when V <= 4096; then ws may be NULL). */
size_t medusa_topk_ws(int64_t R, int64_t V, int32_t k);
/* The top-k runs in two stages: each 4096-wide chunk of a row keeps its own
 * top-k list (the same order), then the row's lists are merged.  The number
 * of chunk lists per row: ceil(V / 4096) (0 for V outside [1, 2^31 - 1]). */
int32_t medusa_topk_lists(int64_t V);
int32_t medusa_topk(const float* logits, int64_t R, int64_t V, int32_t k, int32_t* ids,
                    float* vals, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * medusa_build_tree: fill B tree templates with tokens ("Medusa Heads",
 * section "Attenzione sull'albero e accettazione": the Cartesian product of
 * the heads' top-k forms a prefix-sharing tree; each token sees only its
 * ancestors).
 *   parent, rank [B, N] int32 (templates, validated beforehand on the host)
 *   root_tok [B] int32: the model's own next token (node 0)
 *   topk_ids [K, B, topk] int32: node i at depth d >= 1 gets
 *     topk_ids[d-1, b, rank[b, i]]
 *   ctx [B] int32: committed tokens in the cache
 * Outputs tokens [B, N] int32, pos [B, N] int32 = ctx + depth, mask [B, N]
 * uint64 with bit j set iff node j is node i or one of its ancestors.
 * ---------------------------------------------------------------------- */
int32_t medusa_build_tree(int32_t B, int32_t N, const int32_t* parent, const int32_t* rank,
                          const int32_t* root_tok, const int32_t* topk_ids, int32_t K,
                          int32_t topk, const int32_t* ctx, int32_t* tokens, int32_t* pos,
                          uint64_t* mask, void* stream);

/* ------------------------------------------------------------------------
 * medusa_tree_attention: one tree-masked attention pass ("Medusa Heads",
 * tree section: all candidate tokens are appended at once and a mask lets
 * each see only its ancestors, so every branch is checked in parallel; arXiv
 * abstract page: tree-based attention).
 *   Q  [B, N, Hq, D] (dt)   queries of the N tree nodes (RoPE applied)
 *   Kt, Vt [B, N, Hkv, D]   keys / values of the tree nodes
 *   Kc, Vc [pages, Hkv, P, D]  paged cache pools; logical slot s of sequence
 *          b lives in page page_table[b, s / P] at row s % P (4 <= P <= 4096)
 *   page_table [B, max_pages] int32; ctx [B] int32 committed tokens
 *   max_ctx: host-side upper bound of every ctx[b] (sizes the grid)
 *   mask [B, N] uint64 (from medusa_build_tree)
 *   O  [B, N, Hq, D] (dt)
 * Node i of sequence b attends, with scores q.k * scale and an fp32 softmax,
 * to cache slots 0..ctx[b]-1 and to tree node j iff bit j of mask[b, i].
 * Query head h uses kv head h / (Hq / Hkv).  The call also stores Kt, Vt into
 * cache slots ctx[b] .. ctx[b]+N-1 (those pages must exist in page_table).
 * ws: medusa_tree_attention_ws(...) bytes of scratch (split partials); no
 * initialisation needed.  Calls sharing one ws must not overlap in time.
 * ---------------------------------------------------------------------- */
size_t medusa_tree_attention_ws(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t max_ctx, int32_t P);
int32_t medusa_tree_attention(const void* Q, const void* Kt, const void* Vt, void* Kc, void* Vc,
                              const int32_t* page_table, int32_t max_pages, int32_t P,
                              const int32_t* ctx, int32_t max_ctx, const uint64_t* mask,
                              int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                              float scale, int32_t dt, void* O, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * medusa_tree_attention_splits: how medusa_tree_attention would run a call
 * of these shapes (the plan depends on them only, so equal shapes always
 * take the same arithmetic path).
 *   0: one launch, no key splits: one workgroup per (sequence, query head,
 *      16-node block) over its head's whole key range (bf16 calls with at
 *      most 256 such workgroups and at most 1024 planned keys max_ctx + N);
 *   S >= 1: S key splits per (sequence, head), plus a merge launch when
 *      S > 1;
 *   -1: shapes or dtype medusa_tree_attention rejects, or B = 0 (a call
 *       that enqueues nothing).
 * ---------------------------------------------------------------------- */
int32_t medusa_tree_attention_splits(int32_t B, int32_t N, int32_t Hq, int32_t Hkv, int32_t D,
                                     int32_t max_ctx, int32_t P, int32_t dt);

/* ------------------------------------------------------------------------
 * medusa_tree_attention_noalloc: medusa_tree_attention for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments and results, minus the
 * workspace: the split partials live in a fixed device array inside the
 * library, MEDUSA_ATTN_NOALLOC_MAX_BYTES bytes on each GPU it runs on, held
 * until the process ends.  The call allocates and frees nothing.
 *   Sizes whose medusa_tree_attention_ws(...) exceeds the array return
 *   MEDUSA_ERR_UNSUPPORTED (nothing is enqueued).  The first call on a
 *   device looks up the array's device address (hipGetSymbolAddress); a
 *   failure there returns MEDUSA_ERR_HIP.
 *   Every call on one GPU shares that GPU's array (it keeps the last call's
 *   partials; no call needs it cleared): calls that overlap in time on one
 *   GPU, from any stream or thread, race and give undefined results.  Calls
 *   whose plan is the one launch without key splits
 *   (medusa_tree_attention_splits(...) == 0) write no partials and leave
 *   the array untouched.
 * ---------------------------------------------------------------------- */
#define MEDUSA_ATTN_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int32_t medusa_tree_attention_noalloc(const void* Q, const void* Kt, const void* Vt, void* Kc,
                                      void* Vc, const int32_t* page_table, int32_t max_pages,
                                      int32_t P, const int32_t* ctx, int32_t max_ctx,
                                      const uint64_t* mask, int32_t B, int32_t N, int32_t Hq,
                                      int32_t Hkv, int32_t D, float scale, int32_t dt, void* O,
                                      void* stream);

/* ------------------------------------------------------------------------
 * medusa_accept: longest accepted branch per sequence ("Medusa Heads", tree
 * section: the longest branch the model accepts is kept; greedy keeps a
 * candidate equal to the model's top choice; typical acceptance keeps a
 * candidate whose base-model probability exceeds an entropy-linked
 * threshold).
 *   logits [B, N, V] float: verification logits, row p scores the token that
 *     follows node p
 *   tokens, parent [B, N] int32
 *   K: number of heads = longest possible branch minus one; path has K+1 slots
 *   mode 0 greedy: node i accepted iff its parent is and tokens[i] ==
 *     argmax(logits[parent]) (lowest id on ties)
 *   mode 1 typical: iff its parent is and p(tokens[i]) > min(epsilon,
 *     delta * exp(-H(p))), p = softmax(logits[parent] / temperature),
 *     H natural-log entropy
 * Outputs: accept_len [B] = depth of the deepest accepted node (lowest index
 * on ties); path [B, K+1] node indices root..best, padded with -1;
 * next_token [B] = argmax of logits[best].
 * ws: medusa_accept_ws(B, N) bytes.
 * ---------------------------------------------------------------------- */
size_t medusa_accept_ws(int32_t B, int32_t N);
int32_t medusa_accept(const float* logits, int64_t V, const int32_t* tokens,
                      const int32_t* parent, int32_t B, int32_t N, int32_t K, int32_t mode,
                      float temperature, float epsilon, float delta, int32_t* accept_len,
                      int32_t* path, int32_t* next_token, void* ws, size_t ws_bytes,
                      void* stream);

/* ------------------------------------------------------------------------
 * medusa_accept_sample: sampled verification, the rejection sampling against
 * the base model that keeps Medusa-1's output distribution that of the base
 * model ("Têtes de décodage Medusa", section "Plongée profonde" and its
 * "Questions fréquemment posées" entry on lossless acceleration).
 * The candidates are fixed top-k tokens, so testing them one by one against
 * p = softmax(logits[node] / temperature), renormalised over the tokens not
 * yet rejected, takes child c with probability p(token c) and otherwise ends
 * the branch with a draw from the rest: the law of one draw z ~ p at every
 * visited node.  That is what is computed: for every node u one draw z_u by
 * Gumbel-max, argmax over v of fl(fl(logits[u, v] * fl(1 / temperature)) +
 * G), G = -log(-log(u_v)) in float, u_v = ((w >> 41) + 1/2) / 2^23 where w
 * is word v % 4 of Philox4x64-10 (Salmon et al., SC 2011) with key (seed,
 * step) and counter (v / 4, u, b, 0); lowest v on a tie.  Node i is accepted
 * iff its parent is and tokens[i] == z_parent; accept_len, path as for
 * medusa_accept; next_token [B] = z at the deepest accepted node.
 *   rng [2] uint64 (device): (seed, step).  The call draws with that key and
 *     then adds 1 to step on the device, so a captured decode step replays
 *     with fresh noise.  Calls sharing one rng buffer are ordered by their
 *     stream.  A one-node tree (N = 1, parent [-1]) samples a plain next
 *     token.
 *   temperature > 0.  ws: medusa_accept_ws(B, N) bytes.
 * ---------------------------------------------------------------------- */
int32_t medusa_accept_sample(const float* logits, int64_t V, const int32_t* tokens,
                             const int32_t* parent, int32_t B, int32_t N, int32_t K,
                             float temperature, uint64_t* rng, int32_t* accept_len,
                             int32_t* path, int32_t* next_token, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * kv_compact: keep only the accepted branch in every layer's cache (the
 * branch the model accepted is kept: "Medusa Heads", tree section).
 * For d = 0..accept_len[b]: slot ctx[b]+d <- slot ctx[b]+path[b, d], K and V,
 * all layers, all kv heads; every read happens before any write.
 *   Kc, Vc: HOST arrays of L device pointers, one [pages, Hkv, P, D] pool per
 *   layer (L <= 128); page_table [B, max_pages]; ctx [B]; path [B, K+1];
 *   accept_len [B].
 * Outputs: src_slots, dst_slots [B, K+1] int32 (logical slots, -1 padded;
 * either may be NULL), new_ctx [B] = ctx + accept_len + 1 (must not alias ctx).
 * ---------------------------------------------------------------------- */
int32_t kv_compact(void* const* Kc, void* const* Vc, int32_t L, const int32_t* page_table,
                   int32_t max_pages, int32_t P, const int32_t* ctx, const int32_t* path,
                   const int32_t* accept_len, int32_t B, int32_t K, int32_t Hkv, int32_t D,
                   int32_t dt, int32_t* src_slots, int32_t* dst_slots, int32_t* new_ctx,
                   void* stream);

/* ------------------------------------------------------------------------
 * Backbone pieces of the verification forward pass (the base model checks
 * the whole tree in one pass: "Têtes de décodage Medusa", section "Plongée
 * profonde").  Llama-style: RMSNorm, rotary positions, SwiGLU.
 * ---------------------------------------------------------------------- */

/* out [M, H] float = table[tokens[m], :]; table [V, H] (dt). */
int32_t medusa_embed(const int32_t* tokens, int64_t M, const void* table, int64_t V, int64_t H,
                     int32_t dt, float* out, void* stream);

/* out [M, H] (dt) = x / sqrt(mean(x^2) + eps) * gain; x float [M, H] (16-byte
 * aligned, H a multiple of 4, H <= 8192); gain [H] (dt) or NULL for 1; gain
 * and out aligned to four elements (8 bytes bf16, 16 bytes fp32). */
int32_t medusa_rmsnorm(const float* x, int64_t M, int64_t H, const void* gain, float eps,
                       int32_t dt, void* out, void* stream);

/* medusa_tree_embed: medusa_build_tree, then medusa_embed of the B*N tree
 * tokens and medusa_rmsnorm of those rows with gain (the first block's norm),
 * in one launch; the outputs equal the three calls' bit for bit.  Arguments
 * as there: tokens, pos [B, N], mask [B, N]; x [B*N, H] float (16-byte
 * aligned) = the embedding rows; h [B*N, H] (dt) = RMSNorm(x) * gain (gain
 * NULL for 1).  H a multiple of 4, H <= 8192; table, gain and h aligned to
 * four elements.  lists = 1: topk_ids [K, B, topk] are the heads' top-k lists
 * (topk_vals unused, may be NULL).  lists = S > 1 (<= 64): topk_ids and
 * topk_vals [K, B, S, topk] are per-chunk lists as medusa_heads_lists writes
 * them, and each node's token is found by merging its row's lists in the
 * launch; the outputs equal those from the merged lists bit for bit. */
int32_t medusa_tree_embed(int32_t B, int32_t N, const int32_t* parent, const int32_t* rank,
                          const int32_t* root_tok, const int32_t* topk_ids,
                          const float* topk_vals, int32_t lists, int32_t K,
                          int32_t topk, const int32_t* ctx, int32_t* tokens, int32_t* pos,
                          uint64_t* mask, const void* table, int64_t V, int64_t H, int32_t dt,
                          const void* gain, float eps, float* x, void* h, void* stream);

/* The residual projection of a pre-norm block followed by the next block's
 * RMSNorm: x [M, N] float (16-byte aligned, updated in place) += X W^T with
 * X [M, Kd] and W [N, Kd] (dt), then out [M, N] (dt) = RMSNorm(x) * gain
 * (gain [N] dt or NULL for 1; N a multiple of 4, N <= 8192; gain and out
 * aligned to four elements).  The results
 * equal, bit for bit, medusa_linear(X, W, MEDUSA_EPI_RES_ADD_F32, aux = Y = x)
 * followed by medusa_rmsnorm(x, gain, eps, out): where the projection splits
 * its contraction, the split sum, the residual add and the norm run in one
 * pass per row instead of two launches.  out must not alias x, X or W.
 * ws: medusa_linear_ws(M, Kd, N, 1, dt) bytes (NULL when that is 0). */
int32_t medusa_linear_rmsnorm(const void* X, int64_t M, int64_t Kd, const void* W, int64_t N,
                              int32_t dt, float* x, const void* gain, float eps, void* out,
                              void* ws, size_t ws_bytes, void* stream);

/* The QKV projection with the rotary positions of medusa_qkv_rope fused in:
 * q [M, Hq, D], k [M, Hkv, D], v [M, Hkv, D] (dt) from X [M, Kd] (dt) and
 * W [(Hq + 2 Hkv) D, Kd] whose q and k head rows are pair-interleaved: row
 * 2j of a head holds the weights of element j and row 2j + 1 those of
 * element j + D/2 (the v rows keep their order).  Bit for bit equal to the
 * projection with the plain row order (medusa_linear, stored in dt) followed
 * by medusa_qkv_rope.  Where the projection takes the block-range kernel
 * without a contraction split, the rotation runs in its epilogue; otherwise
 * the projection goes to ws and the rotary pass reads it there.
 * ws: medusa_linear_qkv_rope_ws(...) bytes, 256-byte aligned (NULL when 0).
 * X, W, q, k, v 16-byte aligned; D a multiple of 8 up to 128; base > 1. */
size_t medusa_linear_qkv_rope_ws(int64_t M, int64_t Kd, int32_t Hq, int32_t Hkv, int32_t D,
                                 int32_t dt);
int32_t medusa_linear_qkv_rope(const void* X, int64_t M, int64_t Kd, const void* W, int32_t Hq,
                               int32_t Hkv, int32_t D, const int32_t* pos, float base, int32_t dt,
                               void* q, void* k, void* v, void* ws, size_t ws_bytes, void* stream);

/* Split qkv [M, (Hq + 2 Hkv) * D] (dt) into q [M, Hq, D], k [M, Hkv, D],
 * v [M, Hkv, D] and rotate q and k by position pos[m] (rotate-half pairs
 * (j, j + D/2), angle pos * base^(-2j/D)).  qkv, q, k, v 16-byte aligned;
 * D a multiple of 8 up to 128; base > 1. */
int32_t medusa_qkv_rope(const void* qkv, int64_t M, int32_t Hq, int32_t Hkv, int32_t D,
                        const int32_t* pos, float base, int32_t dt, void* q, void* k, void* v,
                        void* stream);

/* out [M, F] (dt) = SiLU(gu[:, :F]) * gu[:, F:], gu [M, 2F] (dt). */
int32_t medusa_swiglu(const void* gu, int64_t M, int64_t F, int32_t dt, void* out, void* stream);

/* out [B, H] (dt) = h[b, path[b, accept_len[b]], :] with h [B, N, H] (dt),
 * path [B, K+1]: the kept branch's last hidden state, fed to the heads. */
int32_t medusa_gather_rows(const void* h, int32_t B, int32_t N, int64_t H, const int32_t* path,
                           const int32_t* accept_len, int32_t K, int32_t dt, void* out,
                           void* stream);

/* ------------------------------------------------------------------------
 * medusa_decode_tail: the end of one decode step in two launches, with no
 * host involvement: acceptance (greedy, typical or sampled, as medusa_accept
 * and medusa_accept_sample), the cache compaction of kv_compact, the kept
 * branch's last hidden state (medusa_gather_rows), and the commit of the
 * step.  The longest accepted branch is kept and its tokens plus one are
 * emitted ("Medusa Heads", section "Attenzione sull'albero e accettazione";
 * sampled verification: "Têtes de décodage Medusa", section "Plongée
 * profonde").  The outputs equal those of the separate calls bit for bit.
 *   logits [B, N, V] float; tokens, parent [B, N]; mode 0 greedy, 1 typical
 *     (temperature, epsilon, delta), 2 sampled (temperature, rng [2] as for
 *     medusa_accept_sample; step advanced by one).  K <= 8.
 *   Kc, Vc: HOST arrays of L device pools [pages, Hkv, P, D] (dt), page_table
 *     [B, max_pages].
 *   hidden [B, N, H] (dt) -> h_best [B, H] = hidden[b, kept node]; H * element
 *     size a multiple of 16 bytes, both 16-byte aligned.
 *   ctx [B] (in/out): advanced by accept_len + 1.  root [B] (out): the next
 *     root token (= next_token).  accept_len [B], path [B, K+1], next_token [B]
 *     as medusa_accept.
 *   log [B, 2 + 2*cap] int32 (in/out), per sequence: [0] tokens emitted so
 *     far, [1] steps so far, [2, 2+cap) the emitted tokens (path order,
 *     accept_len + 1 per step), [2+cap, 2+2cap) each step's accept_len.
 *     Entries past cap are dropped; the counts keep counting.  Zero it before
 *     a generation.
 *   ws: medusa_decode_tail_ws(B, N) bytes.  Its last part holds per-sequence
 *     counters that must be zero before the first call (zero-fill the
 *     workspace once); every call leaves them zero.  The counters sit at an
 *     offset that depends on B only (after the statistics of a 64-node
 *     tree), so one workspace may serve calls with the same B and any N.
 *     Calls sharing a workspace must be ordered by their stream.
 * ---------------------------------------------------------------------- */
size_t medusa_decode_tail_ws(int32_t B, int32_t N);
int32_t medusa_decode_tail(const float* logits, int64_t V, const int32_t* tokens,
                           const int32_t* parent, int32_t B, int32_t N, int32_t K, int32_t mode,
                           float temperature, float epsilon, float delta, uint64_t* rng,
                           void* const* Kc, void* const* Vc, int32_t L, const int32_t* page_table,
                           int32_t max_pages, int32_t P, int32_t Hkv, int32_t D, int32_t dt,
                           const void* hidden, int64_t H, void* h_best, int32_t* ctx,
                           int32_t* root, int32_t* accept_len, int32_t* path, int32_t* next_token,
                           int32_t* log, int32_t cap, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H_ */
