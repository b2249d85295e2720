"""CPU oracle for the Medusa decode step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The library under
``speculative_decoding_02_amd/`` never imports it, and it imports nothing from
the library: the two share only the seeded input generators in ``synth``.

What it computes is the decode step that the page "Medusa Heads" (Ultralytics
glossary) describes in its sections "Come le teste prevedono i token
successivi" (how the heads predict the next tokens) and "Attenzione sull'albero
e accettazione" (tree attention and acceptance), with the one-pass tree
verification of "Têtes de décodage Medusa" (section "Plongée profonde") and of
the arXiv abstract page "Medusa: Simple LLM Inference Acceleration Framework
with Multiple Decoding Heads".

Form
----
* Plain numpy in float64.  Inputs given as float32 or bfloat16 values are
  upcast exactly.  A matmul (``@``), ``exp``/``log`` and a stable sort are the
  only library primitives used; there is no blocking, fusion or reordering.
* Integer decisions that floating point takes (top-k order, argmax, typical
  acceptance) are taken on logits rounded to float32, the precision the
  library produces logits in: ties in float32 go to the lower token id.
* Loops are plain Python where the sizes are tiny (per node, per head).

Pins (tests/test_oracle_*.py, all ``-m "not gpu"``)
-------------------------------------------------
heads:        zero-initialised heads reproduce lm_head logits exactly (the
              page's printed ``[True, True, True]``); nn.Linear semantics
              via torch; closed form for W1 = 0, b1 = c, W2 = I.
topk:         brute-force repeated max with planted ties.
build_tree:   hand-derived 9-node template of the top-2 x top-3 example
              (tests/golden/c1_tree.json); 6 candidates = itertools.product.
tree_attention: chain tree = causal attention (torch SDPA, fp64); root-only
              = decode attention; Q = 0 gives the mean of visible V; ancestor
              walk + SDPA with an explicit boolean mask on random trees.
decoder:      logits equal Hugging Face ``LlamaForCausalLM`` (fp64) on the
              same weights; sequential greedy equals its greedy ``generate``.
accept_greedy / medusa_generate: Medusa greedy output equals sequential
              greedy decoding on the tiny random model (the lossless claim);
              cheating heads accept the full depth; never-matching heads
              accept nothing.
accept_typical: special cases only (threshold 0 accepts everything; a
              near-one-hot distribution reproduces greedy; monotone in
              epsilon and delta).  The threshold FORMULA ``min(eps,
              delta*exp(-H))`` is not printed on the pages, which only tie
              the threshold to the entropy: parity unpinned for it.
accept_sample: the Philox4x64-10 generator equals numpy's Philox bit
              generator (numpy advances the counter before each block);
              Gumbel-max draws follow softmax(z/T) (chi-square); the first
              and second emitted tokens of a sampled tree step follow the base
              model's distributions (the lossless claim, chi-square); a tiny
              temperature reproduces greedy acceptance.
kv_compact:   compacted cache equals the cache of sequential decoding of the
              same tokens; hand example path (0, 2, 7).
sparse_tree:  hand-derived 5-node example (tests/golden/sparse_tree.json);
              brute force over every prefix-closed tree of n nodes: the kept
              set has the largest expected acceptance; kept sets are
              prefix-closed and pass the template checks.
"""
from __future__ import annotations

import itertools

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# heads ("Medusa Heads", section on how the heads predict the next tokens)
# ----------------------------------------------------------------------------
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z)  (torch's F.silu)."""
    z = np.asarray(z, dtype=F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def linear(x, w, b=None):
    """nn.Linear: y = x W^T (+ b), W stored [out_features, in_features]."""
    y = np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T
    if b is not None:
        y = y + np.asarray(b, dtype=F64)
    return y


def head_hidden(x, w1_k, b1_k):
    """Residual SiLU feed-forward layer of one head: U = x + SiLU(x W1^T + b1)."""
    x = np.asarray(x, dtype=F64)
    return x + silu(linear(x, w1_k, b1_k))


def head_logits(x, w1, b1, w2):
    """Logits of every Medusa head for every row of ``x``.

    Head k reads the same final hidden state as lm_head, applies one residual
    SiLU feed-forward layer, then a vocabulary projection without bias:
    ``logits_k = (x + SiLU(x W1_k^T + b1_k)) W2_k^T``.  Returns [K, M, V].
    """
    return np.stack([linear(head_hidden(x, w1[k], b1[k]), w2[k]) for k in range(len(w1))])


# ----------------------------------------------------------------------------
# top-k and argmax (decisions in float32)
# ----------------------------------------------------------------------------
def f32(x):
    return np.asarray(x, dtype=np.float32)


def topk(values, k):
    """Top-k of a float32 vector: value descending, equal values -> lower index.

    "Le ipotesi migliori delle teste" ("Medusa Heads", tree attention section):
    the heads' best guesses.  Implemented as a full stable sort.
    Returns (ids int32[k], vals float32[k]).
    """
    v = f32(values)
    order = np.argsort(-v, kind="stable")[:k]
    return order.astype(np.int32), v[order]


def argmax(values):
    """Index of the largest float32 value, lowest index on ties."""
    v = f32(values)
    return int(np.flatnonzero(v == v.max())[0])


# ----------------------------------------------------------------------------
# candidate tree ("Medusa Heads", tree attention and acceptance section)
# ----------------------------------------------------------------------------
def cartesian_candidates(topk_lists):
    """All continuations formed by the Cartesian product of per-head top-k lists."""
    return list(itertools.product(*[list(t) for t in topk_lists]))


def build_tree(parent, rank, root_tok, topk_ids, ctx):
    """Fill a tree template with tokens; derive depths, positions and masks.

    Node 0 holds ``root_tok``.  A node at depth d >= 1 with rank r holds
    ``topk_ids[d-1][r]`` (head d proposes the token at t+d+1; every branch of
    head d-1 gets the same proposals of head d).  A node sees itself and its
    ancestors: ``mask[i]`` has bit j set iff tree node j is i or an ancestor.
    Position of a node = ctx + depth.
    Returns dict(tokens int32[N], depth int32[N], pos int32[N], mask uint64[N]).
    """
    n = len(parent)
    tokens = np.zeros(n, np.int32)
    depth = np.zeros(n, np.int32)
    mask = np.zeros(n, np.uint64)
    for i in range(n):
        if i == 0:
            tokens[0], depth[0], mask[0] = root_tok, 0, np.uint64(1)
            continue
        p = int(parent[i])
        depth[i] = depth[p] + 1
        tokens[i] = int(topk_ids[depth[i] - 1][int(rank[i])])
        mask[i] = mask[p] | (np.uint64(1) << np.uint64(i))
    return dict(tokens=tokens, depth=depth, pos=(ctx + depth).astype(np.int32), mask=mask)


def sparse_tree(accuracy, n_nodes):
    """Sparse tree of the most accurate head combinations ("Medusa Heads",
    section "Attenzione sull'albero e accettazione": a sparse 64-node tree
    built from the most accurate combinations beat a dense 256-node one).

    ``accuracy[k][r]`` (in [0, 1]) is the chance that head k+1's rank-r
    candidate is the right token.  Reading: a combination is a rank tuple
    (r1..rd), d <= K, and its accuracy is the product of its heads'
    accuracies (the chance that the whole branch is accepted, heads taken as
    independent); the tree keeps the root and the n_nodes - 1 most accurate
    combinations, ties to the shallower and then the lexicographically
    smaller tuple.  (With accuracies <= 1 a combination is never more
    accurate than its prefix, so the kept set is prefix-closed.)  The sum of
    the kept accuracies is the expected number of accepted candidates.
    Returns (parent int32[n], rank int32[n]) in canonical order (by depth,
    then lexicographic by rank tuple) and the expected acceptance length.
    Enumerates every combination: small K and top-k only."""
    acc = np.asarray(accuracy, dtype=F64)
    K, width = acc.shape
    combos = []
    for d in range(1, K + 1):
        for t in itertools.product(range(width), repeat=d):
            v = 1.0
            for j, r in enumerate(t):
                v = v * float(acc[j, r])
            combos.append((-v, d, t))
    combos.sort()
    kept = [()] + [t for _, _, t in combos[:n_nodes - 1]]
    kept.sort(key=lambda t: (len(t), t))
    index = {t: i for i, t in enumerate(kept)}
    parent = np.array([-1] + [index[t[:-1]] for t in kept[1:]], dtype=np.int32)
    rank = np.array([0] + [t[-1] for t in kept[1:]], dtype=np.int32)
    expected = float(sum(-v for v, _, _ in combos[:n_nodes - 1]))
    return parent, rank, expected


def visible(mask_i, n):
    """Tree node indices whose bit is set in ``mask_i``."""
    m = int(mask_i)
    return [j for j in range(n) if (m >> j) & 1]


# ----------------------------------------------------------------------------
# tree-masked attention ("Medusa Heads", tree attention section; arXiv
# abstract: tree-based attention verifies all candidates in one step)
# ----------------------------------------------------------------------------
def tree_attention(q, k_cache, v_cache, k_tree, v_tree, mask, scale):
    """Softmax attention of every tree node over the cache plus its ancestors.

    q [N, Hq, D]; k_cache/v_cache [ctx, Hkv, D] (logical order); k_tree/v_tree
    [N, Hkv, D]; mask uint64[N].  Node i attends to all ``ctx`` cached keys and
    to tree node j iff bit j of mask[i] is set; masked keys take no part.
    Query head h reads key/value head h // (Hq / Hkv).  Returns [N, Hq, D].
    """
    q = np.asarray(q, F64)
    kc, vc = np.asarray(k_cache, F64), np.asarray(v_cache, F64)
    kt, vt = np.asarray(k_tree, F64), np.asarray(v_tree, F64)
    n, hq, d = q.shape
    group = hq // kt.shape[1]
    out = np.zeros((n, hq, d), F64)
    for i in range(n):
        vis = visible(mask[i], n)
        for h in range(hq):
            g = h // group
            keys = np.concatenate([kc[:, g, :], kt[vis, g, :]], axis=0)
            vals = np.concatenate([vc[:, g, :], vt[vis, g, :]], axis=0)
            s = (keys @ q[i, h]) * float(scale)
            p = np.exp(s - s.max())
            out[i, h] = (p / p.sum()) @ vals
    return out


def cache_rows(pool, page_table_row, n, page_size):
    """Logical rows 0..n-1 of a paged cache pool [pages, Hkv, P, D] -> [n, Hkv, D]."""
    pool = np.asarray(pool)
    slots = np.arange(n)
    pages = np.asarray(page_table_row)[slots // page_size]
    return pool[pages, :, slots % page_size, :]


# ----------------------------------------------------------------------------
# acceptance ("Medusa Heads", tree attention and acceptance section)
# ----------------------------------------------------------------------------
def _accept_sweep(tokens, parent, ok, n_heads):
    """Longest accepted branch given a per-node criterion ``ok(i)``.

    acc[0] = True (the root is the model's own choice); acc[i] = acc[parent] and
    ok(i).  The kept branch ends at the deepest accepted node, lowest index on
    ties.  Returns (accept_len, path int32[n_heads+1] padded with -1, best).
    """
    n = len(parent)
    depth = np.zeros(n, np.int32)
    acc = np.zeros(n, bool)
    acc[0] = True
    for i in range(1, n):
        p = int(parent[i])
        depth[i] = depth[p] + 1
        acc[i] = acc[p] and ok(i)
    best = 0
    for i in range(1, n):
        if acc[i] and depth[i] > depth[best]:
            best = i
    a = int(depth[best])
    path = -np.ones(n_heads + 1, np.int32)
    j = best
    for d in range(a, -1, -1):
        path[d] = j
        j = int(parent[j])
    return a, path, best


def accept_greedy(logits, tokens, parent, n_heads):
    """Greedy acceptance: a candidate is kept when it equals the model's top choice.

    ``logits`` [N, V] are the verification logits of the tree nodes: row p
    scores the token after node p.  Returns dict(accept_len, path, next_token,
    best); next_token = argmax of the kept branch's last row.
    """
    top = [argmax(row) for row in logits]
    a, path, best = _accept_sweep(tokens, parent,
                                  lambda i: int(tokens[i]) == top[int(parent[i])], n_heads)
    return dict(accept_len=a, path=path, next_token=top[best], best=best)


def typical_stats(logits_row, temperature):
    """(log-probabilities, entropy) of softmax(logits / T), in float64."""
    z = f32(logits_row).astype(F64) / float(temperature)
    z = z - z.max()
    logp = z - np.log(np.exp(z).sum())
    p = np.exp(logp)
    ent = -float(np.sum(np.where(p > 0, p * logp, 0.0)))
    return logp, ent


def accept_typical(logits, tokens, parent, n_heads, temperature, epsilon, delta,
                   return_margins=False):
    """Typical acceptance: keep a candidate whose base-model probability is above
    an entropy-linked threshold.

    Reading (the formula itself is not on the pages): with p = softmax(z / T)
    of the parent's row and H its natural-log entropy, accept iff
    ``p(token) > min(epsilon, delta * exp(-H))``.  The next root token is the
    argmax of the kept branch's last row.  With ``return_margins`` also
    returns, per node, ln p(token) - ln(threshold).
    """
    n = len(parent)
    stats = {}
    margins = np.full(n, np.inf)

    def ok(i):
        p = int(parent[i])
        if p not in stats:
            stats[p] = typical_stats(logits[p], temperature)
        logp, ent = stats[p]
        thr = min(float(epsilon), float(delta) * np.exp(-ent))
        lp = logp[int(tokens[i])]
        margins[i] = lp - (np.log(thr) if thr > 0 else -np.inf)
        return bool(np.exp(lp) > thr)

    a, path, best = _accept_sweep(tokens, parent, ok, n_heads)
    out = dict(accept_len=a, path=path, next_token=argmax(logits[best]), best=best)
    if return_margins:
        out["margins"] = margins
    return out


# ----------------------------------------------------------------------------
# sampled verification: rejection sampling against the base model's own
# distribution keeps Medusa-1 lossless ("Têtes de décodage Medusa", section
# "Plongée profonde", and its "Questions fréquemment posées" entry on lossless
# acceleration: exact rejection sampling checks the accepted candidates
# against the base model's distribution)
# ----------------------------------------------------------------------------
_M64 = (1 << 64) - 1
_PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)   # round multipliers
_PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)   # key schedule (Weyl) increments


def _mulhilo64(a, b):
    """High and low 64-bit halves of the 128-bit product of uint64 arrays,
    from 32-bit limbs (numpy has no 128-bit integers)."""
    a = np.asarray(a, np.uint64)
    b = np.asarray(b, np.uint64)
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a0, a1 = a & m32, a >> s32
    b0, b1 = b & m32, b >> s32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> s32) + (p01 & m32) + (p10 & m32)          # < 3 * 2^32: no overflow
    hi = p11 + (p01 >> s32) + (p10 >> s32) + (mid >> s32)
    lo = a * b                                                # wraps modulo 2^64
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011): counter = 4 uint64 words
    (each an array, broadcast together), key = 2 uint64 words.  Each round
    multiplies words 0 and 2 by the two round constants, swaps halves and
    XORs in the round key; the key advances by the Weyl constants.  Returns
    the 4 output words."""
    with np.errstate(over="ignore"):
        c = [np.asarray(w, np.uint64) for w in counter]
        k = [np.uint64(int(w) & _M64) for w in key]
        for _ in range(10):
            hi0, lo0 = _mulhilo64(np.uint64(_PHILOX_M[0]), c[0])
            hi1, lo1 = _mulhilo64(np.uint64(_PHILOX_M[1]), c[2])
            c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
            k = [k[0] + np.uint64(_PHILOX_W[0]), k[1] + np.uint64(_PHILOX_W[1])]
    return c


def sample_uniforms(V, seed, step, b, node):
    """Uniforms in (0, 1) for vocabulary entries 0..V-1 of tree node ``node`` of
    sequence ``b`` at decode step ``step``: key (seed, step), counter
    (v // 4, node, b, 0), output word v % 4; u = (top 23 bits + 1/2) / 2^23,
    exact in float32."""
    v = np.arange(V, dtype=np.uint64)
    words = philox4x64_10([v >> np.uint64(2), np.uint64(node), np.uint64(b), np.uint64(0)],
                          [seed, step])
    w = np.choose((v & np.uint64(3)).astype(np.int64), words)
    return ((w >> np.uint64(41)).astype(F64) + 0.5) / float(1 << 23)


def sample_scores(logits_row, temperature, seed, step, b, node):
    """Gumbel-max scores z/T + G with G = -log(-log(u)): the index of their
    maximum is a draw from softmax(z/T).  The decision is taken in float32,
    the precision of the logits: G is computed in float64 and rounded, and
    the score is float32(float32(z * float32(1/T)) + G)."""
    u = sample_uniforms(len(logits_row), seed, step, b, node)
    g = f32(-np.log(-np.log(u)))
    inv_t = np.float32(1.0) / np.float32(temperature)
    return (f32(logits_row) * inv_t) + g


def sample_token(logits_row, temperature, seed, step, b, node):
    """One draw from softmax(z/T) (lowest index on a tie of scores)."""
    sc = sample_scores(logits_row, temperature, seed, step, b, node)
    return int(np.flatnonzero(sc == sc.max())[0])


def accept_sample(logits, tokens, parent, n_heads, temperature, seed, step, b=0,
                  return_margins=False):
    """Sampled verification of the tree (rejection sampling against the base model).

    Reading: the heads' candidates are fixed (top-k), so the rejection test of
    a candidate x under the base distribution p accepts it with probability
    p(x); probing the children of an accepted node in rank order, each with p
    renormalised over the tokens not yet rejected, and drawing from the rest
    when all are rejected, yields the same joint law as one draw z ~ p at
    that node: the child whose token is z is accepted, and when no child
    carries z, z itself is the next token and the branch ends.  That is how it
    is computed here: z_u = one draw from softmax(logits[u] / T) per node
    (Gumbel-max, counter-based noise keyed by (seed, step)); node i is
    accepted iff its parent is and tokens[i] == z_parent; the next root token
    is z at the deepest accepted node.  Every emitted token is thus a draw
    from the base model given its prefix.  ``return_margins`` adds, per node,
    the gap between its two best scores (near-ties decide in rounding).
    """
    n = len(parent)
    z = []
    gaps = np.full(n, np.inf)
    for u in range(n):
        sc = sample_scores(logits[u], temperature, seed, step, b, u)
        top2 = np.partition(sc, -2)[-2:] if len(sc) > 1 else np.array([-np.inf, sc[0]])
        gaps[u] = float(top2[1] - top2[0])
        z.append(int(np.flatnonzero(sc == sc.max())[0]))
    a, path, best = _accept_sweep(tokens, parent,
                                  lambda i: int(tokens[i]) == z[int(parent[i])], n_heads)
    out = dict(accept_len=a, path=path, next_token=z[best], best=best, samples=z)
    if return_margins:
        out["margins"] = gaps
    return out


# ----------------------------------------------------------------------------
# KV compaction (only the kept branch stays in the cache: "Medusa Heads",
# tree attention section, the longest accepted branch is kept)
# ----------------------------------------------------------------------------
def kv_compact(cache, ctx, path, accept_len):
    """Move the kept branch's rows to slots ctx..ctx+a (logical [S, ...] cache).

    Row ctx+d receives old row ctx+path[d] for d = 0..a (all reads happen
    before any write).  Returns (new_cache, src_slots, dst_slots, new_ctx);
    src/dst are padded with -1 to len(path).
    """
    new = np.array(cache, copy=True)
    a = int(accept_len)
    src = -np.ones(len(path), np.int32)
    dst = -np.ones(len(path), np.int32)
    rows = [np.array(cache[ctx + int(path[d])], copy=True) for d in range(a + 1)]
    for d in range(a + 1):
        new[ctx + d] = rows[d]
        src[d], dst[d] = ctx + int(path[d]), ctx + d
    return new, src, dst, ctx + a + 1


# ----------------------------------------------------------------------------
# Llama-style backbone (the model being verified; the pages fix only that the
# tree is checked in one forward pass of the base model)
# ----------------------------------------------------------------------------
def rmsnorm(x, g, eps):
    x = np.asarray(x, F64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, F64)


def rope(x, pos, base):
    """Rotary embedding, rotate-half convention, over the full head dim.

    x [n, heads, D]; angle(p, j) = p * base^(-2j/D) for j < D/2; the pair
    (x_j, x_{j+D/2}) is rotated by that angle.
    """
    x = np.asarray(x, F64)
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=F64) * 2.0 / d)
    ang = np.asarray(pos, F64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


class KVCache:
    """Per-layer logical K/V caches [capacity, Hkv, D] in float64."""

    def __init__(self, model, capacity):
        shape = (capacity, model.n_kv_heads, model.head_dim)
        self.k = [np.zeros(shape, F64) for _ in range(model.n_layers)]
        self.v = [np.zeros(shape, F64) for _ in range(model.n_layers)]

    def copy(self):
        c = KVCache.__new__(KVCache)
        c.k = [a.copy() for a in self.k]
        c.v = [a.copy() for a in self.v]
        return c


def forward_rows(model, tokens, pos, mask, cache, ctx, layer_hook=None):
    """One forward pass of ``n`` new rows that see the cache and, among
    themselves, what ``mask`` allows (a chain mask = ordinary causal decoding).

    Writes the rows' K/V into cache slots ctx..ctx+n-1.  Returns
    (logits [n, V] float64, final hidden state after the last RMSNorm [n, H]).
    """
    n = len(tokens)
    x = np.asarray(model.embed, F64)[np.asarray(tokens)]
    nh, nkv, hd = model.n_heads, model.n_kv_heads, model.head_dim
    scale = 1.0 / np.sqrt(hd)
    for li, L in enumerate(model.layers):
        h = rmsnorm(x, L["g_attn"], model.eps)
        q = rope(linear(h, L["wq"]).reshape(n, nh, hd), pos, model.rope_base)
        k = rope(linear(h, L["wk"]).reshape(n, nkv, hd), pos, model.rope_base)
        v = linear(h, L["wv"]).reshape(n, nkv, hd)
        o = tree_attention(q, cache.k[li][:ctx], cache.v[li][:ctx], k, v, mask, scale)
        cache.k[li][ctx:ctx + n] = k
        cache.v[li][ctx:ctx + n] = v
        x = x + linear(o.reshape(n, nh * hd), L["wo"])
        h = rmsnorm(x, L["g_mlp"], model.eps)
        x = x + linear(silu(linear(h, L["wg"])) * linear(h, L["wu"]), L["wd"])
        if layer_hook is not None:
            layer_hook(li, x)
    hf = rmsnorm(x, model.g_final, model.eps)
    return linear(hf, model.lm_head), hf


def chain_mask(n):
    """Mask of a single path of n nodes: node i sees nodes 0..i."""
    return np.array([(1 << (i + 1)) - 1 for i in range(n)], dtype=np.uint64)


def prefill(model, prompt, cache):
    """Causal forward over the prompt (positions 0..P-1)."""
    p = len(prompt)
    return forward_rows(model, prompt, np.arange(p), chain_mask(p), cache, 0)


def sequential_greedy(model, prompt, n_new, capacity=None):
    """Plain greedy decoding: one token per forward pass, x_{t+1} = argmax."""
    capacity = capacity or len(prompt) + n_new + 1
    cache = KVCache(model, capacity)
    logits, _ = prefill(model, prompt, cache)
    out = [argmax(logits[-1])]
    ctx = len(prompt)
    while len(out) < n_new:
        logits, _ = forward_rows(model, [out[-1]], [ctx], np.array([1], np.uint64), cache, ctx)
        ctx += 1
        out.append(argmax(logits[-1]))
    return np.array(out, np.int32), cache, ctx


def medusa_generate(model, prompt, n_new, parent, rank, mode="greedy", temperature=1.0,
                    epsilon=0.3, delta=0.09, heads=None, capacity=None, record=None, seed=0,
                    b=0):
    """Medusa decoding loop, steps in the order the pages give them.

    1. Prefill; root = argmax of the last row; heads on the last hidden state
       give per-head top-k (k = max rank + 1 of the template).
    2. Build the tree from the template; verify all nodes in one forward pass
       with the ancestor mask.
    3. Accept the longest branch (greedy, typical or sampled); emit its a+1
       tokens.
    4. Keep only that branch in the cache; feed its last hidden state to the
       heads for the next round; next root = argmax of its last row (a draw
       from it in sampled mode).
    Sampled mode draws the prefill root at step 0 (node 0) and verifies decode
    step s = 1, 2, ... with key (seed, s); ``b`` is the sequence's index in a
    batch, the third word of every draw's counter (a batch of sequences
    decoded together draws sequence b's noise from its own counters).
    ``heads`` (optional) replaces the learned heads by a function
    hidden_row -> [K, V] logits (used by pins).  ``record`` collects per-step
    dicts.  Returns (tokens int32[n_new], cache, ctx).
    """
    parent = np.asarray(parent)
    rank = np.asarray(rank)
    depth_of = np.zeros(len(parent), np.int32)
    for i in range(1, len(parent)):
        depth_of[i] = depth_of[parent[i]] + 1
    n_heads = int(depth_of.max())
    width = int(rank.max()) + 1
    n = len(parent)
    capacity = capacity or len(prompt) + n_new + n + 1
    cache = KVCache(model, capacity)
    logits, hf = prefill(model, prompt, cache)
    ctx = len(prompt)

    def head_topk(hrow):
        lg = heads(hrow) if heads is not None else head_logits(hrow[None], model.w1, model.b1, model.w2)[:, 0]
        return [topk(lg[k], width)[0] for k in range(n_heads)]

    if mode == "sample":
        root = sample_token(logits[-1], temperature, seed, 0, b, 0)
    else:
        root = argmax(logits[-1])
    ids = head_topk(hf[-1])
    out = []
    step = 0
    while len(out) < n_new:
        step += 1
        tree = build_tree(parent, rank, root, ids, ctx)
        logits, hf = forward_rows(model, tree["tokens"], tree["pos"], tree["mask"], cache, ctx)
        lf = f32(logits)
        if mode == "greedy":
            res = accept_greedy(lf, tree["tokens"], parent, n_heads)
        elif mode == "sample":
            res = accept_sample(lf, tree["tokens"], parent, n_heads, temperature, seed, step, b=b)
        else:
            res = accept_typical(lf, tree["tokens"], parent, n_heads, temperature, epsilon, delta,
                                 return_margins=True)
        a, path = res["accept_len"], res["path"]
        out.extend(int(tree["tokens"][path[d]]) for d in range(a + 1))
        for li in range(model.n_layers):
            cache.k[li], _, _, _ = kv_compact(cache.k[li], ctx, path, a)
            cache.v[li], src, dst, new_ctx = kv_compact(cache.v[li], ctx, path, a)
        if record is not None:
            record.append(dict(ctx=ctx, tree=tree, accept=res, src=src, dst=dst))
        ctx = new_ctx
        root = res["next_token"]
        ids = head_topk(hf[res["best"]])
    return np.array(out[:n_new], np.int32), cache, ctx
