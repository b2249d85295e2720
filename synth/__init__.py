"""Seeded synthetic inputs for the Medusa decode step.

This module is shared by both sides of every parity check (the CPU oracle in
``oracle/`` and the HIP library in ``speculative_decoding_02_amd/``) and holds
none of the method's arithmetic: it only draws seeded random numbers, rounds
draws to bfloat16, and enumerates / prunes tree *shapes*, which are inputs to
both sides.

Recipes (the workloads the pages describe, made synthetic):

* ``tiny_decoder`` - a 2-layer Llama-style decoder, hidden 256, 4 heads of
  dim 64, vocab 1000, with 3 Medusa heads whose vocab projection is a copy of
  lm_head and whose feed-forward weight is perturbed by N(0, 0.01) (the heads'
  initialisation described in "Medusa Heads", section on how the heads predict
  the following tokens).
* ``tree_template`` - the Cartesian product of per-head top-k ranks, in
  canonical order (root first, then breadth first, rank tuples in
  lexicographic order inside one depth).
* ``prune_template`` - seeded removal of random leaves until a node budget is
  met (the pages speak of a sparse 64-node tree).
* attention / head inputs ~ N(0, 1) or N(0, std) as stated per function.

Every generator takes an explicit seed and returns numpy arrays; bf16 tensors
are returned as their raw uint16 bit patterns plus an exact float32 view.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_bits", "bf16_to_f32", "round_bf16", "rngs",
    "tree_template", "prune_template", "chain_template", "template_depth",
    "TinyDecoder", "tiny_decoder", "attention_inputs", "heads_inputs",
    "random_template_batch",
]


# ----------------------------------------------------------------------------
# bfloat16 rounding of drawn values (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of ``x`` (float32) rounded to bfloat16, RNE."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x) -> np.ndarray:
    """float32 array holding ``x`` rounded to bfloat16 values."""
    return bf16_to_f32(bf16_bits(x))


def rngs(seed: int, n: int):
    """``n`` independent generators spawned from ``SeedSequence(seed)``, in order."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


# ----------------------------------------------------------------------------
# tree shapes (inputs to both the oracle and the library)
# ----------------------------------------------------------------------------
def tree_template(widths):
    """Cartesian-product tree of rank tuples for per-depth top-k ``widths``.

    Node 0 is the root (the token the model itself picked).  A node at depth
    d >= 1 is a rank tuple (r1..rd) with r_j < widths[j-1]; its parent is
    (r1..r_{d-1}).  Order: by depth, then lexicographic by rank tuple.
    Returns ``(parent int32[N], rank int32[N])``; the root has parent -1,
    rank 0.
    """
    tuples = [()]
    for d in range(1, len(widths) + 1):
        tuples += list(itertools.product(*[range(w) for w in widths[:d]]))
    index = {t: i for i, t in enumerate(tuples)}
    parent = np.array([-1] + [index[t[:-1]] for t in tuples[1:]], dtype=np.int32)
    rank = np.array([0] + [t[-1] for t in tuples[1:]], dtype=np.int32)
    return parent, rank


def chain_template(n):
    """A single path of ``n`` nodes: node i's parent is i-1, every rank 0."""
    parent = np.arange(-1, n - 1, dtype=np.int32)
    rank = np.zeros(n, dtype=np.int32)
    return parent, rank


def template_depth(parent) -> np.ndarray:
    """Depth of every node (root 0), walking parent links (parents precede children)."""
    depth = np.zeros(len(parent), dtype=np.int32)
    for i in range(1, len(parent)):
        depth[i] = depth[parent[i]] + 1
    return depth


def prune_template(parent, rank, n_keep, seed):
    """Remove uniformly drawn current leaves (never the root) until ``n_keep`` remain.

    Leaves are listed in canonical (index) order before each draw and one is
    removed with ``default_rng(seed).integers``.  Survivors keep their relative
    order; parent indices are remapped.
    """
    parent = np.asarray(parent, dtype=np.int64)
    rank = np.asarray(rank, dtype=np.int32)
    n = len(parent)
    if n_keep >= n:
        return parent.astype(np.int32).copy(), rank.copy()
    rng = np.random.default_rng(seed)
    alive = np.ones(n, dtype=bool)
    n_children = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        n_children[parent[i]] += 1
    while alive.sum() > n_keep:
        leaves = [i for i in range(1, n) if alive[i] and n_children[i] == 0]
        victim = leaves[int(rng.integers(len(leaves)))]
        alive[victim] = False
        n_children[parent[victim]] -= 1
    keep = np.flatnonzero(alive)
    new_index = -np.ones(n, dtype=np.int64)
    new_index[keep] = np.arange(len(keep))
    new_parent = np.array([-1] + [new_index[parent[i]] for i in keep[1:]], dtype=np.int32)
    return new_parent, rank[keep].copy()


def random_template_batch(widths, n_keep, seeds):
    """One pruned template per seed, stacked to ``[B, n_keep]`` arrays."""
    full_p, full_r = tree_template(widths)
    ps, rs = zip(*[prune_template(full_p, full_r, n_keep, s) for s in seeds])
    return np.stack(ps), np.stack(rs)


# ----------------------------------------------------------------------------
# the tiny random decoder with Medusa heads (fp32)
# ----------------------------------------------------------------------------
@dataclass
class TinyDecoder:
    vocab: int
    hidden: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    rope_base: float
    eps: float
    embed: np.ndarray            # [V, H]
    layers: list                 # dicts: wq wk wv wo [out,in], wg wu [F,H], wd [H,F], g_attn g_mlp [H]
    g_final: np.ndarray          # [H]
    lm_head: np.ndarray          # [V, H]
    w1: np.ndarray               # [K, H, H] (row = output feature)
    b1: np.ndarray               # [K, H]
    w2: np.ndarray               # [K, V, H]
    meta: dict = field(default_factory=dict)

    @property
    def n_medusa(self):
        return self.w1.shape[0]


def tiny_decoder(seed=1, vocab=1000, hidden=256, n_layers=2, n_heads=4, head_dim=64,
                 ffn=688, n_medusa=3, std=0.02, head_std=0.01, n_kv_heads=None,
                 bf16=False) -> TinyDecoder:
    """Random-init Llama-style decoder plus Medusa heads.

    Draw order (one spawned generator each): embedding, then per layer
    wq wk wv wo wg wu wd, then lm_head, then the K head W1 matrices.
    All linear / embedding weights ~ N(0, std); norm gains 1; W1 ~ N(0, head_std);
    b1 = 0; W2_k = copy of lm_head.  With ``bf16`` every drawn weight is
    rounded to bfloat16 values (still returned as float32).
    """
    n_kv_heads = n_heads if n_kv_heads is None else n_kv_heads
    n_draw = 1 + 7 * n_layers + 1 + 1
    g = rngs(seed, n_draw)
    it = iter(g)
    rnd = (lambda a: round_bf16(a)) if bf16 else (lambda a: a)

    def draw(shape, s):
        return rnd(next(it).standard_normal(shape, dtype=np.float32) * np.float32(s))

    embed = draw((vocab, hidden), std)
    layers = []
    qd, kd = n_heads * head_dim, n_kv_heads * head_dim
    for _ in range(n_layers):
        layers.append(dict(
            wq=draw((qd, hidden), std), wk=draw((kd, hidden), std), wv=draw((kd, hidden), std),
            wo=draw((hidden, qd), std), wg=draw((ffn, hidden), std), wu=draw((ffn, hidden), std),
            wd=draw((hidden, ffn), std),
            g_attn=np.ones(hidden, np.float32), g_mlp=np.ones(hidden, np.float32)))
    lm_head = draw((vocab, hidden), std)
    w1 = draw((n_medusa, hidden, hidden), head_std)
    b1 = np.zeros((n_medusa, hidden), np.float32)
    w2 = np.broadcast_to(lm_head, (n_medusa, vocab, hidden)).copy()
    return TinyDecoder(vocab, hidden, n_layers, n_heads, n_kv_heads, head_dim, ffn, 10000.0,
                       1e-5, embed, layers, np.ones(hidden, np.float32), lm_head, w1, b1, w2,
                       meta=dict(seed=seed, std=std, head_std=head_std, bf16=bf16))


def prompt_tokens(seed, n, vocab):
    """``n`` uniform random token ids in [0, vocab)."""
    return np.random.default_rng(seed).integers(0, vocab, size=n).astype(np.int32)


# ----------------------------------------------------------------------------
# single-kernel inputs
# ----------------------------------------------------------------------------
def attention_inputs(seed, B, N, Hq, Hkv, D, ctx, page_size=16, extra_pages=0,
                     permute_pages=False, bf16=True, widths=(4, 3, 2, 2, 1)):
    """Inputs for one tree-masked attention call over a paged KV cache.

    ``ctx`` is an int or a per-sequence list.  Q, tree K/V and cached K/V are
    N(0, 1) (bf16-rounded when ``bf16``).  Each sequence gets its own tree,
    ``widths`` Cartesian product pruned to N nodes (seed = seed*1000 + b).
    The page pool holds ceil((ctx_b + N)/P) pages per sequence (+extra), in a
    seeded permutation when ``permute_pages``; slots past ctx_b are filled
    with a sentinel-free N(0,1) draw so stale data is visible if misused.
    Returns a dict of numpy arrays.
    """
    ctxs = np.array([ctx] * B if np.isscalar(ctx) else list(ctx), dtype=np.int32)
    gq, gk, gv, gkc, gvc, gperm = rngs(seed, 6)
    rnd = round_bf16 if bf16 else (lambda a: a)
    Q = rnd(gq.standard_normal((B, N, Hq, D), dtype=np.float32))
    Kt = rnd(gk.standard_normal((B, N, Hkv, D), dtype=np.float32))
    Vt = rnd(gv.standard_normal((B, N, Hkv, D), dtype=np.float32))
    pages_per = [(int(c) + N + page_size - 1) // page_size + extra_pages for c in ctxs]
    max_pages = max(pages_per)
    n_pages = int(sum(pages_per))
    order = gperm.permutation(n_pages) if permute_pages else np.arange(n_pages)
    page_table = -np.ones((B, max_pages), dtype=np.int32)
    o = 0
    for b in range(B):
        page_table[b, :pages_per[b]] = order[o:o + pages_per[b]]
        o += pages_per[b]
    Kc = rnd(gkc.standard_normal((n_pages, Hkv, page_size, D), dtype=np.float32))
    Vc = rnd(gvc.standard_normal((n_pages, Hkv, page_size, D), dtype=np.float32))
    parents, ranks = [], []
    for b in range(B):
        p, r = tree_template(widths)
        p, r = prune_template(p, r, N, seed * 1000 + b)
        if len(p) < N:
            raise ValueError("tree smaller than N")
        parents.append(p)
        ranks.append(r)
    return dict(Q=Q, Kt=Kt, Vt=Vt, Kc=Kc, Vc=Vc, page_table=page_table, ctx=ctxs,
                parent=np.stack(parents), rank=np.stack(ranks), page_size=page_size,
                scale=np.float32(1.0 / np.sqrt(D)))


def heads_inputs(seed, M, H, V, K, w1_std=0.01, w2_std=0.02, x_std=1.0, bf16=True):
    """X [M,H] ~ N(0,x_std); W1 [K,H,H], b1 [K,H] ~ N(0,w1_std); W2 [K,V,H] ~ N(0,w2_std)."""
    gx, g1, gb, g2 = rngs(seed, 4)
    rnd = round_bf16 if bf16 else (lambda a: a)
    X = rnd(gx.standard_normal((M, H), dtype=np.float32) * np.float32(x_std))
    W1 = rnd(g1.standard_normal((K, H, H), dtype=np.float32) * np.float32(w1_std))
    b1 = rnd(gb.standard_normal((K, H), dtype=np.float32) * np.float32(w1_std))
    W2 = rnd(g2.standard_normal((K, V, H), dtype=np.float32) * np.float32(w2_std))
    return dict(X=X, W1=W1, b1=b1, W2=W2)


# ----------------------------------------------------------------------------
# large random decoders, drawn on the GPU (seeded torch generator)
# ----------------------------------------------------------------------------
def device_llama(seed, n_layers=32, hidden=4096, n_heads=32, n_kv_heads=None, head_dim=128,
                 ffn=11008, vocab=32000, n_medusa=5, std=0.02, head_std=0.01, dtype=None,
                 device="cuda"):
    """Random-init Llama-style decoder + Medusa heads as device tensors.

    Same recipe as ``tiny_decoder`` (weights ~ N(0, std), gains 1, W1 ~
    N(0, head_std), b1 = 0, W2_k = lm_head) but drawn by a seeded torch
    generator on ``device`` in float32 and cast to ``dtype`` (default bf16).
    Draw order: embedding, per layer wq wk wv wo wg wu wd, lm_head, W1.
    Returns a dict with ``meta``, ``embed``, ``layers`` (list of dicts with
    the Llama layout), ``g_final``, ``lm_head``, ``w1``, ``b1``, ``w2``.
    """
    import torch

    dtype = dtype or torch.bfloat16
    n_kv_heads = n_heads if n_kv_heads is None else n_kv_heads
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))

    def draw(shape, s):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return t.mul_(s).to(dtype)

    ones = lambda n: torch.ones(n, device=device, dtype=dtype)
    qd, kd = n_heads * head_dim, n_kv_heads * head_dim
    out = dict(meta=dict(vocab=vocab, hidden=hidden, n_layers=n_layers, n_heads=n_heads,
                         n_kv_heads=n_kv_heads, head_dim=head_dim, ffn=ffn, rope_base=10000.0,
                         eps=1e-5, seed=seed))
    out["embed"] = draw((vocab, hidden), std)
    out["layers"] = []
    for _ in range(n_layers):
        out["layers"].append(dict(
            wq=draw((qd, hidden), std), wk=draw((kd, hidden), std), wv=draw((kd, hidden), std),
            wo=draw((hidden, qd), std), wg=draw((ffn, hidden), std), wu=draw((ffn, hidden), std),
            wd=draw((hidden, ffn), std), g_attn=ones(hidden), g_mlp=ones(hidden)))
    out["lm_head"] = draw((vocab, hidden), std)
    out["g_final"] = ones(hidden)
    out["w1"] = draw((n_medusa, hidden, hidden), head_std)
    out["b1"] = torch.zeros((n_medusa, hidden), device=device, dtype=dtype)
    out["w2"] = out["lm_head"].unsqueeze(0).repeat(n_medusa, 1, 1).contiguous()
    return out
