"""Pins of the oracle's tree-masked attention (CPU only): chain tree = causal
attention, root-only = decode attention, closed forms, and an ancestor walk
against torch's scaled_dot_product_attention with an explicit boolean mask."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import medusa_oracle as orc


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, attn_mask=None, is_causal=False, scale=None):
    """torch SDPA in float64 on [n, H, D] tensors (heads as batch)."""
    t = lambda a: torch.tensor(np.ascontiguousarray(np.transpose(a, (1, 0, 2))), dtype=torch.float64)
    m = None if attn_mask is None else torch.tensor(attn_mask)
    o = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, is_causal=is_causal, scale=scale)
    return np.transpose(o.numpy(), (1, 0, 2))


@pytest.mark.parametrize("n", [1, 5, 17])
def test_chain_tree_is_causal_attention(n):
    H, D = 3, 16
    q, k, v = _rand(1, n, H, D), _rand(2, n, H, D), _rand(3, n, H, D)
    got = orc.tree_attention(q, np.zeros((0, H, D)), np.zeros((0, H, D)), k, v,
                             orc.chain_mask(n), 1 / np.sqrt(D))
    ref = _sdpa(q, k, v, is_causal=True, scale=1 / np.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_chain_tree_after_cache_is_causal_attention():
    ctx, n, H, D = 11, 6, 2, 8
    kc, vc = _rand(4, ctx, H, D), _rand(5, ctx, H, D)
    q, k, v = _rand(6, n, H, D), _rand(7, n, H, D), _rand(8, n, H, D)
    got = orc.tree_attention(q, kc, vc, k, v, orc.chain_mask(n), 0.3)
    allowed = np.zeros((n, ctx + n), bool)
    for i in range(n):
        allowed[i, :ctx + i + 1] = True
    ref = _sdpa(q, np.concatenate([kc, k]), np.concatenate([vc, v]), attn_mask=allowed, scale=0.3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_root_only_tree_is_decode_attention():
    ctx, H, D = 40, 4, 32
    kc, vc = _rand(9, ctx, H, D), _rand(10, ctx, H, D)
    q, k, v = _rand(11, 1, H, D), _rand(12, 1, H, D), _rand(13, 1, H, D)
    got = orc.tree_attention(q, kc, vc, k, v, np.array([1], np.uint64), 1 / np.sqrt(D))
    ref = _sdpa(q, np.concatenate([kc, k]), np.concatenate([vc, v]), scale=1 / np.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values_and_constant_values():
    ctx, H, D = 5, 2, 4
    parent, rank = synth.tree_template((2, 3))
    t = orc.build_tree(parent, rank, 0, [[0, 1], [0, 1, 2]], 0)
    n = len(parent)
    kc, vc = _rand(14, ctx, H, D), _rand(15, ctx, H, D)
    k, v = _rand(16, n, H, D), _rand(17, n, H, D)
    got = orc.tree_attention(np.zeros((n, H, D)), kc, vc, k, v, t["mask"], 1.0)
    for i in range(n):
        anc = [i]
        while anc[-1] != 0:
            anc.append(int(parent[anc[-1]]))
        ref = np.concatenate([vc, v[sorted(anc)]]).mean(axis=0)
        np.testing.assert_allclose(got[i], ref, rtol=1e-12, atol=1e-12)
    const = np.full((n, H, D), 2.5)
    got = orc.tree_attention(_rand(18, n, H, D), kc, np.full((ctx, H, D), 2.5), k, const,
                             t["mask"], 0.7)
    np.testing.assert_allclose(got, const, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_pruned_tree_against_ancestor_walk_sdpa(seed):
    """Visible set built by walking parent links (not from the bitmask)."""
    n, ctx, Hq, Hkv, D = 64, 9, 4, 2, 8
    parent, rank = synth.tree_template((4, 3, 2, 2, 1))
    parent, rank = synth.prune_template(parent, rank, n, seed)
    t = orc.build_tree(parent, rank, 0, np.zeros((5, 4), np.int32), ctx)
    q = _rand(20 + seed, n, Hq, D)
    kc, vc = _rand(30 + seed, ctx, Hkv, D), _rand(40 + seed, ctx, Hkv, D)
    k, v = _rand(50 + seed, n, Hkv, D), _rand(60 + seed, n, Hkv, D)
    got = orc.tree_attention(q, kc, vc, k, v, t["mask"], 0.35)
    allowed = np.zeros((n, ctx + n), bool)
    allowed[:, :ctx] = True
    for i in range(n):
        j = i
        while j >= 0:
            allowed[i, ctx + j] = True
            j = int(parent[j])
    keys = np.repeat(np.concatenate([kc, k]), Hq // Hkv, axis=1)
    vals = np.repeat(np.concatenate([vc, v]), Hq // Hkv, axis=1)
    ref = _sdpa(q, keys, vals, attn_mask=allowed, scale=0.35)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_paged_cache_rows():
    d = synth.attention_inputs(3, B=2, N=4, Hq=2, Hkv=2, D=8, ctx=[20, 37], page_size=16,
                               permute_pages=True, bf16=False, widths=(2, 2))
    for b in range(2):
        rows = orc.cache_rows(d["Kc"], d["page_table"][b], int(d["ctx"][b]), 16)
        for s in range(int(d["ctx"][b])):
            page = d["page_table"][b][s // 16]
            np.testing.assert_array_equal(rows[s], d["Kc"][page, :, s % 16, :])
