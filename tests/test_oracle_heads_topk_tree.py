"""Pins of the oracle's heads, top-k and tree construction against what the
pages fix and against independent library semantics (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import medusa_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- heads ----
def test_zero_init_heads_reproduce_lm_head_exactly():
    """The page's snippet: zero-initialised residual layer + W2 copied from
    lm_head => every head's logits equal lm_head(h) exactly ([True, True, True])."""
    H, V, K = 256, 1000, 3
    g = synth.rngs(7, 2)
    lm = g[0].standard_normal((V, H)).astype(np.float32) * 0.05
    h = g[1].standard_normal((1, H)).astype(np.float32)
    w1 = np.zeros((K, H, H), np.float32)
    b1 = np.zeros((K, H), np.float32)
    w2 = np.broadcast_to(lm, (K, V, H)).copy()
    got = orc.head_logits(h, w1, b1, w2)
    ref = orc.linear(h, lm)
    assert [np.array_equal(got[k], ref) for k in range(K)] == [True, True, True]


def test_heads_match_torch_nn_linear_semantics():
    """head_k(h) = out(h + F.silu(layer(h))) with torch.nn.Linear modules (fp64)."""
    H, V, K, M = 48, 80, 3, 5
    d = synth.heads_inputs(3, M, H, V, K, w1_std=0.2, w2_std=0.1, bf16=False)
    got = orc.head_logits(d["X"], d["W1"], d["b1"], d["W2"])
    h = torch.tensor(d["X"], dtype=torch.float64)
    for k in range(K):
        layer = torch.nn.Linear(H, H).double()
        out = torch.nn.Linear(H, V, bias=False).double()
        with torch.no_grad():
            layer.weight.copy_(torch.tensor(d["W1"][k]))
            layer.bias.copy_(torch.tensor(d["b1"][k]))
            out.weight.copy_(torch.tensor(d["W2"][k]))
            ref = out(h + torch.nn.functional.silu(layer(h))).numpy()
        np.testing.assert_allclose(got[k], ref, rtol=1e-12, atol=1e-12)


def test_heads_closed_form_identity_projection():
    """W1 = 0, b1 = c, W2 = I (H = V): logits = x + SiLU(c), SiLU from its closed form."""
    gold = _gold("silu_closed_form.json")
    c = np.array(gold["z"], np.float64)
    H = len(c)
    x = np.arange(2 * H, dtype=np.float64).reshape(2, H) / 7.0
    got = orc.head_logits(x, np.zeros((1, H, H)), c[None], np.eye(H)[None])[0]
    np.testing.assert_allclose(got, x + np.array(gold["silu"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.silu(c), gold["silu"], rtol=0, atol=1e-15)
    assert np.signbit(orc.silu(np.array([-0.0])))[0]


# ---------------------------------------------------------------- top-k ----
def _topk_brute(v, k):
    v = list(np.asarray(v, np.float32))
    taken, ids = set(), []
    for _ in range(k):
        best = None
        for i, x in enumerate(v):
            if i in taken:
                continue
            if best is None or x > v[best]:
                best = i
        taken.add(best)
        ids.append(best)
    return ids


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    v = rng.integers(-5, 5, size=300).astype(np.float32)  # many exact ties
    v[rng.integers(0, 300, 10)] = 7.0
    for k in (1, 3, 10, 64):
        ids, vals = orc.topk(v, k)
        assert list(ids) == _topk_brute(v, k)
        assert np.array_equal(vals, v[ids])


def test_topk_signed_zero_is_a_tie():
    v = np.array([0.0, -0.0, 0.0, -1.0], np.float32)
    v[0] = -0.0
    ids, _ = orc.topk(v, 3)
    assert list(ids) == [0, 1, 2]
    assert orc.argmax(v) == 0


# ----------------------------------------------------------------- tree ----
def test_c1_template_matches_hand_derivation():
    gold = _gold("c1_tree.json")
    parent, rank = synth.tree_template(gold["widths"])
    assert parent.tolist() == gold["parent"]
    assert rank.tolist() == gold["rank"]
    t = orc.build_tree(parent, rank, 5, [[11, 12], [21, 22, 23]], ctx=100)
    assert t["depth"].tolist() == gold["depth"]
    assert [int(m) for m in t["mask"]] == gold["mask"]
    assert t["pos"].tolist() == [100 + d for d in gold["depth"]]
    leaves = [i for i in range(len(parent)) if i not in set(parent.tolist())]
    assert leaves == gold["leaves"]


def test_top2_x_top3_gives_six_prefix_sharing_candidates():
    """Root-to-leaf token paths of the built tree = Cartesian product of the
    top-2 of head 1 and the top-3 of head 2; head 2's tokens repeat under
    every head-1 branch."""
    gold = _gold("c1_tree.json")
    parent, rank = synth.tree_template(gold["widths"])
    ids = [[101, 102], [201, 202, 203]]
    t = orc.build_tree(parent, rank, 7, ids, ctx=0)
    leaves = [i for i in range(len(parent)) if i not in set(parent.tolist())]
    paths = []
    for leaf in leaves:
        p, j = [], leaf
        while j > 0:
            p.append(int(t["tokens"][j]))
            j = int(parent[j])
        paths.append(tuple(reversed(p)))
    assert len(paths) == gold["n_candidates"] == 6
    assert sorted(paths) == sorted(orc.cartesian_candidates(ids))
    assert sorted(paths) == sorted(itertools.product(*ids))
    assert t["tokens"][3:6].tolist() == t["tokens"][6:9].tolist()


def test_full_and_pruned_templates():
    parent, rank = synth.tree_template((4, 3, 2, 2, 1))
    assert len(parent) == _gold("c1_tree.json")["full_tree_nodes_4_3_2_2_1"] == 1 + 4 + 12 + 24 + 48 + 48
    for seed in range(5):
        p, r = synth.prune_template(parent, rank, 64, seed)
        assert len(p) == 64 and p[0] == -1
        assert all(0 <= p[i] < i for i in range(1, 64))
        t = orc.build_tree(p, r, 1, np.arange(5 * 4).reshape(5, 4), ctx=0)
        for i in range(64):
            m = int(t["mask"][i])
            assert m & 1 and (m >> i) & 1
            assert bin(m).count("1") == t["depth"][i] + 1
        # siblings keep distinct ranks
        for i in range(64):
            kids = [int(r[j]) for j in range(64) if p[j] == i]
            assert len(kids) == len(set(kids))


def test_chain_masks():
    p, r = synth.chain_template(10)
    t = orc.build_tree(p, r, 0, np.zeros((9, 1), np.int32), ctx=3)
    assert [int(m) for m in t["mask"]] == [(1 << (i + 1)) - 1 for i in range(10)]
    assert np.array_equal(orc.chain_mask(10), t["mask"])
