"""Pins of the oracle's sampled verification (CPU only).

"Têtes de décodage Medusa" (section "Plongée profonde", and the entry of its
"Questions fréquemment posées" on lossless acceleration) states that
rejection sampling against the base model keeps Medusa-1's output
distribution that of the base model.  The pins:

* the counter-based generator (Philox4x64-10) equals numpy's Philox bit
  generator word for word;
* Gumbel-max draws follow softmax(z / T) (chi-square on a fixed stream);
* the tokens a sampled tree step emits follow the base model's distributions
  (first token after the root, and the next one given it): the lossless claim;
* a tiny temperature reproduces greedy acceptance.
The streams are fixed (seeded), so every check is deterministic.
"""
import numpy as np
import pytest
from scipy import stats

import synth
from oracle import medusa_oracle as orc


def _np_philox_block(counter, key):
    """numpy's Philox: the state's counter is advanced before each block of four."""
    bg = np.random.Philox(counter=np.array(counter, np.uint64), key=np.array(key, np.uint64))
    return [int(x) for x in bg.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((5, 0, 0, 0), (7, 9)),
    ((123456789, 42, 7, 3), (0xDEADBEEFCAFEF00D, 0x0123456789ABCDEF)),
    ((2**64 - 2, 17, 0, 2**63), (2**64 - 1, 2**64 - 1)),
])
def test_philox_matches_numpy(counter, key):
    nxt = list(counter)
    nxt[0] = (nxt[0] + 1) % 2**64  # (no carry in these cases)
    mine = orc.philox4x64_10([np.uint64(w) for w in nxt], key)
    assert [int(w) for w in mine] == _np_philox_block(counter, key)


def test_philox_vectorised_counters():
    """Array counters give each element the block of its own counter."""
    key = (31, 4)
    words = orc.philox4x64_10([np.arange(1, 9, dtype=np.uint64), np.uint64(3), np.uint64(1),
                               np.uint64(0)], key)
    for i in range(8):
        assert [int(w[i]) for w in words] == _np_philox_block((i, 3, 1, 0), key)


def test_uniforms_open_interval_float32_exact():
    u = orc.sample_uniforms(4099, seed=11, step=5, b=2, node=7)
    assert u.min() > 0.0 and u.max() < 1.0
    np.testing.assert_array_equal(u, u.astype(np.float32).astype(np.float64))
    # word v % 4 of block v // 4
    words = orc.philox4x64_10([np.uint64(1), np.uint64(7), np.uint64(2), np.uint64(0)], (11, 5))
    assert u[6] == ((int(words[2]) >> 41) + 0.5) / 2**23


def _chi2_p(counts, probs):
    counts = np.asarray(counts, np.float64)
    probs = np.asarray(probs, np.float64)
    exp = probs / probs.sum() * counts.sum()
    return stats.chisquare(counts, exp).pvalue


def test_gumbel_max_follows_softmax():
    z = np.array([0.3, -1.2, 2.0, 0.0, 1.1], np.float32)
    T = 0.7
    p = np.exp(z / T - (z / T).max())
    p /= p.sum()
    n = 12000
    counts = np.zeros(len(z))
    for step in range(n):
        counts[orc.sample_token(z, T, seed=3, step=step, b=0, node=0)] += 1
    assert _chi2_p(counts, p) > 1e-4
    # and not the uniform distribution (the test can fail)
    assert _chi2_p(counts, np.full(len(z), 1 / len(z))) < 1e-6


def _toy_tree():
    # root 0; children 1, 2, 3 (tokens 0, 2, 4); node 1 has children 4, 5 (tokens 1, 3)
    parent = np.array([-1, 0, 0, 0, 1, 1], np.int32)
    tokens = np.array([5, 0, 2, 4, 1, 3], np.int32)
    rng = np.random.default_rng(8)
    logits = (rng.standard_normal((6, 6)) * 1.3).astype(np.float32)
    return parent, tokens, logits


def test_sampled_tree_step_is_lossless():
    """First emitted token after the root ~ p_root; given that it is child 1's
    token, the next emitted token ~ p_node1 (whether node 1's child is taken
    or the branch ends with a draw at node 1)."""
    parent, tokens, logits = _toy_tree()
    T = 1.0

    def soft(row):
        e = np.exp(row / T - (row / T).max())
        return e / e.sum()

    n = 6000
    first = np.zeros(6)
    second = np.zeros(6)
    for step in range(n):
        r = orc.accept_sample(logits, tokens, parent, 2, T, seed=21, step=step)
        a, path = r["accept_len"], r["path"]
        emitted = [int(tokens[path[d]]) for d in range(1, a + 1)] + [r["next_token"]]
        first[emitted[0]] += 1
        if emitted[0] == tokens[1]:
            second[emitted[1]] += 1
    assert _chi2_p(first, soft(logits[0])) > 1e-4
    assert second.sum() > 300
    assert _chi2_p(second, soft(logits[1])) > 1e-4
    # a rule that ignores the draws (greedy) would not pass
    assert _chi2_p(first, np.eye(6)[orc.argmax(logits[0])] * 0.999 + 0.001 / 6) < 1e-6


def test_sampled_acceptance_walks_the_draws():
    """Node i is accepted iff its parent is and its token is the parent's draw;
    the next token is the draw at the deepest accepted node."""
    parent, tokens, logits = _toy_tree()
    for step in range(50):
        r = orc.accept_sample(logits, tokens, parent, 2, 0.8, seed=2, step=step)
        z = r["samples"]
        u, walk = 0, [0]
        while True:
            kids = [i for i in range(len(parent)) if parent[i] == u and tokens[i] == z[u]]
            if not kids:
                break
            u = kids[0]
            walk.append(u)
        assert r["accept_len"] == len(walk) - 1
        assert list(r["path"][:len(walk)]) == walk
        assert r["next_token"] == z[u]


@pytest.mark.parametrize("seed", range(3))
def test_tiny_temperature_is_greedy(seed):
    rng = np.random.default_rng(seed)
    N, V = 40, 300
    p, _ = synth.prune_template(*synth.tree_template((4, 3, 2, 2, 1)), N, seed)
    logits = (rng.standard_normal((N, V)) * 2).astype(np.float32)
    tokens = rng.integers(0, V, N).astype(np.int32)
    for i in range(1, N):
        if rng.random() < 0.6:
            tokens[i] = orc.argmax(logits[p[i]])
    g = orc.accept_greedy(logits, tokens, p, 5)
    s = orc.accept_sample(logits, tokens, p, 5, 1e-4, seed=seed, step=1)
    assert s["accept_len"] == g["accept_len"]
    np.testing.assert_array_equal(s["path"], g["path"])
    assert s["next_token"] == g["next_token"]


def test_generate_sequence_index_selects_its_counters():
    """A batch's sequence b draws with counter word b: on the same prompt,
    sequence 0 reproduces the default run and sequence 1 draws other noise
    (its prefill draw equals a direct draw with b = 1)."""
    m = synth.tiny_decoder(seed=1)
    prompt = synth.prompt_tokens(7, 12, m.vocab)
    parent, rank = synth.tree_template((2, 2))
    a0, _, _ = orc.medusa_generate(m, prompt, 12, parent, rank, mode="sample", temperature=1.0,
                                   seed=4)
    b0, _, _ = orc.medusa_generate(m, prompt, 12, parent, rank, mode="sample", temperature=1.0,
                                   seed=4, b=0)
    b1, _, _ = orc.medusa_generate(m, prompt, 12, parent, rank, mode="sample", temperature=1.0,
                                   seed=4, b=1)
    assert a0.tolist() == b0.tolist()
    assert a0.tolist() != b1.tolist()
    cache = orc.KVCache(m, 64)
    logits, _ = orc.prefill(m, prompt, cache)
    assert b1[0] == orc.sample_token(logits[-1], 1.0, 4, 0, 1, 0)
