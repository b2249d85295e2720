"""Pins of the oracle's decoder, acceptance rules, decode loop and KV
compaction (CPU only).

* The backbone equals Hugging Face ``LlamaForCausalLM`` in float64 on the
  same weights, and sequential greedy equals its greedy ``generate``.
* Medusa greedy decoding emits exactly the tokens of sequential greedy
  decoding (the lossless claim of "Têtes de décodage Medusa", section
  "Plongée profonde", and of "Medusa Heads": greedy acceptance keeps a
  candidate only when it is the model's top choice).
* Typical acceptance: special cases only (its threshold formula is unpinned).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import medusa_oracle as orc


@pytest.fixture(scope="module")
def tiny():
    return synth.tiny_decoder(seed=1)


def _hf_model(m):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=m.vocab, hidden_size=m.hidden, intermediate_size=m.ffn,
                      num_hidden_layers=m.n_layers, num_attention_heads=m.n_heads,
                      num_key_value_heads=m.n_kv_heads, rms_norm_eps=m.eps,
                      max_position_embeddings=1024, tie_word_embeddings=False,
                      attention_bias=False, mlp_bias=False, rope_theta=m.rope_base)
    hf = LlamaForCausalLM(cfg).double().eval()
    sd = {"model.embed_tokens.weight": m.embed, "model.norm.weight": m.g_final,
          "lm_head.weight": m.lm_head}
    names = dict(wq="self_attn.q_proj", wk="self_attn.k_proj", wv="self_attn.v_proj",
                 wo="self_attn.o_proj", wg="mlp.gate_proj", wu="mlp.up_proj", wd="mlp.down_proj",
                 g_attn="input_layernorm", g_mlp="post_attention_layernorm")
    for i, L in enumerate(m.layers):
        for k, n in names.items():
            sd[f"model.layers.{i}.{n}.weight"] = L[k]
    hf.load_state_dict({k: torch.tensor(np.asarray(v), dtype=torch.float64) for k, v in sd.items()})
    return hf


def test_backbone_matches_hf_llama(tiny):
    prompt = synth.prompt_tokens(2, 32, tiny.vocab)
    cache = orc.KVCache(tiny, 64)
    logits, _ = orc.prefill(tiny, prompt, cache)
    hf = _hf_model(tiny)
    with torch.no_grad():
        ref = hf(torch.tensor(prompt[None], dtype=torch.long)).logits[0].numpy()
    # Hugging Face evaluates the rotary angles in float32 even in a float64 model
    # (observed max difference 1.6e-7); a wrong rotary convention, norm or
    # projection orientation differs at O(0.1).
    np.testing.assert_allclose(logits, ref, rtol=0, atol=1e-6)


def test_sequential_greedy_matches_hf_generate(tiny):
    prompt = synth.prompt_tokens(3, 32, tiny.vocab)
    toks, _, _ = orc.sequential_greedy(tiny, prompt, 12)
    hf = _hf_model(tiny)
    with torch.no_grad():
        out = hf.generate(torch.tensor(prompt[None], dtype=torch.long), max_new_tokens=12,
                          do_sample=False, num_beams=1, pad_token_id=0)
    assert toks.tolist() == out[0, 32:].tolist()


@pytest.mark.parametrize("widths,seed", [((2, 3), 1), ((3, 2, 2), 5)])
def test_medusa_greedy_equals_sequential_greedy(widths, seed):
    m = synth.tiny_decoder(seed=seed)
    prompt = synth.prompt_tokens(seed + 100, 32, m.vocab)
    parent, rank = synth.tree_template(widths)
    n_new = 64 if seed == 1 else 24
    seq, seq_cache, _ = orc.sequential_greedy(m, prompt, n_new)
    rec = []
    med, med_cache, ctx = orc.medusa_generate(m, prompt, n_new, parent, rank, record=rec)
    assert med.tolist() == seq.tolist()
    # the compacted cache equals the sequentially built cache where both are defined
    upto = len(prompt) + n_new - 1
    for li in range(m.n_layers):
        np.testing.assert_allclose(med_cache.k[li][:upto], seq_cache.k[li][:upto], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(med_cache.v[li][:upto], seq_cache.v[li][:upto], rtol=1e-9, atol=1e-12)


def test_cheating_heads_accept_full_depth_and_never_matching_accept_nothing(tiny):
    prompt = synth.prompt_tokens(4, 16, tiny.vocab)
    n_new = 30
    seq, _, _ = orc.sequential_greedy(tiny, prompt, n_new + 8)
    parent, rank = synth.tree_template((2, 2, 2))
    # heads that know the true continuation: rank 0 of head k = token k steps ahead.
    # The heads get the kept branch's hidden state; recover the position from the
    # number of tokens emitted so far via the record.
    state = {"emitted": 0}

    def cheat(_h):
        e = state["emitted"]
        lg = np.zeros((3, tiny.vocab))
        for k in range(3):
            idx = e + 1 + k
            if idx < len(seq):
                lg[k, seq[idx]] = 10.0
        return lg

    class Rec(list):
        def append(self, x):
            super().append(x)
            state["emitted"] += x["accept"]["accept_len"] + 1

    rec = Rec()
    out, _, _ = orc.medusa_generate(tiny, prompt, n_new, parent, rank, heads=cheat, record=rec)
    assert out.tolist() == seq[:n_new].tolist()
    assert all(r["accept"]["accept_len"] == 3 for r in rec[:-1])

    # heads whose proposals never contain the model's choice -> 1 token per step
    rec2 = []
    seq_set = set(seq.tolist())
    bad = [t for t in range(tiny.vocab) if t not in seq_set][:2]

    def never2(_h):
        lg = np.full((3, tiny.vocab), -1.0)
        lg[:, bad] = 5.0
        return lg

    out2, _, _ = orc.medusa_generate(tiny, prompt, n_new, parent, rank, heads=never2, record=rec2)
    assert out2.tolist() == seq[:n_new].tolist()
    assert all(r["accept"]["accept_len"] == 0 for r in rec2)
    assert len(rec2) == n_new


def _random_tree_logits(seed, n=64, V=50, sharp=1.0):
    parent, rank = synth.tree_template((4, 3, 2, 2, 1))
    parent, rank = synth.prune_template(parent, rank, n, seed)
    rng = np.random.default_rng(seed)
    logits = (rng.standard_normal((n, V)) * sharp).astype(np.float32)
    tokens = rng.integers(0, V, n).astype(np.int32)
    return parent, tokens, logits


def test_typical_threshold_zero_accepts_deepest_lowest_index():
    parent, tokens, logits = _random_tree_logits(0)
    depth = synth.template_depth(parent)
    for eps, delta in ((0.3, 0.0), (0.0, 0.09)):
        r = orc.accept_typical(logits, tokens, parent, 5, 1.0, eps, delta)
        assert r["accept_len"] == depth.max()
        assert r["best"] == int(np.flatnonzero(depth == depth.max())[0])
        assert r["path"][0] == 0 and r["path"][-1] == r["best"]


def test_typical_near_one_hot_is_greedy():
    for seed in range(5):
        parent, tokens, logits = _random_tree_logits(seed, V=20, sharp=1.0)
        # make the children's tokens often the argmax of their parent
        for i in range(1, len(parent)):
            if i % 3:
                tokens[i] = orc.argmax(logits[parent[i]])
        g = orc.accept_greedy(logits, tokens, parent, 5)
        t = orc.accept_typical(logits, tokens, parent, 5, 1e-3, 0.3, 0.09)
        assert (t["accept_len"], t["path"].tolist(), t["next_token"]) == \
            (g["accept_len"], g["path"].tolist(), g["next_token"])


def test_typical_monotone_in_epsilon_and_delta():
    for seed in range(5):
        parent, tokens, logits = _random_tree_logits(seed, V=8, sharp=0.5)
        prev = None
        for eps in (0.01, 0.05, 0.1, 0.2, 0.5):
            a = orc.accept_typical(logits, tokens, parent, 5, 1.0, eps, 1.0)["accept_len"]
            assert prev is None or a <= prev
            prev = a
        prev = None
        for delta in (0.01, 0.05, 0.2, 0.5, 1.0):
            a = orc.accept_typical(logits, tokens, parent, 5, 1.0, 1.0, delta)["accept_len"]
            assert prev is None or a <= prev
            prev = a


def _one_child(row, tok):
    """Root + one child carrying ``tok``; the root's logits row decides."""
    logits = np.stack([np.asarray(row, np.float32), np.zeros(len(row), np.float32)])
    return logits, np.array([0, tok], np.int32), np.array([-1, 0], np.int32)


@pytest.mark.parametrize("V", [2, 7, 1000])
def test_typical_uniform_row_entropy_is_log_v(V):
    """Uniform logits: p(x) = 1/V and H = ln V, so the threshold is
    min(eps, delta / V): delta < 1 accepts, delta > 1 rejects (an entropy in
    another base, or with a sign error, fails one of the two)."""
    logits, tok, par = _one_child(np.full(V, 0.37), 1)
    assert orc.accept_typical(logits, tok, par, 1, 1.0, 1.0, 0.5)["accept_len"] == 1
    assert orc.accept_typical(logits, tok, par, 1, 1.0, 1.0, 2.0)["accept_len"] == 0
    r = orc.accept_typical(logits, tok, par, 1, 1.0, 1.0, 0.5, return_margins=True)
    # margin = ln p - ln thr = ln(1/V) - ln(0.5/V) = ln 2
    assert r["margins"][1] == pytest.approx(np.log(2.0), abs=1e-6)


def test_typical_two_point_distribution_closed_form():
    """p = (1/4, 3/4) (logits 0 and ln 3, the rest -60): H = ln 4 - (3/4) ln 3.
    Token 0 (p = 1/4) is accepted iff delta e^-H < 1/4; the decision flips
    where the closed form says, and the temperature divides the logits
    (T = 2 on doubled logits gives the same law)."""
    V = 6
    row = np.full(V, -60.0)
    row[0], row[1] = 0.0, np.log(3.0)
    H = np.log(4.0) - 0.75 * np.log(3.0)
    d_star = 0.25 * np.exp(H)
    for T, r_ in ((1.0, row), (2.0, 2 * row)):
        logits, tok, par = _one_child(r_, 0)
        assert orc.accept_typical(logits, tok, par, 1, T, 1.0, d_star * (1 - 1e-4))["accept_len"] == 1
        assert orc.accept_typical(logits, tok, par, 1, T, 1.0, d_star * (1 + 1e-4))["accept_len"] == 0
        # the hard threshold epsilon binds when it is the smaller one
        assert orc.accept_typical(logits, tok, par, 1, T, 0.2499, 10.0)["accept_len"] == 1
        assert orc.accept_typical(logits, tok, par, 1, T, 0.2501, 10.0)["accept_len"] == 0


def test_greedy_accept_hand_example():
    """Top-2 x top-3 tree; the model's choices make the branch (1, 0) win."""
    parent, rank = synth.tree_template((2, 3))
    t = orc.build_tree(parent, rank, 9, [[3, 4], [5, 6, 7]], 0)
    V = 10
    logits = np.zeros((9, V), np.float32)
    logits[0, 4] = 1   # root -> 4 (node 2)
    logits[1, 6] = 1
    logits[2, 5] = 1   # node 2 -> 5 (node 6)
    logits[6, 8] = 1   # next token after node 6
    r = orc.accept_greedy(logits, t["tokens"], parent, 2)
    assert r["accept_len"] == 2
    assert r["path"].tolist() == [0, 2, 6]
    assert r["next_token"] == 8


def test_kv_compact_hand_example():
    ctx = 10
    cache = np.arange(30 * 3, dtype=np.float64).reshape(30, 3)
    new, src, dst, nctx = orc.kv_compact(cache, ctx, np.array([0, 2, 7, -1]), 2)
    assert src.tolist() == [10, 12, 17, -1]
    assert dst.tolist() == [10, 11, 12, -1]
    assert nctx == 13
    np.testing.assert_array_equal(new[10], cache[10])
    np.testing.assert_array_equal(new[11], cache[12])
    np.testing.assert_array_equal(new[12], cache[17])
    np.testing.assert_array_equal(new[:10], cache[:10])
    np.testing.assert_array_equal(new[13:], cache[13:])
    # overlapping move: path (0, 1, 3) moves slot 13 into 12 after 12 was read
    new, _, _, _ = orc.kv_compact(cache, ctx, np.array([0, 2, 3]), 2)
    np.testing.assert_array_equal(new[11], cache[12])
    np.testing.assert_array_equal(new[12], cache[13])
