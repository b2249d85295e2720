"""GPU end to end on the tiny fp32 decoder: Medusa greedy decoding through
libmedusa emits exactly the tokens of the oracle's sequential greedy decoding
(the lossless claim of greedy acceptance), and so does plain one-token greedy
decoding through the same library.  Sampled verification emits the oracle's
sampled Medusa decoding token for token (same counter-based stream)."""
import numpy as np
import pytest
import torch

import synth
from oracle import medusa_oracle as orc
from gpu_util import case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c1():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m = synth.tiny_decoder(seed=1)
    prompt = synth.prompt_tokens(101, 32, m.vocab)
    seq, _, _ = orc.sequential_greedy(m, prompt, 64)
    return m, prompt, seq


def _report(seq, got):
    diff = [i for i in range(len(seq)) if seq[i] != got[i]]
    return f"first mismatch at {diff[:1]}: oracle {seq.tolist()[:diff[0]+3] if diff else ''} gpu {got.tolist()[:diff[0]+3] if diff else ''}"


def test_c1_medusa_greedy_equals_oracle_sequential_greedy(c1):
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, seq = c1
    case("c1 medusa greedy (2,3) tree")
    dm = DeviceModel(m, dtype=torch.float32)
    parent, rank = synth.tree_template((2, 3))
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 64 + 16)
    rec = []
    got = dec.generate(prompt, 64, record=rec)
    assert got.tolist() == seq.tolist(), _report(seq, got)
    assert sum(a + 1 for a in rec) >= 64 and len(rec) <= 64


def test_c1_plain_greedy_equals_oracle(c1):
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, seq = c1
    case("c1 plain greedy (single-node tree)")
    dm = DeviceModel(m, dtype=torch.float32)
    dec = MedusaDecoder(dm, np.array([-1]), np.array([0]), capacity=32 + 64 + 16)
    got = dec.generate(prompt, 64)
    assert got.tolist() == seq.tolist(), _report(seq, got)


def test_c1_medusa_greedy_deeper_tree_and_typical_runs(c1):
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, seq = c1
    case("c1 medusa greedy (3,2,2) + typical")
    dm = DeviceModel(m, dtype=torch.float32)
    parent, rank = synth.tree_template((3, 2, 2))
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 64 + 32)
    got = dec.generate(prompt, 40)
    assert got.tolist() == seq[:40].tolist(), _report(seq[:40], got)
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 64 + 32, mode="typical")
    rec = []
    got = dec.generate(prompt, 40, record=rec)
    assert len(got) == 40 and all(0 <= a <= 3 for a in rec)


def test_c1_graph_replays_match_eager_and_oracle(c1):
    """The decode step recorded once as a HIP graph and replayed step after
    step (with eager host reads and other GPU work in between) emits the same
    tokens as eager stepping and as the oracle."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, seq = c1
    case("c1 graph replay")
    dm = DeviceModel(m, dtype=torch.float32)
    parent, rank = synth.tree_template((2, 3))
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 64 + 16)
    got = dec.generate(prompt, 64, graph=True)
    assert got.tolist() == seq.tolist(), _report(seq, got)
    # replay the same graph for a second generation (state reset by prefill)
    scratch = torch.randn(1000, device="cuda").sum()  # unrelated eager work
    got2 = dec.generate(prompt, 64, graph=True)
    assert got2.tolist() == seq.tolist()
    assert torch.isfinite(scratch)


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_c1_medusa_sampled_equals_oracle_sampled(c1, T):
    """Sampled verification (rejection sampling against the base model, draws
    from the shared Philox stream keyed by the seed) emits the oracle's tokens;
    the graph-replayed step emits the same."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, _ = c1
    case(f"c1 medusa sampled T={T}")
    parent, rank = synth.tree_template((2, 3))
    ref, _, _ = orc.medusa_generate(m, prompt, 48, parent, rank, mode="sample", temperature=T,
                                    seed=5)
    dm = DeviceModel(m, dtype=torch.float32)
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 48 + 16, mode="sample", temperature=T,
                        seed=5)
    got = dec.generate(prompt, 48)
    assert got.tolist() == ref.tolist(), _report(ref, got)
    assert got2_equal(dec, prompt, ref)


def got2_equal(dec, prompt, ref):
    got = dec.generate(prompt, len(ref), graph=True)
    assert got.tolist() == ref.tolist(), _report(ref, got)
    return True


@pytest.mark.parametrize("mode", ["greedy", "sample"])
def test_c1_separate_tail_equals_oracle(c1, mode):
    """The decode step with its tail as separate launches (accept, kv_compact,
    gather_rows, host read per step) emits the same tokens as the oracle, as
    the fused tail does; the fused tail's accept lengths (from its device log)
    equal the separate path's."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, prompt, seq = c1
    case(f"c1 separate tail {mode}")
    parent, rank = synth.tree_template((2, 3))
    kw = dict(mode="sample", temperature=0.8, seed=9) if mode == "sample" else {}
    ref = seq[:48] if mode == "greedy" else orc.medusa_generate(m, prompt, 48, parent, rank,
                                                                 mode="sample", temperature=0.8,
                                                                 seed=9)[0]
    dm = DeviceModel(m, dtype=torch.float32)
    recs = {}
    for tail in ("separate", "fused"):
        dec = MedusaDecoder(dm, parent, rank, capacity=32 + 48 + 16, tail=tail, **kw)
        rec = []
        got = dec.generate(prompt, 48, record=rec, graph=True)
        assert got.tolist() == ref.tolist(), _report(ref, got)
        recs[tail] = rec
    assert recs["fused"] == recs["separate"]


def _prompts(B, n, V, seed0=300):
    return np.stack([synth.prompt_tokens(seed0 + b, n, V) for b in range(B)])


@pytest.mark.parametrize("tail", ["fused", "separate"])
def test_c1_batched_greedy_equals_oracle_per_sequence(c1, tail):
    """Three sequences decoded together (their trees' rows through every
    projection at once, each with its own pages and context) emit exactly
    each prompt's sequential greedy tokens, eagerly and from a replayed graph."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, _, _ = c1
    case(f"c1 batched greedy B=3 tail={tail}")
    B, n_new = 3, 40
    prompts = _prompts(B, 32, m.vocab)
    refs = [orc.sequential_greedy(m, prompts[b], n_new)[0] for b in range(B)]
    dm = DeviceModel(m, dtype=torch.float32)
    parent, rank = synth.tree_template((2, 3))
    dec = MedusaDecoder(dm, parent, rank, capacity=32 + 3 * n_new + 16, batch=B, tail=tail)
    for graph in (False, True):
        rec = []
        got = dec.generate(prompts, n_new, record=rec, graph=graph)
        assert got.shape == (B, n_new)
        for b in range(B):
            assert got[b].tolist() == refs[b].tolist(), f"sequence {b}: " + _report(refs[b], got[b])
        assert len(rec) == B and all(len(r) == len(rec[0]) for r in rec)


def test_c1_batched_sampled_equals_oracle_per_sequence(c1):
    """Sampled verification of a batch: sequence b emits the oracle's sampled
    decoding of its prompt with counter word b."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m, _, _ = c1
    case("c1 batched sampled B=2")
    B, n_new, T, seed = 2, 32, 0.8, 11
    prompts = _prompts(B, 24, m.vocab, seed0=500)
    parent, rank = synth.tree_template((2, 3))
    refs = [orc.medusa_generate(m, prompts[b], n_new, parent, rank, mode="sample", temperature=T,
                                seed=seed, b=b)[0] for b in range(B)]
    dm = DeviceModel(m, dtype=torch.float32)
    dec = MedusaDecoder(dm, parent, rank, capacity=24 + 3 * n_new + 16, batch=B, mode="sample",
                        temperature=T, seed=seed)
    got = dec.generate(prompts, n_new, graph=True)
    for b in range(B):
        assert got[b].tolist() == refs[b].tolist(), f"sequence {b}: " + _report(refs[b], got[b])
