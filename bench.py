#!/usr/bin/env python3
"""Benchmark of the Medusa decode step on one MI355X.

Workload (synthetic, seeded, random-init): a Llama-7B-shaped decoder in bf16
(32 layers, hidden 4096, 32 heads x 128, FFN 11008, vocab 32000) with 5 Medusa
heads (W1 ~ N(0, 0.01), b1 = 0, W2 = lm_head), a 512-token random prompt and
a 64-node verification tree (Cartesian product of top-(4,3,2,2,1), pruned to
64 nodes by seeded leaf removal).  One step = one pass of the whole hot path:
tree build, the 64-row verification forward with tree-masked attention over
the paged KV cache, acceptance, KV compaction, and the heads + top-k on the
kept branch's hidden state.  ``value`` = accepted (emitted) tokens per second
over the K timed steps, inputs resident in HBM.

Also reported on the same line:
  roofline       the dominant kernel of the step (the gate/up projection, a
                 weight-streaming GEMM, HBM-bound) from HIP events on its
                 launching stream over the timed steps;
  tree_attention the tree-attention kernel alone at the 7B layer shape
                 (32 heads x 128, 2048 cached tokens + 64 tree nodes), KV
                 buffers rotated over > 256 MB so the MALL cannot serve them;
  cpu_baseline   the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "accepted tokens/s + tree-attn HBM GB/s (% peak), 7B-shape, 64-node tree"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense bf16
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_7b_counters.md")


def measured_traffic(label, source):
    """Calibrated HBM bytes per launch of ``label`` from the committed counter
    summary, or None when absent or taken on a different version of
    ``source`` (the kernel changed since the counters were read)."""
    import hashlib
    try:
        line = [l for l in open(TRAFFIC_FILE) if l.startswith("traffic_json: ")][0]
        d = json.loads(line[len("traffic_json: "):])
        cur = hashlib.sha256(open(os.path.join(ROOT, "speculative_decoding_02_amd", "csrc", source),
                                  "rb").read()).hexdigest()[:16]
        if d["sources"].get(source) != cur:
            return None
        return d[label]["traffic_bytes"]
    except (OSError, IndexError, KeyError, ValueError):
        return None


def graph_time_us(torch, launches, reps=10, inner=2):
    """Mean duration (us) of one call of ``launches`` (a list of zero-argument
    callables, each one kernel launch), from HIP events around replays of a
    graph that holds ``inner`` passes over the list, on the replay stream."""
    for f in launches:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(inner):
                for f in launches:
                    f()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        per.append(1000.0 * a.elapsed_time(b) / (inner * len(launches)))
    per.sort()
    return sum(per) / len(per), per[len(per) // 2]


def c2_inputs(torch, M, synth, copies=17):
    """Tree-attention inputs at the 7B layer shape (KV copies rotated > MALL)."""
    import numpy as np
    B, N, H, D, ctx, P = 1, 64, 32, 128, 2048, 16
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    bf = torch.bfloat16
    pages = (ctx + N + P - 1) // P
    Q = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Kt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Vt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Kc = [torch.randn((pages, H, P, D), generator=gen, device=dev).to(bf) for _ in range(copies)]
    Vc = [torch.randn((pages, H, P, D), generator=gen, device=dev).to(bf) for _ in range(copies)]
    parent, rank = synth.tree_template((4, 3, 2, 2, 1))
    parent, rank = synth.prune_template(parent, rank, N, 2)
    i32 = dict(dtype=torch.int32, device=dev)
    pt = torch.arange(pages, **i32)[None].contiguous()
    ctx_t = torch.tensor([ctx], **i32)
    topk = torch.zeros((5, 1, 4), **i32)
    _, _, mask = M.medusa_build_tree(torch.tensor(parent[None], **i32), torch.tensor(rank[None], **i32),
                                     torch.zeros(1, **i32), topk, ctx_t)
    out = torch.empty_like(Q)
    ws = M._ws(M.tree_attention_ws_bytes(B, N, H, H, D, ctx), dev)
    scale = 1.0 / np.sqrt(D)
    call = lambda i: M.medusa_tree_attention(Q, Kt, Vt, Kc[i], Vc[i], pt, ctx_t, ctx, mask, scale,
                                             out=out, ws=ws)
    return call, dict(B=B, N=N, H=H, D=D, ctx=ctx, P=P, kc_bytes=Kc[0].numel() * 2)


def tree_attention_c2(torch, M, synth, reps=10, copies=17):
    """Tree attention alone at the 7B layer shape; returns a dict of figures."""
    call, c = c2_inputs(torch, M, synth, copies)
    B, N, H, D, ctx = c["B"], c["N"], c["H"], c["D"], c["ctx"]
    launches = [lambda i=i: call(i) for i in range(copies)]
    us, us_med = graph_time_us(torch, launches, reps=reps)
    kv = (ctx + N) * H * D * 2 * 2          # cached + tree K and V read
    nbytes = kv + 2 * B * N * H * D * 2 + N * 8 + N * H * D * 2 * 2  # + Q, O, masks, appended tree K/V
    flops = 4.0 * N * H * D * (ctx + N)     # QK^T and PV, upper bound (all keys)
    gbs = nbytes / (us * 1e-6) / 1e9
    return dict(workload="7B layer: 32 heads x 128, ctx 2048 + 64-node tree, bf16, 16-token pages",
                plan=M.tree_attention_splits(B, N, H, H, D, ctx, c["P"]),
                us=round(us, 3), us_median=round(us_med, 3),
                bytes=nbytes, gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4),
                tflops=round(flops / (us * 1e-6) / 1e12, 2),
                verified_tree_tokens_per_s=round(N / (us * 1e-6), 1),
                timing="HIP events around graph replays of back-to-back launches",
                traffic=measured_traffic("tree_attention", "tree_attention.hip"),
                kv_copies_rotated=copies, rotated_mb=round(copies * 2 * c["kc_bytes"] / 1e6, 1))


def tree_attention_step_shape(torch, M, synth, ctx, max_ctx, reps=10, copies=17):
    """Tree attention alone at the decode step's shape: the 7B layer (32
    heads x 128, 64-node tree) at ``ctx`` cached tokens, planned for
    ``max_ctx`` as the decoder plans it; KV rotated over > 256 MB."""
    import numpy as np
    B, N, H, D, P = 1, 64, 32, 128, 16
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    bf = torch.bfloat16
    pages = (max_ctx + N + P - 1) // P
    Q = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Kt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Vt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Kc = [torch.randn((pages, H, P, D), generator=gen, device=dev).to(bf) for _ in range(copies)]
    Vc = [torch.randn((pages, H, P, D), generator=gen, device=dev).to(bf) for _ in range(copies)]
    parent, rank = synth.prune_template(*synth.tree_template((4, 3, 2, 2, 1)), N, 2)
    i32 = dict(dtype=torch.int32, device=dev)
    pt = torch.arange(pages, **i32)[None].contiguous()
    ctx_t = torch.tensor([ctx], **i32)
    _, _, mask = M.medusa_build_tree(torch.tensor(parent[None], **i32), torch.tensor(rank[None], **i32),
                                     torch.zeros(1, **i32), torch.zeros((5, 1, 4), **i32), ctx_t)
    out = torch.empty_like(Q)
    ws = M._ws(M.tree_attention_ws_bytes(B, N, H, H, D, max_ctx), dev)
    scale = 1.0 / np.sqrt(D)
    launches = [lambda i=i: M.medusa_tree_attention(Q, Kt, Vt, Kc[i], Vc[i], pt, ctx_t, max_ctx, mask, scale,
                                                    out=out, ws=ws) for i in range(copies)]
    us, us_med = graph_time_us(torch, launches, reps=reps)
    nbytes = (ctx + N) * H * D * 2 * 2 + 2 * B * N * H * D * 2 + N * 8 + N * H * D * 2 * 2
    gbs = nbytes / (us * 1e-6) / 1e9
    return dict(workload=f"7B layer: 32 heads x 128, ctx {ctx} + 64-node tree (planned for max_ctx "
                         f"{max_ctx}), bf16, 16-token pages",
                plan=M.tree_attention_splits(B, N, H, H, D, max_ctx, P),
                us=round(us, 3), us_median=round(us_med, 3), bytes=nbytes, gbs=round(gbs, 1),
                frac=round(gbs / HBM_PEAK_GBS, 4),
                traffic=measured_traffic("tree_attention_step", "tree_attention.hip"))


def hbm_copy_rate(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy of ``nbytes`` (HIP events): GB/s counting the
    bytes read and written, the plain-copy rate the kernels' fractions are
    also reported against."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (best * 1e-3) / 1e9, 1)


def c1_generation(torch, synth):
    """The tiny fp32 decoder (2 layers, hidden 256, 4x64 heads, vocab 1000, 3
    heads, top-2 x top-3 tree): 64 tokens of Medusa greedy decoding from a
    32-token prompt, the step graph-replayed; prefill and decode timed apart."""
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder
    m = synth.tiny_decoder(seed=1)
    prompt = synth.prompt_tokens(101, 32, m.vocab)
    parent, rank = synth.tree_template((2, 3))
    dec = MedusaDecoder(DeviceModel(m, dtype=torch.float32), parent, rank, capacity=32 + 64 + 16)
    dec.generate(prompt, 64, graph=True)  # records the step graph
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec.prefill(prompt)
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t0
    rec = []
    t0 = time.perf_counter()
    toks = dec.generate(prompt, 64, record=rec, graph=True)
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t0
    t_dec = max(t_all - t_pre, 1e-9)
    return dict(workload="tiny fp32 decoder (2 layers, hidden 256, vocab 1000) + 3 heads, top-2 x top-3 "
                         "tree (9 nodes), prompt 32, 64 greedy tokens",
                tokens=len(toks), steps=len(rec), mean_accept_len=round(float(sum(rec)) / len(rec), 3),
                tokens_per_s=round(64 / t_dec, 1), prefill_ms=round(1000 * t_pre, 3),
                decode_ms=round(1000 * t_dec, 3))


def c4_generation(torch, model, parent, rank, prompt, mode, n_new=256, **kw):
    """The configuration as stated: 256 tokens generated from the 512-token
    prompt with the step graph-replayed (the device log read once per batch
    of steps); prefill timed apart and excluded from tokens/s."""
    from speculative_decoding_02_amd.decoder import MedusaDecoder
    import numpy as np
    dec = MedusaDecoder(model, parent, rank, capacity=len(prompt) + n_new + 64, mode=mode, **kw)
    dec.generate(prompt, n_new, graph=True)  # records the step graph, warms up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec.prefill(prompt)
    torch.cuda.synchronize()
    t_pre = time.perf_counter() - t0
    rec = []
    t0 = time.perf_counter()
    dec.generate(prompt, n_new, record=rec, graph=True)
    torch.cuda.synchronize()
    t_all = time.perf_counter() - t0
    t_dec = max(t_all - t_pre, 1e-9)
    del dec
    torch.cuda.empty_cache()
    return dict(tokens=n_new, steps=len(rec), mean_accept_len=round(float(np.mean(rec)), 3),
                tokens_per_s=round(n_new / t_dec, 2), ms_per_step=round(1000 * t_dec / len(rec), 3),
                prefill_ms=round(1000 * t_pre, 2), decode_s=round(t_dec, 4), **kw)


def heads_c3(torch, M, rows, reps=10):
    """The five Medusa heads + per-head top-10 at the 7B shape (H 4096, V 32000)
    on ``rows`` hidden rows: stage 1 (residual SiLU layer), stage 2 (vocabulary
    projection, fp32 logits kept in the workspace), top-k."""
    K, H, V, k = 5, 4096, 32000, 10
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    bf = torch.bfloat16
    X = torch.randn((rows, H), generator=gen, device="cuda").to(bf)
    W1 = torch.randn((K, H, H), generator=gen, device="cuda").mul_(0.01).to(bf)
    b1 = torch.randn((K, H), generator=gen, device="cuda").mul_(0.01).to(bf)
    W2 = torch.randn((K, V, H), generator=gen, device="cuda").mul_(0.02).to(bf)
    ids = torch.empty((K, rows, k), dtype=torch.int32, device="cuda")
    vals = torch.empty((K, rows, k), dtype=torch.float32, device="cuda")
    ws = M._ws(M._lib.medusa_heads_ws(rows, H, K, V, k, M.BF16), "cuda")
    call = lambda: M.medusa_heads(X, W1, b1, W2, topk=k, ids=ids, vals=vals, ws=ws, want_logits=False)
    us, us_med = graph_time_us(torch, [call], reps=reps, inner=2)
    nbytes = K * (H * H * 2 + H * 2 + V * H * 2) + rows * H * 2 + K * rows * k * 8
    flops = 2.0 * rows * K * (H * H + V * H)
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    out = dict(workload=f"5 heads, H 4096, V 32000, {rows} rows, top-10, bf16",
               us=round(us, 2), us_median=round(us_med, 2), bytes=nbytes, gbs=round(gbs, 1),
               hbm_frac=round(gbs / HBM_PEAK_GBS, 4), tflops=round(tf, 1),
               mfma_frac=round(tf / MFMA_PEAK_TFLOPS, 4), rows_per_s=round(rows / (us * 1e-6), 1),
               timing="HIP events around graph replays")
    del X, W1, b1, W2, ws
    torch.cuda.empty_cache()
    return out


def batched_attention_c5(torch, M, synth, reps=5):
    """Batched tree verification attention over a 13B-shaped stack: 16
    sequences of U{256..4096} cached tokens (seeded), 40 heads x 128, 16-token
    pages in a seeded permuted order, each sequence its own pruned 64-node
    tree; 40 layer launches, alternating over two layer pools (each larger
    than the 256 MB MALL, so every launch streams its KV from HBM)."""
    import numpy as np
    B, N, H, D, P, L = 16, 64, 40, 128, 16, 40
    rng = np.random.default_rng(np.random.SeedSequence(5))
    lens = rng.integers(256, 4097, B)
    max_ctx = 4096
    max_pages = (max_ctx + N + P - 1) // P
    npg = [(int(l) + N + P - 1) // P for l in lens]
    perm = rng.permutation(sum(npg))
    pt = np.zeros((B, max_pages), np.int32)
    o = 0
    for b in range(B):
        pt[b, :npg[b]] = perm[o:o + npg[b]]
        o += npg[b]
    parents, ranks = [], []
    for b in range(B):
        pa, ra = synth.prune_template(*synth.tree_template((4, 3, 2, 2, 1)), N, 100 + b)
        parents.append(pa)
        ranks.append(ra)
    dev, bf = "cuda", torch.bfloat16
    i32 = dict(dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    pools = [(torch.randn((sum(npg), H, P, D), generator=gen, device=dev).to(bf),
              torch.randn((sum(npg), H, P, D), generator=gen, device=dev).to(bf)) for _ in range(2)]
    Q = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Kt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    Vt = torch.randn((B, N, H, D), generator=gen, device=dev).to(bf)
    ctx = torch.tensor(lens.astype(np.int32), **i32)
    _, _, mask = M.medusa_build_tree(torch.tensor(np.stack(parents), **i32), torch.tensor(np.stack(ranks), **i32),
                                     torch.zeros(B, **i32), torch.zeros((5, B, 4), **i32), ctx)
    ptab = torch.tensor(pt, **i32)
    out = torch.empty_like(Q)
    ws = M._ws(M.tree_attention_ws_bytes(B, N, H, H, D, max_ctx, P), dev)
    scale = 1.0 / np.sqrt(D)
    launches = [lambda li=li: M.medusa_tree_attention(Q, Kt, Vt, pools[li % 2][0], pools[li % 2][1], ptab, ctx,
                                                      max_ctx, mask, scale, out=out, ws=ws)
                for li in range(L)]
    us, us_med = graph_time_us(torch, launches, reps=reps, inner=1)  # per launch
    per_layer = int(sum(int(l) + N for l in lens)) * H * D * 2 * 2 + 2 * B * N * H * D * 2 + B * N * 8 \
        + B * N * H * D * 2 * 2
    gbs = per_layer / (us * 1e-6) / 1e9
    stack_ms = us * L / 1000.0
    res = dict(workload="16 sequences, cached U{256..4096} (seeded), 40 heads x 128, 40 layers, "
                        "16-token pages in permuted order, 64-node tree each, bf16",
               cached_tokens=[int(x) for x in lens], ms_per_stack=round(stack_ms, 3),
               us_per_layer=round(us, 2), bytes_per_layer=per_layer, gbs=round(gbs, 1),
               frac=round(gbs / HBM_PEAK_GBS, 4),
               verified_tree_tokens_per_s=round(B * N / (stack_ms * 1e-3), 1),
               timing="HIP events around graph replays of the 40 layer launches (two layer pools, "
                      "alternating)")
    del pools, Q, Kt, Vt, ws
    torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, dec, model_src, emitted_per_step, sample_layers, reps=3):
    """The oracle, as is, on a bounded sample of one decode step (host cores):
    its BLAS pool runs one thread per CPU this process may use."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=len(os.sched_getaffinity(0))):
        return _cpu_baseline(torch, dec, model_src, emitted_per_step, sample_layers, reps)


def _cpu_baseline(torch, dec, model_src, emitted_per_step, sample_layers, reps):
    import numpy as np
    from threadpoolctl import threadpool_info
    import synth
    from oracle import medusa_oracle as orc

    meta = model_src["meta"]
    H, V = meta["hidden"], meta["vocab"]
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    layers = []
    for L in model_src["layers"][:sample_layers]:
        layers.append({k: host(v) for k, v in L.items()})
    tiny = synth.TinyDecoder(V, H, sample_layers, meta["n_heads"], meta["n_kv_heads"],
                             meta["head_dim"], meta["ffn"], meta["rope_base"], meta["eps"],
                             host(model_src["embed"]), layers, host(model_src["g_final"]),
                             host(model_src["lm_head"]), host(model_src["w1"]), host(model_src["b1"]),
                             host(model_src["w2"]))
    last = dec.last
    ctx = dec.ctx_sample
    tokens = last["tokens"][0].cpu().numpy()
    pos = last["pos"][0].cpu().numpy()
    mask = last["mask"][0].cpu().numpy().view(np.uint64)
    cache = orc.KVCache(tiny, ctx + 64)
    for li in range(sample_layers):
        for pool, dst in ((dec.Kc[li], cache.k[li]), (dec.Vc[li], cache.v[li])):
            rows = pool.float().cpu().numpy().transpose(0, 2, 1, 3).reshape(-1, meta["n_kv_heads"],
                                                                             meta["head_dim"])
            dst[:ctx] = rows[:ctx]
    parent = dec.parent[0].cpu().numpy()
    passes = []
    for _ in range(reps):  # the same step again (the tree rows overwrite their own slots)
        stamps = []
        t0 = time.perf_counter()
        logits, hf = orc.forward_rows(tiny, tokens, pos, mask, cache, ctx,
                                      layer_hook=lambda li, x: stamps.append(time.perf_counter()))
        t1 = time.perf_counter()
        res = orc.accept_greedy(orc.f32(logits), tokens, parent, dec.K)
        hl = orc.head_logits(hf[res["best"]][None], tiny.w1, tiny.b1, tiny.w2)
        ids = [orc.topk(hl[k, 0], dec.width)[0] for k in range(dec.K)]
        t2 = time.perf_counter()
        # embedding + the sampled layers; final norm + lm_head; accept + heads
        passes.append((stamps[-1] - t0, t1 - stamps[-1], t2 - t1))
    passes.sort()
    t_layers, t_head, t_tail = passes[len(passes) // 2]
    t_head += t_tail
    # lm_head, accept and heads ran in full; the layers are scaled to all of them
    step_s = t_layers * meta["n_layers"] / sample_layers + t_head
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return dict(value=round(emitted_per_step / step_s, 4), unit="tokens/s", cores=int(threads),
                kind="oracle", affinity_cpus=len(os.sched_getaffinity(0)), nproc=os.cpu_count(),
                cpu_model=cpu_model(),
                sample=(f"one 64-node verification step at ctx={ctx}, run {reps} times (median): "
                        f"{sample_layers} of {meta['n_layers']} layers timed ({t_layers:.2f} s, "
                        f"scaled x{meta['n_layers'] / sample_layers:g}) plus lm_head, greedy accept "
                        f"and the 5 heads + top-k in full ({t_head:.2f} s); tokens/step from the GPU "
                        f"run ({emitted_per_step:.3f})"),
                step_seconds_extrapolated=round(step_s, 3), _ids=len(ids))


def batched_projections_f4(torch, M, rows=1024, reps=5):
    """One 7B layer's projections for batched tree verification (16 sequences
    x 64 nodes = 1024 rows, bf16): QKV 4096 -> 12288 with rotary positions (as
    the decoder calls it), O 4096 -> 4096 + residual,
    gate/up 4096 -> 2 x 11008 + SwiGLU, down 11008 -> 4096 + residual; the
    MFMA-bound tiling.  Graph-timed; FLOPs = 2 * rows * (sum of K x N)."""
    H, F, Q = 4096, 11008, 12288
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    bf = torch.bfloat16
    w = lambda n, k: torch.randn((n, k), generator=gen, device="cuda").mul_(0.02).to(bf)
    Wqkv, Wo, Wgu, Wd = w(Q, H), w(H, H), w(2 * F, H), w(H, F)
    h = torch.randn((rows, H), generator=gen, device="cuda").to(bf)
    o = torch.randn((rows, H), generator=gen, device="cuda").to(bf)
    x = torch.randn((rows, H), generator=gen, device="cuda")
    pos = torch.arange(600, 600 + rows, dtype=torch.int32, device="cuda")
    q, k, v = (torch.empty((rows, 32, 128), device="cuda", dtype=bf) for _ in range(3))
    f = torch.empty((rows, F), device="cuda", dtype=bf)
    ws = M._ws(max([M.linear_ws_bytes(rows, kk, n, 1, M.BF16) for kk, n in ((H, H), (H, 2 * F), (F, H))] +
                   [M.qkv_rope_ws_bytes(rows, H, 32, 32, 128, M.BF16)]), "cuda")
    launches = [lambda: M.medusa_linear_qkv_rope(h, Wqkv, 32, 32, 128, pos, 10000.0, q=q, k=k, v=v, ws=ws),
                lambda: M.medusa_linear(o, Wo, M.EPI_RES_ADD_F32, aux=x, out=x, ws=ws),
                lambda: M.medusa_linear(h, Wgu, M.EPI_SWIGLU, out=f, ws=ws),
                lambda: M.medusa_linear(f, Wd, M.EPI_RES_ADD_F32, aux=x, out=x, ws=ws)]
    us, med = graph_time_us(torch, launches, reps=reps, inner=2)
    us_layer = us * len(launches)
    flops = 2.0 * rows * (H * Q + H * H + H * 2 * F + F * H)
    tf = flops / (us_layer * 1e-6) / 1e12
    return dict(workload=f"one 7B layer's projections at {rows} rows (16 sequences x 64 tree nodes), bf16",
                us_per_layer=round(us_layer, 1), tflops=round(tf, 1), mfma_frac=round(tf / MFMA_PEAK_TFLOPS, 4),
                timing="HIP events around graph replays of the four launches")


def sampled_accept_us(torch, M):
    """Sampled verification alone on one step's verification logits (64 nodes,
    vocab 32000): one Philox4x64-10 block per 4 entries, Gumbel-max per node,
    the tree sweep.  Graph-timed; the step counter advances every call."""
    import numpy as np
    import synth
    N, V, K = 64, 32000, 5
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    logits = torch.randn((1, N, V), generator=gen, device="cuda")
    parent, _ = synth.prune_template(*synth.tree_template((4, 3, 2, 2, 1)), N, 2)
    par = torch.tensor(parent[None], dtype=torch.int32, device="cuda")
    tok = torch.zeros((1, N), dtype=torch.int32, device="cuda")
    rng = M.rng_state(1, 0)
    out = (torch.empty(1, dtype=torch.int32, device="cuda"),
           torch.empty((1, K + 1), dtype=torch.int32, device="cuda"),
           torch.empty(1, dtype=torch.int32, device="cuda"))
    ws = M._ws(M._lib.medusa_accept_ws(1, N), "cuda")
    us, med = graph_time_us(torch, [lambda: M.medusa_accept_sample(logits, tok, par, K, 1.0, rng,
                                                                    out=out, ws=ws)], reps=10, inner=20)
    return dict(us=round(us, 2), us_median=round(med, 2), nodes=N, vocab=V,
                logits_gbs=round(N * V * 4 / (us * 1e-6) / 1e9, 1))


def kernels_only(torch, M, synth, log):
    """Counter-pass workload: 32 gate/up projection launches (64 rows, 7B
    shapes, one weight copy per layer as in the step), 17 tree-attention
    launches at the 7B layer shape, and a 1 GiB device copy whose byte count
    calibrates FETCH_SIZE / WRITE_SIZE."""
    H, F = 4096, 11008
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    hin = torch.randn((64, H), generator=gen, device="cuda").to(torch.bfloat16)
    gout = torch.empty((64, F), device="cuda", dtype=torch.bfloat16)
    gws = M._ws(M.linear_ws_bytes(64, H, 2 * F, 1, M.BF16), "cuda")
    log("[bench] kernels-only: gate/up launches")
    for _ in range(32):
        w = torch.randn((2 * F, H), generator=gen, device="cuda").mul_(0.02).to(torch.bfloat16)
        torch.cuda.synchronize()
        M.medusa_linear(hin, w, M.EPI_SWIGLU, out=gout, ws=gws)
        torch.cuda.synchronize()
        del w
    log("[bench] kernels-only: tree attention")
    call, _ = c2_inputs(torch, M, synth, 17)
    for i in range(17):
        call(i)
    torch.cuda.synchronize()
    log("[bench] kernels-only: 1 GiB calibration copy")
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"kernels_only": True, "copy_bytes": 1 << 30,
                      "gate_up_bytes_per_launch": 2 * F * H * 2 + 64 * H * 2 + 64 * F * 2}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--mode", default="greedy", choices=["greedy", "typical"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-layers", type=int, default=16)
    ap.add_argument("--skip-c2", action="store_true")
    ap.add_argument("--skip-plain", action="store_true")
    ap.add_argument("--skip-extra", action="store_true",
                    help="skip the heads (64 and 1024 rows) and batched-attention measurements")
    ap.add_argument("--heads-only", action="store_true",
                    help="run only the five heads + top-10 at 64 and 1024 rows (for kernel traces)")
    ap.add_argument("--attn-only", action="store_true",
                    help="run only tree attention at the 7B layer shape (2048 cached tokens) and at "
                         "the decode step's shape, for per-shape kernel traces")
    ap.add_argument("--config", choices=["c1", "c2", "c3", "c5"],
                    help="run one configuration's measurement alone and print its JSON object: "
                         "c1 the tiny fp32 model's 64 greedy tokens, c2 tree attention at the 7B "
                         "layer (and at the decode step's shape), c3 the five heads + top-10 at 64 "
                         "and 1024 rows, c5 the ragged 16-sequence 13B attention stack (c4 is the "
                         "default run)")
    ap.add_argument("--f4-only", action="store_true",
                    help="run only one 7B layer's four projections at 1024 rows (the large-row "
                         "tiling), for kernel traces and counter passes")
    ap.add_argument("--skip-generation", action="store_true",
                    help="skip the 256-token generations (greedy, typical) and the tiny fp32 model")
    ap.add_argument("--kernels-only", action="store_true",
                    help="run only the dominant projection kernel (32 launches over 7B-shaped "
                         "gate/up weights), the tree-attention launches and a 1 GiB copy, "
                         "for hardware-counter passes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the one-GPU Medusa step; runs on more than one GPU are not "
              "part of this implementation: it would shard tree attention by head or sequence "
              "and the heads' vocabulary projection by vocabulary slice, one GPU's share being "
              "what this measures.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from speculative_decoding_02_amd import medusa as M
    from speculative_decoding_02_amd.decoder import DeviceModel, MedusaDecoder

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    if args.kernels_only:
        kernels_only(torch, M, synth, log)
        return
    if args.config == "c1":
        print(json.dumps({"c1_tiny_fp32": c1_generation(torch, synth)}))
        return
    if args.config == "c5":
        print(json.dumps({"batched_attention_c5": batched_attention_c5(torch, M, synth)}))
        return
    if args.config == "c3":
        args.heads_only = True
    if args.config == "c2":
        args.attn_only = True
    if args.heads_only:
        print(json.dumps({"heads_c3": heads_c3(torch, M, 64), "heads_c3b": heads_c3(torch, M, 1024)}))
        return
    if args.f4_only:
        print(json.dumps({"batched_projections_f4": batched_projections_f4(torch, M)}))
        return
    if args.attn_only:
        from speculative_decoding_02_amd.decoder import plan_cache
        cap = 512 + 6 * (args.warmup + args.steps) + 128
        print(json.dumps({"tree_attention": tree_attention_c2(torch, M, synth),
                          "tree_attention_step": tree_attention_step_shape(
                              torch, M, synth, 531, plan_cache(cap, 64, 16)[2])}))
        return
    log("[bench] drawing the random 7B-shaped decoder on the GPU")
    src = synth.device_llama(seed=4)
    model = DeviceModel.from_llama(src)
    parent, rank = synth.prune_template(*synth.tree_template((4, 3, 2, 2, 1)), 64, 2)
    prompt = synth.prompt_tokens(4, 512, 32000)
    capacity = 512 + 6 * (args.warmup + args.steps) + 128
    def timed_steps(d, steps, warmup, prompts=None):
        """Warm up, restart from the prompt, then time `steps` graph replays.
        The fused tail logs the emitted tokens on the device, so the timed
        replays run back to back and the log is read once afterwards; the
        separate tail reads accept_len after every step.  Returns (emitted,
        accept lengths, seconds) of the first sequence; with a batch, also
        the batch's total emitted tokens as d.batch_emitted."""
        pr = prompt if prompts is None else prompts
        d.prefill(pr)
        d.capture()
        for _ in range(warmup):
            d.step_graph()
        d.prefill(pr)  # timed steps start from the prompt again
        torch.cuda.synchronize()
        accs = []
        t0 = time.perf_counter()
        for _ in range(steps):
            acc, _, _ = d.step_graph()
            if not d.fused:
                accs.append(int(acc.item()))
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        if d.fused:
            lga = d.log.cpu().numpy()
            lg = lga[0]
            cap = (len(lg) - 2) // 2
            assert int(lg[1]) == steps
            accs = [int(a) for a in lg[2 + cap:2 + cap + steps]]
            d.batch_emitted = int(lga[:, 0].sum())
        return sum(a + 1 for a in accs), accs, sec

    dec = MedusaDecoder(model, parent, rank, capacity=capacity, mode=args.mode)
    log(f"[bench] prefill 512 + record the step graph + {args.warmup} warmup + {args.steps} timed "
        "steps (graph replays back to back; the decode log is read once at the end)")
    emitted, accepts, secs = timed_steps(dec, args.steps, args.warmup)
    dec.ctx_sample = 512 + emitted - (accepts[-1] + 1)  # ctx of the last timed step
    step_ms = 1000.0 * secs / args.steps
    tok_s = emitted / secs
    sep = None
    if not args.skip_plain:
        log("[bench] the same step with the tail as separate launches and a host read per step")
        sdec = MedusaDecoder(model, parent, rank, capacity=capacity, mode=args.mode, tail="separate")
        s_emit, s_acc, s_sec = timed_steps(sdec, args.steps, args.warmup)
        sep = dict(tokens_per_s=round(s_emit / s_sec, 2), ms_per_step=round(1000 * s_sec / args.steps, 3),
                   mean_accept_len=round(float(np.mean(s_acc)), 3))
        del sdec

    # dominant kernel: the gate/up projection (SwiGLU epilogue), weight
    # streaming; one step's 32 launches over the model's own weights
    H, F = 4096, 11008
    hin = torch.randn((64, H), device="cuda").to(torch.bfloat16)
    gout = torch.empty((64, F), device="cuda", dtype=torch.bfloat16)
    gws = M._ws(M.linear_ws_bytes(64, H, 2 * F, 1, M.BF16), "cuda")
    gu_launches = [lambda L=L: M.medusa_linear(hin, L["wgu"], M.EPI_SWIGLU, out=gout, ws=gws)
                   for L in model.t["layers"]]
    gu_us, gu_med = graph_time_us(torch, gu_launches, reps=10, inner=2)
    gu_bytes = 2 * F * H * 2 + 64 * H * 2 + 64 * F * 2
    gu_gbs = gu_bytes / (gu_us * 1e-6) / 1e9

    plain = None
    if not args.skip_plain:
        log("[bench] plain one-token greedy decoding on the same path")
        pdec = MedusaDecoder(model, np.array([-1]), np.array([0]), capacity=capacity)
        p_emit, _, p_sec = timed_steps(pdec, args.steps, 3)
        plain = round(p_emit / p_sec, 2)
        del pdec

    def other_mode(mode, tree=None, **kw):
        """Emitted tokens/s of the same step with another acceptance rule (and tree)."""
        tp, tr = tree if tree is not None else (parent, rank)
        odec = MedusaDecoder(model, tp, tr, capacity=capacity, mode=mode, **kw)
        o_emit, o_acc, dt_ = timed_steps(odec, args.steps, args.warmup)
        del odec
        return dict(tokens_per_s=round(o_emit / dt_, 2), mean_accept_len=round(float(np.mean(o_acc)), 3),
                    ms_per_step=round(1000 * dt_ / args.steps, 3), **kw)

    typical = sampled = sparse = None
    if args.mode == "greedy" and not args.skip_plain:
        log("[bench] typical acceptance (epsilon 0.3, delta 0.09) on the same model")
        typical = other_mode("typical", epsilon=0.3, delta=0.09)
        log("[bench] sampled verification (temperature 1, seed 0) on the same model")
        sampled = other_mode("sample", temperature=1.0, seed=0)
        sampled["accept_kernel"] = sampled_accept_us(torch, M)
        log("[bench] typical acceptance on a 64-node tree of the most accurate combinations")
        acc_table = np.array([[0.7 * 0.5 ** r for r in range(4)] for _ in range(5)], np.float32)
        sp, sr, exp_acc = M.medusa_tree_from_accuracy(acc_table, 64)
        sparse = other_mode("typical", tree=(sp, sr), epsilon=0.3, delta=0.09)
        sparse["tree"] = "64 nodes from a synthetic accuracy table a[d][r] = 0.7 * 0.5^r (5 heads x top-4)"
        sparse["table_expected_accept"] = round(exp_acc, 4)

    batched = None
    if not args.skip_extra:
        log("[bench] batched decoding: 16 sequences x 64-node trees (1024 verification rows)")
        Bb, bsteps = 16, 10
        bprompts = np.stack([synth.prompt_tokens(40 + b, 512, 32000) for b in range(Bb)])
        # each sequence verifies its own pruned 64-node template
        bparent, brank = synth.random_template_batch((4, 3, 2, 2, 1), 64, [100 + b for b in range(Bb)])
        bdec = MedusaDecoder(model, bparent, brank, capacity=512 + 6 * (2 + bsteps) + 128,
                             mode=args.mode, batch=Bb)
        _, b_acc, b_sec = timed_steps(bdec, bsteps, 2, prompts=bprompts)
        batched = dict(workload="16 sequences (prompts of 512, own pages and contexts), each with its "
                                "own pruned 64-node tree: 1024 rows through every projection, batched "
                                "attention, fused tail; greedy",
                       sequences=Bb, steps=bsteps, tokens_per_s=round(bdec.batch_emitted / b_sec, 1),
                       ms_per_step=round(1000 * b_sec / bsteps, 3),
                       verified_tree_tokens_per_s=round(Bb * 64 * bsteps / b_sec, 1),
                       mean_accept_len_seq0=round(float(np.mean(b_acc)), 3))
        del bdec
        torch.cuda.empty_cache()

    gen = c1 = None
    if not args.skip_generation:
        log("[bench] the configuration as stated: 256 tokens from the 512-token prompt, greedy then typical")
        gen = {"greedy": c4_generation(torch, model, parent, rank, prompt, "greedy"),
               "typical": c4_generation(torch, model, parent, rank, prompt, "typical", epsilon=0.3,
                                        delta=0.09)}
        log("[bench] the tiny fp32 decoder: 64 greedy tokens")
        c1 = c1_generation(torch, synth)
    c2 = step_attn = None
    if not args.skip_c2:
        from speculative_decoding_02_amd.decoder import plan_cache
        c2 = tree_attention_c2(torch, M, synth)
        step_attn = tree_attention_step_shape(torch, M, synth, dec.ctx_sample, dec.max_ctx)
    log("[bench] plain device-to-device copy (the measured streaming rate)")
    copy_gbs = hbm_copy_rate(torch)
    c3 = c3b = c5 = f4 = None
    if not args.skip_extra:
        log("[bench] heads at the 7B shape: 64 rows, then 1024 rows")
        c3 = heads_c3(torch, M, 64)
        c3b = heads_c3(torch, M, 1024, reps=3)
        log("[bench] batched tree attention over a 13B-shaped stack")
        c5 = batched_attention_c5(torch, M, synth)
        log("[bench] one layer's projections at 1024 rows")
        f4 = batched_projections_f4(torch, M)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded sample)")
        cpu = cpu_baseline(torch, dec, src, emitted / args.steps, args.cpu_sample_layers)
        cpu.pop("_ids", None)

    line = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and prompt)",
        "config": {"workload": "Medusa decode step, random Llama-7B-shaped bf16 decoder "
                               "(32 layers, hidden 4096, 32x128 heads, FFN 11008, vocab 32000) + "
                               "5 Medusa heads, prompt 512, 64-node tree (4,3,2,2,1) pruned",
                   "mode": args.mode, "tree_nodes": 64, "prompt": 512, "batch": 1},
        "mean_accept_len": round(float(np.mean(accepts)), 3),
        "tokens_per_step": round(emitted / args.steps, 3),
        "verified_tree_tokens_per_s": round(64 * args.steps / secs, 1),
        "plain_decode_tokens_per_s": plain,
        "tail_separate": sep,
        "batched_decode_f4": batched,
        "typical": typical,
        "sampled": sampled,
        "sparse_tree_typical": sparse,
        "c4_generation": gen,
        "c1_tiny_fp32": c1,
        "hbm_copy_gbs": copy_gbs,
        "roofline": {"bound": "hbm", "kernel": "gemm_xdma_kernel (gate/up projection, SwiGLU epilogue)",
                     "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                     "frac_of_copy": round(gu_gbs / copy_gbs, 4),
                     "traffic": measured_traffic("gate_up_projection", "gemm.hip"),
                     "bytes_per_launch": gu_bytes, "us_per_launch": round(gu_us, 2),
                     "us_median": round(gu_med, 2),
                     "timing": "HIP events around graph replays of the 32 per-step launches"},
        "tree_attention": dict(c2, frac_of_copy=round(c2["gbs"] / copy_gbs, 4)) if c2 else None,
        "tree_attention_step": dict(step_attn, frac_of_copy=round(step_attn["gbs"] / copy_gbs, 4))
        if step_attn else None,
        "heads_c3": c3,
        "heads_c3b": c3b,
        "batched_attention_c5": c5,
        "batched_projections_f4": f4,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
