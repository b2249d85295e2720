"""Medusa decode loop on one GPU, driven entirely through libmedusa.

One decode step ("Medusa Heads", sections "Come le teste prevedono i token
successivi" and "Attenzione sull'albero e accettazione"):

  tree build  (root token + per-head top-k -> N tree tokens, positions, masks;
              with the embedding rows and the first RMSNorm: medusa_tree_embed)
  verification forward of the N tree rows in ONE pass (Llama-style layers;
      tree-masked attention over the paged KV cache + the tree's own keys)
  tail        (medusa_decode_tail: accept, greedy / typical / sampled, keep only
              the accepted branch in every layer's cache, the kept branch's
              last hidden state, next root token, context length, decode log)
  heads       (that hidden state -> the next round's top-k)

``tail="separate"`` runs the same step with the individual calls
(medusa_build_tree, medusa_embed, medusa_rmsnorm, medusa_accept, kv_compact,
medusa_gather_rows) and host copies.  Python only allocates device buffers,
uploads static inputs (weights, tree template, prompts) and reads back the
emitted tokens; every computation is a library kernel.  Weight layout chosen for the GPU: Wq|Wk|Wv stacked into one
[(Hq+2Hkv)*D, H] matrix, and gate/up interleaved in 16-row blocks so the
down-projection input comes straight out of the SwiGLU epilogue.
"""
from __future__ import annotations

import numpy as np
import torch

from . import medusa as M


def interleave_gate_up(wg: np.ndarray, wu: np.ndarray) -> np.ndarray:
    """[F,H] gate and up -> [2F,H] with block j = gate rows 16j.. then up rows 16j.."""
    F, H = wg.shape
    assert F % 16 == 0
    return np.stack([wg.reshape(F // 16, 16, H), wu.reshape(F // 16, 16, H)], axis=1).reshape(2 * F, H)


def max_step_context(plen: int, n_new: int, K: int, B: int) -> int:
    """The largest context length a decode step of ``generate`` can start
    from, for prompts of ``plen`` tokens and ``n_new`` new ones per sequence.

    Every step emits 1..K+1 tokens per sequence.  One sequence: a step starts
    only while fewer than n_new tokens are out, and the batches of steps run
    back to back before a read never start one past that (a batch of r =
    ceil(remaining / (K+1)) steps starts its last step after at most
    (r-1)(K+1) < remaining more tokens), so the bound is plen + n_new - 1.
    B sequences: the loop runs until the slowest one is done, at most n_new
    steps, while the fastest may emit K+1 tokens in each, so the bound is
    plen + (n_new - 1)(K+1)."""
    if n_new <= 0:
        return plen
    return plen + (n_new - 1) * (1 if B == 1 else K + 1)


def plan_cache(capacity: int, N: int, page_size: int):
    """Pages per sequence, slots per sequence and the attention calls'
    max_ctx for a requested ``capacity`` of cached tokens and N-node trees.

    Every attention call (a prefill chunk of up to 64 rows, or a tree of N)
    needs ctx + rows <= slots, so max_ctx = slots - 64; the slots cover the
    requested capacity plus one tree and one chunk."""
    max_pages = (capacity + N + 64 + page_size - 1) // page_size
    slots = max_pages * page_size
    return max_pages, slots, slots - 64


def check_generation(plen: int, n_new: int, K: int, B: int, max_ctx: int) -> None:
    """Raise ValueError unless every attention call of a generation of n_new
    tokens from prompts of plen starts at a context <= max_ctx (a longer one
    would be clamped by the kernels, dropping keys): the prefill's chunks
    start below plen, the decode steps at most at max_step_context."""
    worst = max(max_step_context(plen, n_new, K, B), plen)
    if worst > max_ctx:
        raise ValueError(f"a step may start at context {worst} > max_ctx {max_ctx}: "
                         "raise the capacity")


class DeviceModel:
    """Device copy of a Llama-style decoder with Medusa heads.

    ``src`` is any object with the fields of ``synth.TinyDecoder`` (numpy
    arrays), or None together with ``tensors`` (a dict of ready device tensors,
    used for large random models generated on the GPU).
    """

    def __init__(self, src=None, dtype=torch.float32, device="cuda", tensors=None, meta=None):
        self.dtype, self.device = dtype, torch.device(device)
        if src is not None:
            meta = dict(vocab=src.vocab, hidden=src.hidden, n_layers=src.n_layers,
                        n_heads=src.n_heads, n_kv_heads=src.n_kv_heads, head_dim=src.head_dim,
                        ffn=src.ffn, rope_base=src.rope_base, eps=src.eps)
            up = lambda a: torch.tensor(np.ascontiguousarray(a, dtype=np.float32)).to(
                device=self.device, dtype=dtype)
            t = dict(embed=up(src.embed), g_final=up(src.g_final), lm_head=up(src.lm_head),
                     w1=up(src.w1), b1=up(src.b1), w2=up(src.w2), layers=[])
            Hq, Hkv, D = src.n_heads, src.n_kv_heads, src.head_dim
            for L in src.layers:
                t["layers"].append(dict(
                    wqkv_rp=up(np.concatenate([M.interleave_rope_pairs(L["wq"], Hq, D),
                                               M.interleave_rope_pairs(L["wk"], Hkv, D), L["wv"]],
                                              axis=0)),
                    wo=up(L["wo"]),
                    wgu=up(interleave_gate_up(L["wg"], L["wu"])), wd=up(L["wd"]),
                    g_attn=up(L["g_attn"]), g_mlp=up(L["g_mlp"])))
            tensors = t
        self.meta = meta
        self.t = tensors
        if "wqkv_rp" not in tensors["layers"][0]:  # Llama layout -> GPU layout (one-time copy)
            self.t = dict(tensors)
            self.t["layers"] = [self._gpu_layout(L, meta) for L in tensors["layers"]]
        for k, v in meta.items():
            if k != "seed":
                setattr(self, k, v)
        self.n_medusa = tensors["w1"].shape[0]


    @staticmethod
    def _gpu_layout(L, meta):
        """QKV rows concatenated with the q and k heads pair-interleaved (for the
        projection with rotary positions fused), gate/up interleaved in 16-row
        blocks (for the SwiGLU epilogue)."""
        wg, wu = L["wg"], L["wu"]
        F, H = wg.shape
        wgu = torch.stack([wg.reshape(F // 16, 16, H), wu.reshape(F // 16, 16, H)], 1)
        D = meta["head_dim"]
        wqkv = torch.cat([M.interleave_rope_pairs(L["wq"], meta["n_heads"], D),
                          M.interleave_rope_pairs(L["wk"], meta["n_kv_heads"], D), L["wv"]], 0)
        return dict(wqkv_rp=wqkv.contiguous(), wo=L["wo"],
                    wgu=wgu.reshape(2 * F, H).contiguous(), wd=L["wd"], g_attn=L["g_attn"],
                    g_mlp=L["g_mlp"])

    @classmethod
    def from_llama(cls, d):
        """Build from ``synth.device_llama`` output (tensors already on the GPU)."""
        t = {k: v for k, v in d.items() if k != "meta"}
        return cls(None, dtype=d["embed"].dtype, device=d["embed"].device, tensors=t,
                   meta=dict(d["meta"]))


class MedusaDecoder:
    """Paged-KV Medusa decoding of B sequences at once (B = ``batch``, default 1).

    ``parent``, ``rank``: the tree template (node 0 = root): ``[N]``, shared
    by the batch, or ``[batch, N]``, one template per sequence (the same node
    count; the heads run to the deepest template and give each head's top-k
    for the widest, of which a narrower template uses a prefix).  A
    single-node template turns the loop into plain greedy decoding (no heads).  ``mode``: "greedy", "typical" or "sample" (sampled
    verification with the counter-based stream keyed by ``seed``: the
    prefill's next token draws at step 0, decode step s at step s; sequence b
    draws with counter word b).  Each sequence owns ``capacity`` cache slots
    (its own pages); the verification forward runs the B trees' B*N rows
    through every projection at once.
    """

    def __init__(self, model: DeviceModel, parent, rank, capacity, page_size=16, mode="greedy",
                 temperature=1.0, epsilon=0.3, delta=0.09, seed=0, tail="fused", batch=1):
        self.m = model
        parent = np.asarray(parent, np.int32)
        rank = np.asarray(rank, np.int32)
        self.B = B = int(batch)
        if B < 1:
            raise ValueError(f"batch {batch}")
        if parent.ndim == 1:
            parent = np.tile(parent, (B, 1))
        if rank.ndim == 1:
            rank = np.tile(rank, (B, 1))
        if parent.ndim != 2 or parent.shape[0] != B or rank.shape != parent.shape:
            raise ValueError(f"templates {parent.shape} / {rank.shape} for a batch of {B}")
        self.N = parent.shape[1]
        depth = np.zeros(parent.shape, np.int32)
        for i in range(1, self.N):
            depth[:, i] = depth[np.arange(B), np.clip(parent[:, i], 0, i - 1)] + 1
        self.K = int(depth.max())
        self.width = int(rank.max()) + 1
        if self.K > 0:
            for b in range(B):
                M.medusa_tree_validate(parent[b], rank[b], self.K, self.width)
        dev = model.device
        if mode not in ("greedy", "typical", "sample"):
            raise ValueError(f"mode {mode!r}")
        if tail not in ("fused", "separate"):
            raise ValueError(f"tail {tail!r}")
        self.fused = tail == "fused"
        self.sampled = mode == "sample"
        self.mode = 0 if mode == "greedy" else 1
        self.T, self.eps, self.delta = temperature, epsilon, delta
        self.P = page_size
        self.max_pages, self.capacity, self.max_ctx = plan_cache(capacity, self.N, page_size)
        i32 = dict(dtype=torch.int32, device=dev)
        self.parent = torch.tensor(parent, **i32)
        self.rank = torch.tensor(rank, **i32)
        # sequence b owns pages b*max_pages .. (b+1)*max_pages-1 of every pool
        self.page_table = torch.arange(B * self.max_pages, **i32).reshape(B, self.max_pages).contiguous()
        shape = (B * self.max_pages, model.n_kv_heads, page_size, model.head_dim)
        self.Kc = [torch.zeros(shape, dtype=model.dtype, device=dev) for _ in range(model.n_layers)]
        self.Vc = [torch.zeros(shape, dtype=model.dtype, device=dev) for _ in range(model.n_layers)]
        self.ctx = torch.zeros(B, **i32)
        self.ctx_host = 0
        self.root = torch.zeros(B, **i32)
        Kh = max(self.K, 1)
        if self.K > model.n_medusa:
            raise ValueError(f"the tree is {self.K} deep; the model has {model.n_medusa} heads")
        self.topk_ids = torch.zeros((Kh, B, self.width), **i32)
        self.topk_vals = torch.zeros((Kh, B, self.width), dtype=torch.float32, device=dev)
        # the fused step takes the heads' per-chunk top-k lists and merges them
        # inside the tree build (one launch fewer than a separate merge)
        S = M._lib.medusa_topk_lists(model.vocab)
        self.list_ids = torch.zeros((Kh, B, S, self.width), **i32)
        self.list_vals = torch.zeros((Kh, B, S, self.width), dtype=torch.float32, device=dev)
        self.attn_ws = M._ws(max(M.tree_attention_ws_bytes(B, n, model.n_heads, model.n_kv_heads,
                                                           model.head_dim, self.max_ctx, page_size)
                                 for n in range(1, 65)), dev)
        self.acc_ws = M._ws(M._lib.medusa_accept_ws(B, 64), dev)
        dt = M._dt(model.t["embed"])
        self.heads_ws = M._ws(M._lib.medusa_heads_ws(B, model.hidden, model.n_medusa, model.vocab,
                                                     self.width, dt), dev)
        # split-contraction scratch of the verification projections (rows <= 64 per sequence)
        H, F, V = model.hidden, model.ffn, model.vocab
        qkv_n = (model.n_heads + 2 * model.n_kv_heads) * model.head_dim
        shapes = [(H, qkv_n), (model.n_heads * model.head_dim, H), (H, 2 * F), (F, H), (H, V)]
        self.lin_ws = M._ws(max([M.linear_ws_bytes(B * n, kd, nn, 1, dt) for n in range(1, 65)
                                 for kd, nn in shapes] + [256]), dev)
        self.qkv_ws = M._ws(max([M._lib.medusa_linear_qkv_rope_ws(B * n, H, model.n_heads,
                                                                  model.n_kv_heads,
                                                                  model.head_dim, dt)
                                 for n in range(1, 65)] + [256]), dev)
        self.out = (torch.zeros(B, **i32), torch.zeros((B, self.K + 1), **i32), torch.zeros(B, **i32))
        # sampled mode: (seed, step) on the device, advanced by every draw; a
        # one-node tree draws the prefill's next token
        self.seed = seed
        self.rng = M.rng_state(seed, 0, dev)
        self.one_tok = torch.zeros((B, 1), **i32)
        self.one_parent = torch.full((B, 1), -1, **i32)
        self.one_out = (torch.zeros(B, **i32), torch.zeros((B, 1), **i32), torch.zeros(B, **i32))
        # the fused tail: per-sequence arrival counters (zero-filled here, left
        # zero by every call), the kept hidden rows, and the decode log
        self.tail_ws = M._ws(M._lib.medusa_decode_tail_ws(B, 64), dev)
        self.h_best = torch.zeros((B, model.hidden), dtype=model.dtype, device=dev)
        self.log = M.decode_log(B, self.capacity, dev)
        self.new_ctx = torch.zeros(B, **i32)
        self.src = torch.zeros((B, self.K + 1), **i32)
        self.dst = torch.zeros((B, self.K + 1), **i32)

    # ------------------------------------------------------------------
    def forward(self, tokens, pos, mask):
        """Verification forward of n rows per sequence (tokens/pos [B,n] int32,
        mask [B,n] int64).

        Stores the rows' K/V at cache slots ctx..ctx+n-1.  Returns (logits
        [B*n,V] float32, final hidden [B*n,H] model dtype), rows sequence-major."""
        m, t = self.m, self.m.t
        x = M.medusa_embed(tokens.reshape(-1), t["embed"])
        h = M.medusa_rmsnorm(x, t["layers"][0]["g_attn"], m.eps, m.dtype)
        return self._layers(x, h, pos, mask)

    def _layers(self, x, h, pos, mask):
        """The layers, final norm and lm_head over B*n rows: x [B*n, H] float
        (the residual stream, updated in place), h = the first block's RMSNorm
        of x."""
        m, t = self.m, self.m.t
        rows = x.shape[0]
        n = rows // self.B
        scale = 1.0 / float(np.sqrt(m.head_dim))
        layers = t["layers"]
        for li, L in enumerate(layers):
            q, k, v = M.medusa_linear_qkv_rope(h, L["wqkv_rp"], m.n_heads, m.n_kv_heads,
                                               m.head_dim, pos.reshape(-1), m.rope_base,
                                               ws=self.qkv_ws)
            o = M.medusa_tree_attention(q.view(self.B, n, m.n_heads, m.head_dim),
                                        k.view(self.B, n, m.n_kv_heads, m.head_dim),
                                        v.view(self.B, n, m.n_kv_heads, m.head_dim),
                                        self.Kc[li], self.Vc[li], self.page_table, self.ctx,
                                        self.max_ctx, mask, scale, ws=self.attn_ws)
            # residual projections carry the next RMSNorm (the last one: the final norm)
            h = M.medusa_linear_rmsnorm(o.reshape(rows, -1), L["wo"], x, L["g_mlp"], m.eps,
                                        ws=self.lin_ws)
            f = M.medusa_linear(h, L["wgu"], M.EPI_SWIGLU, ws=self.lin_ws)
            g_next = layers[li + 1]["g_attn"] if li + 1 < len(layers) else t["g_final"]
            h = M.medusa_linear_rmsnorm(f, L["wd"], x, g_next, m.eps, ws=self.lin_ws)
        hN = h
        logits = M.medusa_linear(hN, t["lm_head"], y_f32=True, ws=self.lin_ws)
        return logits, hN

    def _heads(self, h_rows):
        """The first K heads (K = the tree's depth) on the rows: per-chunk
        top-k lists for the fused step, merged top-k lists otherwise."""
        if self.K == 0:
            return
        t = self.m.t
        w1, b1, w2 = t["w1"][:self.K], t["b1"][:self.K], t["w2"][:self.K]
        if self.fused:
            M.medusa_heads_lists(h_rows, w1, b1, w2, self.width, ids=self.list_ids,
                                 vals=self.list_vals, ws=self.heads_ws)
        else:
            M.medusa_heads(h_rows, w1, b1, w2, self.width, logits=None, ids=self.topk_ids,
                           vals=self.topk_vals, ws=self.heads_ws, want_logits=False)

    def _set_ctx(self, c):
        self.ctx.fill_(int(c))
        self.ctx_host = c

    def prefill(self, prompt):
        """Causal forward over the prompts ([P] for one sequence, or [B, P]) in
        chunks of <= 64 chain-masked rows per sequence."""
        prompt = np.asarray(prompt, np.int32).reshape(self.B, -1)
        dev = self.m.device
        B = self.B
        self._set_ctx(0)
        self.rng.copy_(M.rng_state(self.seed, 0, dev))  # a generation's draws start at step 0
        self.log.zero_()
        c, plen = 0, prompt.shape[1]
        while c < plen:
            n = min(64, plen - c)
            tok = torch.tensor(prompt[:, c:c + n], dtype=torch.int32, device=dev).contiguous()
            pos = torch.arange(c, c + n, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
            mask = torch.tensor([[(1 << (i + 1)) - 1 if i < 63 else -1 for i in range(n)]] * B,
                                dtype=torch.int64, device=dev)
            logits, hN = self.forward(tok, pos, mask)
            c += n
            self._set_ctx(c)
        last = logits.view(B, n, -1)[:, n - 1].contiguous()
        if self.sampled:
            _, _, nxt = M.medusa_accept_sample(last[:, None], self.one_tok, self.one_parent, 0,
                                               self.T, self.rng, out=self.one_out, ws=self.acc_ws)
            self.root.copy_(nxt)
        else:
            ids, _ = M.medusa_topk(last, 1)
            self.root.copy_(ids.reshape(B))
        self._heads(hN.view(B, n, -1)[:, n - 1].contiguous())

    def step(self):
        """One Medusa decode step of the batch (all on the GPU); returns
        (accept_len [B], path [B,K+1], tokens [B,N]) tensors."""
        if self.fused:
            tokens, pos, mask, x, h = M.medusa_tree_embed(
                self.parent, self.rank, self.root, self.list_ids, self.ctx, self.m.t["embed"],
                self.m.t["layers"][0]["g_attn"], self.m.eps, topk_vals=self.list_vals)
            logits, hN = self._layers(x, h, pos, mask)
            acc, path, nxt, hbest = M.medusa_decode_tail(
                logits.view(self.B, self.N, -1), tokens, self.parent, self.K,
                2 if self.sampled else self.mode, self.Kc, self.Vc, self.page_table,
                hN.view(self.B, self.N, -1), self.ctx, self.root, self.log,
                temperature=self.T, epsilon=self.eps, delta=self.delta, rng=self.rng,
                h_best=self.h_best, out=self.out, ws=self.tail_ws)
            if self.K > 0:
                self._heads(hbest)
            self.last = dict(tokens=tokens, logits=logits, hN=hN, pos=pos, mask=mask)
            return acc, path, tokens
        tokens, pos, mask = M.medusa_build_tree(self.parent, self.rank, self.root,
                                                self.topk_ids, self.ctx)
        logits, hN = self.forward(tokens, pos, mask)
        lv = logits.view(self.B, self.N, -1)
        if self.sampled:
            acc, path, nxt = M.medusa_accept_sample(lv, tokens, self.parent, self.K, self.T,
                                                    self.rng, out=self.out, ws=self.acc_ws)
        else:
            acc, path, nxt = M.medusa_accept(lv, tokens, self.parent, self.K, self.mode,
                                             self.T, self.eps, self.delta, out=self.out,
                                             ws=self.acc_ws)
        M.kv_compact(self.Kc, self.Vc, self.page_table, self.ctx, path, acc, new_ctx=self.new_ctx,
                     src=self.src, dst=self.dst)
        if self.K > 0:
            hbest = M.medusa_gather_rows(hN.view(self.B, self.N, -1), path, acc)
            self._heads(hbest)
        self.root.copy_(nxt)
        self.ctx.copy_(self.new_ctx)
        self.last = dict(tokens=tokens, logits=logits, hN=hN, pos=pos, mask=mask)
        return acc, path, tokens

    # ------------------------------------------------------------------
    def capture(self):
        """Record one decode step as a HIP graph (replayed by ``step_graph``).

        Every call of the step reads its changing state (ctx, root token,
        top-k ids) from device memory and has static shapes, so one recording
        serves every later step; recording runs nothing.  Workspaces are all
        preallocated, so the graph holds no allocation and no memset."""
        self.graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(self.graph, stream=stream):
                self.g_out = self.step()
                self.g_last = self.last
        torch.cuda.current_stream().wait_stream(stream)
        return self.graph

    def step_graph(self):
        """Replay the recorded step; same outputs as ``step``."""
        self.graph.replay()
        self.last = self.g_last
        return self.g_out

    def generate(self, prompt, n_new, record=None, graph=False):
        """Prefill, then Medusa steps until every sequence has emitted n_new
        tokens.  Returns int32 [n_new] (one sequence) or [B, n_new].

        With the fused tail the emitted tokens collect in the device log and
        the host reads only the counts, after batches of steps: at least
        ceil(remaining / (K + 1)) more steps are needed (remaining counted for
        the sequence that is furthest behind), so that many run back to back
        before the next read.  ``record`` receives each step's accept length
        (a list per sequence when B > 1)."""
        B = self.B
        plen = np.asarray(prompt).reshape(B, -1).shape[1]
        check_generation(plen, n_new, self.K, B, self.max_ctx)
        self.prefill(prompt)
        if graph and getattr(self, "graph", None) is None:
            self.capture()
        if self.fused:
            cap = (self.log.shape[1] - 2) // 2
            if n_new + self.K + 1 > cap:
                raise ValueError(f"n_new={n_new} exceeds the decode log ({cap} tokens)")
            done = 0
            while done < n_new:
                for _ in range(max(1, -(-(n_new - done) // (self.K + 1)))):
                    self.step_graph() if graph else self.step()
                done = int(self.log[:, 0].min().item())
            lg = self.log.cpu().numpy()
            if record is not None:
                recs = [[int(a) for a in lg[b, 2 + cap:2 + cap + int(lg[b, 1])]] for b in range(B)]
                record.extend(recs[0] if B == 1 else recs)
            self.ctx_host += done
            out = lg[:, 2:2 + n_new].astype(np.int32)
            return out[0] if B == 1 else out
        outs = [[] for _ in range(B)]
        recs = [[] for _ in range(B)]
        while min(len(o) for o in outs) < n_new:
            acc, path, tokens = self.step_graph() if graph else self.step()
            a_h = acc.cpu().numpy()
            p_h = path.cpu().numpy()
            t_h = tokens.cpu().numpy()
            for b in range(B):
                a = int(a_h[b])
                outs[b].extend(int(t_h[b, j]) for j in p_h[b, :a + 1])
                recs[b].append(a)
            self.ctx_host += int(a_h[0]) + 1
        if record is not None:
            record.extend(recs[0] if B == 1 else recs)
        out = np.array([o[:n_new] for o in outs], np.int32)
        return out[0] if B == 1 else out
