"""Thin Python binding of libmedusa (the C ABI in include/medusa.h).

Argument marshalling only: every function takes torch tensors that live in
GPU memory, checks dtype / shape / contiguity, passes raw pointers and the
current HIP stream to the library, and raises ``MedusaError`` on a non-zero
status.  No step of the decode path is computed here; torch provides device
memory and streams.  The library must be built (``__graft_entry__.build()``);
importing this module without it raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MEDUSA_LIB", os.path.join(_HERE, "libmedusa.so"))

F32, BF16 = 0, 1
EPI_NONE, EPI_BIAS_SILU_RES, EPI_RES_ADD_F32, EPI_SWIGLU = 0, 1, 2, 3
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_SIGS = {
    "medusa_status_string": (C.c_char_p, [i32]),
    "medusa_last_error": (C.c_char_p, []),
    "medusa_abi_version": (i32, []),
    "medusa_tree_validate": (i32, [vp, vp, i32, i32, i32]),
    "medusa_linear_ws": (sz, [i64, i64, i64, i32, i32]),
    "medusa_linear": (i32, [vp, i64, i64, i64, vp, i64, i32, i32, i32, vp, vp, vp, i32, vp, sz,
                            vp]),
    "medusa_heads_ws": (sz, [i64, i64, i32, i64, i32, i32]),
    "medusa_heads": (i32, [vp, i64, i64, i32, vp, vp, vp, i64, i32, vp, i32, vp, vp, vp, sz, vp]),
    "medusa_topk_ws": (sz, [i64, i64, i32]),
    "medusa_topk_lists": (i32, [i64]),
    "medusa_heads_lists": (i32, [vp, i64, i64, i32, vp, vp, vp, i64, i32, i32, vp, vp, vp, sz, vp]),
    "medusa_topk": (i32, [vp, i64, i64, i32, vp, vp, vp, sz, vp]),
    "medusa_build_tree": (i32, [i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]),
    "medusa_tree_attention_ws": (sz, [i32, i32, i32, i32, i32, i32, i32]),
    "medusa_tree_attention_splits": (i32, [i32, i32, i32, i32, i32, i32, i32, i32]),
    "medusa_tree_attention": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, i32, i32, i32,
                                    i32, i32, f32, i32, vp, vp, sz, vp]),
    "medusa_tree_attention_noalloc": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, i32,
                                            i32, i32, i32, i32, f32, i32, vp, vp]),
    "medusa_accept_ws": (sz, [i32, i32]),
    "medusa_accept": (i32, [vp, i64, vp, vp, i32, i32, i32, i32, f32, f32, f32, vp, vp, vp, vp,
                            sz, vp]),
    "medusa_accept_sample": (i32, [vp, i64, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz,
                                   vp]),
    "medusa_tree_from_accuracy": (i32, [vp, i32, i32, i32, vp, vp, vp]),
    "kv_compact": (i32, [C.POINTER(vp), C.POINTER(vp), i32, vp, i32, i32, vp, vp, vp, i32, i32,
                         i32, i32, i32, vp, vp, vp, vp]),
    "medusa_embed": (i32, [vp, i64, vp, i64, i64, i32, vp, vp]),
    "medusa_rmsnorm": (i32, [vp, i64, i64, vp, f32, i32, vp, vp]),
    "medusa_linear_rmsnorm": (i32, [vp, i64, i64, vp, i64, i32, vp, vp, f32, vp, vp, sz, vp]),
    "medusa_linear_qkv_rope_ws": (sz, [i64, i64, i32, i32, i32, i32]),
    "medusa_linear_qkv_rope": (i32, [vp, i64, i64, vp, i32, i32, i32, vp, f32, i32, vp, vp, vp, vp,
                                     sz, vp]),
    "medusa_qkv_rope": (i32, [vp, i64, i32, i32, i32, vp, f32, i32, vp, vp, vp, vp]),
    "medusa_swiglu": (i32, [vp, i64, i64, i32, vp, vp]),
    "medusa_gather_rows": (i32, [vp, i32, i32, i64, vp, vp, i32, i32, vp, vp]),
    "medusa_tree_embed": (i32, [i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp,
                                i64, i64, i32, vp, f32, vp, vp, vp]),
    "medusa_decode_tail_ws": (sz, [i32, i32]),
    "medusa_decode_tail": (i32, [vp, i64, vp, vp, i32, i32, i32, i32, f32, f32, f32, vp,
                                 C.POINTER(vp), C.POINTER(vp), i32, vp, i32, i32, i32, i32, i32,
                                 vp, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]),
}
EXPORTS = tuple(_SIGS)


class MedusaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


def load_library(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"libmedusa.so not found at {path}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = load_library()


def raw():
    """The loaded ctypes library (for the ABI tests)."""
    return _lib


def _check(fn, status):
    if status != 0:
        raise MedusaError(fn, status, _lib.medusa_last_error().decode())


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _ws(nbytes, device):
    """A zero-filled workspace (the projection's arrival counters must start
    at zero; the library leaves them zero)."""
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("workspace allocation during graph capture: preallocate it")
    nbytes = max(int(nbytes), 256)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
def medusa_tree_from_accuracy(accuracy, N):
    """Sparse tree of the N most accurate combinations (host): accuracy [K, topk]
    -> (parent int32[N], rank int32[N], expected accepted candidates)."""
    import numpy as np
    acc = np.ascontiguousarray(np.asarray(accuracy, dtype=np.float32))
    K, topk = acc.shape
    parent = np.zeros(N, np.int32)
    rank = np.zeros(N, np.int32)
    expected = C.c_double(0.0)
    _check("medusa_tree_from_accuracy", _lib.medusa_tree_from_accuracy(
        acc.ctypes.data, K, topk, N, parent.ctypes.data, rank.ctypes.data, C.byref(expected)))
    return parent, rank, expected.value


def medusa_tree_validate(parent, rank, K, topk):
    """Host-side check of a tree template (numpy/int32 or torch CPU arrays)."""
    import numpy as np
    p = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    r = np.ascontiguousarray(np.asarray(rank, dtype=np.int32))
    _check("medusa_tree_validate", _lib.medusa_tree_validate(
        p.ctypes.data, r.ctypes.data, len(p), int(K), int(topk)))


def linear_ws_bytes(M, Kd, N, batch, dt):
    return _lib.medusa_linear_ws(M, Kd, N, batch, dt)


def qkv_rope_ws_bytes(M, Kd, Hq, Hkv, D, dt):
    return _lib.medusa_linear_qkv_rope_ws(M, Kd, Hq, Hkv, D, dt)


def medusa_linear(X, W, epilogue=EPI_NONE, bias=None, aux=None, out=None, y_f32=False,
                  x_bstride=0, ws=None):
    """Y = epilogue(X W^T).  W [batch, N, Kd] or [N, Kd]; X [M, Kd] or [batch, M, Kd]."""
    dt = _dt(W)
    batch = W.shape[0] if W.dim() == 3 else 1
    N, Kd = W.shape[-2], W.shape[-1]
    M = X.shape[-2]
    if X.dim() == 3 and x_bstride == 0:
        x_bstride = M * Kd
    if out is None:
        cols = N // 2 if epilogue == EPI_SWIGLU else N
        ydt = torch.float32 if (y_f32 or epilogue == EPI_RES_ADD_F32) else W.dtype
        shape = (batch, M, cols) if batch > 1 or W.dim() == 3 else (M, cols)
        out = torch.empty(shape, dtype=ydt, device=W.device)
    need = _lib.medusa_linear_ws(M, Kd, N, batch, dt)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, W.device)
    _check("medusa_linear", _lib.medusa_linear(
        _p(X), x_bstride, M, Kd, _p(W), N, batch, dt, epilogue, _p(bias), _p(aux), _p(out),
        int(bool(y_f32)), _p(ws) if need else None, ws.numel() if need else 0, _stream()))
    return out


def medusa_heads(X, W1, b1, W2, topk=0, logits=None, ids=None, vals=None, ws=None,
                 want_logits=True):
    """Logits [K, M, V] (float) and per-head top-k of the Medusa heads on X [M, H].

    With ``want_logits=False`` and no ``logits`` buffer the logits stay in the
    workspace and only the top-k is returned."""
    dt = _dt(X)
    K, H = W1.shape[0], W1.shape[1]
    V = W2.shape[1]
    M = X.shape[0]
    dev = X.device
    if logits is None and want_logits:
        logits = torch.empty((K, M, V), dtype=torch.float32, device=dev)
    if ids is None:
        ids = torch.empty((K, M, max(topk, 1)), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((K, M, max(topk, 1)), dtype=torch.float32, device=dev)
    need = _lib.medusa_heads_ws(M, H, K, V, topk, dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check("medusa_heads", _lib.medusa_heads(
        _p(X), M, H, K, _p(W1), _p(b1), _p(W2), V, dt, _p(logits), topk,
        _p(ids) if topk else None, _p(vals) if topk else None, _p(ws), ws.numel(), _stream()))
    return logits, ids[..., :topk], vals[..., :topk]


def medusa_heads_lists(X, W1, b1, W2, topk, ids=None, vals=None, ws=None):
    """Per-chunk top-k lists of the K heads' logits on X [M, H]: ids [K, M, S,
    topk] int32 and vals [K, M, S, topk] float, S = medusa_topk_lists(V)."""
    dt = _dt(X)
    K, H = W1.shape[0], W1.shape[1]
    V = W2.shape[1]
    M = X.shape[0]
    S = _lib.medusa_topk_lists(V)
    dev = X.device
    if ids is None:
        ids = torch.empty((K, M, S, topk), dtype=torch.int32, device=dev)
    if vals is None:
        vals = torch.empty((K, M, S, topk), dtype=torch.float32, device=dev)
    if tuple(ids.shape) != (K, M, S, topk) or tuple(vals.shape) != (K, M, S, topk):
        raise ValueError(f"lists must be [K, M, S, topk] = {(K, M, S, topk)}")
    need = _lib.medusa_heads_ws(M, H, K, V, topk, dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check("medusa_heads_lists", _lib.medusa_heads_lists(
        _p(X), M, H, K, _p(W1), _p(b1), _p(W2), V, dt, topk, _p(ids), _p(vals), _p(ws),
        ws.numel(), _stream()))
    return ids, vals


def medusa_topk(logits, k, ids=None, vals=None, ws=None):
    R, V = logits[..., 0].numel(), logits.shape[-1]
    dev = logits.device
    ids = ids if ids is not None else torch.empty(logits.shape[:-1] + (k,), dtype=torch.int32, device=dev)
    vals = vals if vals is not None else torch.empty(logits.shape[:-1] + (k,), dtype=torch.float32, device=dev)
    need = _lib.medusa_topk_ws(R, V, k)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, dev)
    _check("medusa_topk", _lib.medusa_topk(_p(logits), R, V, k, _p(ids), _p(vals),
                                           _p(ws) if need else None, ws.numel() if need else 0,
                                           _stream()))
    return ids, vals


def medusa_build_tree(parent, rank, root_tok, topk_ids, ctx, tokens=None, pos=None, mask=None):
    """parent, rank [B, N]; root_tok [B]; topk_ids [K, B, topk]; ctx [B] (all int32, GPU)."""
    B, N = parent.shape
    K, topk = topk_ids.shape[0], topk_ids.shape[-1]
    dev = parent.device
    tokens = tokens if tokens is not None else torch.empty((B, N), dtype=torch.int32, device=dev)
    pos = pos if pos is not None else torch.empty((B, N), dtype=torch.int32, device=dev)
    mask = mask if mask is not None else torch.empty((B, N), dtype=torch.int64, device=dev)
    _check("medusa_build_tree", _lib.medusa_build_tree(
        B, N, _p(parent), _p(rank), _p(root_tok), _p(topk_ids), K, topk, _p(ctx), _p(tokens),
        _p(pos), _p(mask), _stream()))
    return tokens, pos, mask


def tree_attention_ws_bytes(B, N, Hq, Hkv, D, max_ctx, P=16):
    return _lib.medusa_tree_attention_ws(B, N, Hq, Hkv, D, max_ctx, P)


def tree_attention_splits(B, N, Hq, Hkv, D, max_ctx, P=16, bf16=True):
    """The plan medusa_tree_attention takes for these shapes: 0 = one launch
    without key splits, S >= 1 = S key splits (+ a merge launch if S > 1)."""
    return _lib.medusa_tree_attention_splits(B, N, Hq, Hkv, D, int(max_ctx), P,
                                             BF16 if bf16 else F32)


def medusa_tree_attention(Q, Kt, Vt, Kc, Vc, page_table, ctx, max_ctx, mask, scale, out=None,
                          ws=None):
    """Q [B,N,Hq,D]; Kt,Vt [B,N,Hkv,D]; Kc,Vc [pages,Hkv,P,D]; page_table [B,max_pages];
    ctx [B]; mask [B,N] (int64 bit patterns).  ws must be zero-filled at first use."""
    dt = _dt(Q)
    B, N, Hq, D = Q.shape
    Hkv, P = Kc.shape[1], Kc.shape[2]
    out = out if out is not None else torch.empty_like(Q)
    need = _lib.medusa_tree_attention_ws(B, N, Hq, Hkv, D, int(max_ctx), P)
    if ws is None or ws.numel() < need:
        ws = _ws(need, Q.device)
    _check("medusa_tree_attention", _lib.medusa_tree_attention(
        _p(Q), _p(Kt), _p(Vt), _p(Kc), _p(Vc), _p(page_table), page_table.shape[1], P, _p(ctx),
        int(max_ctx), _p(mask), B, N, Hq, Hkv, D, float(scale), dt, _p(out), _p(ws), ws.numel(),
        _stream()))
    return out


NOALLOC_MAX_BYTES = 32 << 20  # MEDUSA_ATTN_NOALLOC_MAX_BYTES


def medusa_tree_attention_noalloc(Q, Kt, Vt, Kc, Vc, page_table, ctx, max_ctx, mask, scale,
                                  out):
    """medusa_tree_attention without a workspace: the library's fixed per-GPU
    array holds the split partials (calls on one GPU must not overlap).  The
    caller passes the output buffer; nothing is allocated."""
    dt = _dt(Q)
    B, N, Hq, D = Q.shape
    Hkv, P = Kc.shape[1], Kc.shape[2]
    _check("medusa_tree_attention_noalloc", _lib.medusa_tree_attention_noalloc(
        _p(Q), _p(Kt), _p(Vt), _p(Kc), _p(Vc), _p(page_table), page_table.shape[1], P, _p(ctx),
        int(max_ctx), _p(mask), B, N, Hq, Hkv, D, float(scale), dt, _p(out), _stream()))
    return out


def medusa_accept(logits, tokens, parent, K, mode=0, temperature=1.0, epsilon=0.3, delta=0.09,
                  out=None, ws=None):
    """logits [B,N,V] float; tokens, parent [B,N] int32 -> (accept_len [B], path [B,K+1], next [B])."""
    B, N, V = logits.shape
    dev = logits.device
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    need = _lib.medusa_accept_ws(B, N)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    acc, path, nxt = out
    _check("medusa_accept", _lib.medusa_accept(
        _p(logits), V, _p(tokens), _p(parent), B, N, K, int(mode), float(temperature),
        float(epsilon), float(delta), _p(acc), _p(path), _p(nxt), _p(ws), ws.numel(), _stream()))
    return acc, path, nxt


def rng_state(seed, step=0, device="cuda"):
    """Device (seed, step) pair for medusa_accept_sample (uint64 bit patterns)."""
    import numpy as np
    return torch.from_numpy(np.array([seed, step], dtype=np.uint64).view(np.int64)).to(device)


def medusa_accept_sample(logits, tokens, parent, K, temperature, rng, out=None, ws=None):
    """Sampled verification.  logits [B,N,V] float; tokens, parent [B,N] int32;
    rng: 2-element int64 device tensor (seed, step) holding uint64 bit patterns,
    advanced by one on the device -> (accept_len [B], path [B,K+1], next [B])."""
    B, N, V = logits.shape
    dev = logits.device
    if rng.numel() != 2 or rng.dtype != torch.int64:
        raise ValueError("rng must be a 2-element int64 tensor (seed, step)")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    need = _lib.medusa_accept_ws(B, N)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    acc, path, nxt = out
    _check("medusa_accept_sample", _lib.medusa_accept_sample(
        _p(logits), V, _p(tokens), _p(parent), B, N, K, float(temperature), _p(rng), _p(acc),
        _p(path), _p(nxt), _p(ws), ws.numel(), _stream()))
    return acc, path, nxt


def kv_compact(Kc_list, Vc_list, page_table, ctx, path, accept_len, new_ctx=None, src=None, dst=None):
    """Kc_list / Vc_list: one [pages,Hkv,P,D] pool per layer."""
    L = len(Kc_list)
    B, K1 = path.shape
    Hkv, P, D = Kc_list[0].shape[1], Kc_list[0].shape[2], Kc_list[0].shape[3]
    dev = path.device
    new_ctx = new_ctx if new_ctx is not None else torch.empty(B, dtype=torch.int32, device=dev)
    src = src if src is not None else torch.empty((B, K1), dtype=torch.int32, device=dev)
    dst = dst if dst is not None else torch.empty((B, K1), dtype=torch.int32, device=dev)
    karr = (vp * L)(*[_p(t) for t in Kc_list])
    varr = (vp * L)(*[_p(t) for t in Vc_list])
    _check("kv_compact", _lib.kv_compact(
        karr, varr, L, _p(page_table), page_table.shape[1], P, _p(ctx), _p(path), _p(accept_len),
        B, K1 - 1, Hkv, D, _dt(Kc_list[0]), _p(src), _p(dst), _p(new_ctx), _stream()))
    return new_ctx, src, dst


def medusa_embed(tokens, table, out=None):
    M = tokens.numel()
    V, H = table.shape
    out = out if out is not None else torch.empty((M, H), dtype=torch.float32, device=table.device)
    _check("medusa_embed", _lib.medusa_embed(_p(tokens), M, _p(table), V, H, _dt(table), _p(out), _stream()))
    return out


def medusa_rmsnorm(x, gain, eps, dtype, out=None):
    M, H = x.shape
    out = out if out is not None else torch.empty((M, H), dtype=dtype, device=x.device)
    _check("medusa_rmsnorm", _lib.medusa_rmsnorm(_p(x), M, H, _p(gain), float(eps), _dt(out),
                                                 _p(out), _stream()))
    return out


def medusa_linear_rmsnorm(X, W, x, gain, eps, out=None, ws=None):
    """x += X W^T (x float [M, N], in place); returns RMSNorm(x) * gain in W's dtype."""
    dt = _dt(W)
    N, Kd = W.shape
    M = X.shape[0]
    out = out if out is not None else torch.empty((M, N), dtype=W.dtype, device=W.device)
    need = _lib.medusa_linear_ws(M, Kd, N, 1, dt)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, W.device)
    _check("medusa_linear_rmsnorm", _lib.medusa_linear_rmsnorm(
        _p(X), M, Kd, _p(W), N, dt, _p(x), _p(gain), float(eps), _p(out),
        _p(ws) if need else None, ws.numel() if need else 0, _stream()))
    return out


def interleave_rope_pairs(w, heads, D):
    """Rows of ``heads`` heads of D -> pair-interleaved: row 2j of a head takes
    row j, row 2j+1 takes row j + D/2 (numpy or torch, [heads*D, ...])."""
    lead = w.shape[1:]
    x = w.reshape(heads, 2, D // 2, *lead)
    if isinstance(w, np.ndarray):
        return np.swapaxes(x, 1, 2).reshape(heads * D, *lead)
    return x.transpose(1, 2).reshape(heads * D, *lead).contiguous()


def medusa_linear_qkv_rope(X, W, Hq, Hkv, D, pos, base, q=None, k=None, v=None, ws=None):
    """q, k, v of the pair-interleaved QKV weight W (see interleave_rope_pairs), rotated."""
    M, Kd = X.shape
    dev, dt = X.device, W.dtype
    q = q if q is not None else torch.empty((M, Hq, D), dtype=dt, device=dev)
    k = k if k is not None else torch.empty((M, Hkv, D), dtype=dt, device=dev)
    v = v if v is not None else torch.empty((M, Hkv, D), dtype=dt, device=dev)
    need = _lib.medusa_linear_qkv_rope_ws(M, Kd, Hq, Hkv, D, _dt(W))
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, dev)
    _check("medusa_linear_qkv_rope", _lib.medusa_linear_qkv_rope(
        _p(X), M, Kd, _p(W), Hq, Hkv, D, _p(pos), float(base), _dt(W), _p(q), _p(k), _p(v),
        _p(ws) if need else None, ws.numel() if need else 0, _stream()))
    return q, k, v


def medusa_qkv_rope(qkv, Hq, Hkv, D, pos, base, q=None, k=None, v=None):
    M = qkv.shape[0]
    dev, dt = qkv.device, qkv.dtype
    q = q if q is not None else torch.empty((M, Hq, D), dtype=dt, device=dev)
    k = k if k is not None else torch.empty((M, Hkv, D), dtype=dt, device=dev)
    v = v if v is not None else torch.empty((M, Hkv, D), dtype=dt, device=dev)
    _check("medusa_qkv_rope", _lib.medusa_qkv_rope(_p(qkv), M, Hq, Hkv, D, _p(pos), float(base),
                                                   _dt(qkv), _p(q), _p(k), _p(v), _stream()))
    return q, k, v


def medusa_swiglu(gu, out=None):
    M, F2 = gu.shape
    out = out if out is not None else torch.empty((M, F2 // 2), dtype=gu.dtype, device=gu.device)
    _check("medusa_swiglu", _lib.medusa_swiglu(_p(gu), M, F2 // 2, _dt(gu), _p(out), _stream()))
    return out


def medusa_gather_rows(h, path, accept_len, out=None):
    """h [B, N, H] -> out [B, H] = h[b, path[b, accept_len[b]]]."""
    B, N, H = h.shape
    out = out if out is not None else torch.empty((B, H), dtype=h.dtype, device=h.device)
    _check("medusa_gather_rows", _lib.medusa_gather_rows(
        _p(h), B, N, H, _p(path), _p(accept_len), path.shape[1] - 1, _dt(h), _p(out), _stream()))
    return out


def decode_log(B, cap, device="cuda"):
    """A zeroed decode log for medusa_decode_tail: [B, 2 + 2*cap] int32."""
    return torch.zeros((B, 2 + 2 * cap), dtype=torch.int32, device=device)


def medusa_decode_tail(logits, tokens, parent, K, mode, Kc_list, Vc_list, page_table, hidden,
                       ctx, root, log, temperature=1.0, epsilon=0.3, delta=0.09, rng=None,
                       h_best=None, out=None, ws=None):
    """The decode step's tail: accept (mode 0 greedy, 1 typical, 2 sampled),
    compact every layer's cache, gather the kept hidden row, set root, advance
    ctx and append to the decode log.  Returns (accept_len, path, next, h_best).

    ws must be zero-filled when first allocated (the call leaves its counters
    zero); the default allocates one per call."""
    B, N, V = logits.shape
    H = hidden.shape[-1]
    dev = logits.device
    L = len(Kc_list)
    Hkv, P, D = Kc_list[0].shape[1], Kc_list[0].shape[2], Kc_list[0].shape[3]
    if mode == 2 and (rng is None or rng.numel() != 2 or rng.dtype != torch.int64):
        raise ValueError("sampled mode needs rng: a 2-element int64 tensor (seed, step)")
    if out is None:
        out = (torch.empty(B, dtype=torch.int32, device=dev),
               torch.empty((B, K + 1), dtype=torch.int32, device=dev),
               torch.empty(B, dtype=torch.int32, device=dev))
    h_best = h_best if h_best is not None else torch.empty((B, H), dtype=hidden.dtype, device=dev)
    need = _lib.medusa_decode_tail_ws(B, N)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    acc, path, nxt = out
    karr = (vp * L)(*[_p(t) for t in Kc_list])
    varr = (vp * L)(*[_p(t) for t in Vc_list])
    cap = (log.shape[1] - 2) // 2
    _check("medusa_decode_tail", _lib.medusa_decode_tail(
        _p(logits), V, _p(tokens), _p(parent), B, N, K, int(mode), float(temperature),
        float(epsilon), float(delta), _p(rng) if mode == 2 else None, karr, varr, L,
        _p(page_table), page_table.shape[1], P, Hkv, D, _dt(Kc_list[0]), _p(hidden), H,
        _p(h_best), _p(ctx), _p(root), _p(acc), _p(path), _p(nxt), _p(log), cap, _p(ws),
        ws.numel(), _stream()))
    return acc, path, nxt, h_best


def medusa_tree_embed(parent, rank, root_tok, topk_ids, ctx, table, gain, eps, out=None,
                      topk_vals=None):
    """medusa_build_tree + medusa_embed + medusa_rmsnorm in one launch.
    ``topk_ids`` [K, B, topk] (the heads' top-k), or per-chunk lists
    [K, B, S, topk] with their ``topk_vals`` (medusa_heads_lists), merged in
    the launch.
    Returns (tokens [B,N], pos [B,N], mask [B,N] int64, x [B*N,H] float, h [B*N,H])."""
    B, N = parent.shape
    if topk_ids.dim() == 4:
        K, _, lists, topk = topk_ids.shape
    else:
        (K, _, topk), lists = topk_ids.shape, 1
    V, H = table.shape
    dev = parent.device
    if out is None:
        out = (torch.empty((B, N), dtype=torch.int32, device=dev),
               torch.empty((B, N), dtype=torch.int32, device=dev),
               torch.empty((B, N), dtype=torch.int64, device=dev),
               torch.empty((B * N, H), dtype=torch.float32, device=dev),
               torch.empty((B * N, H), dtype=table.dtype, device=dev))
    tokens, pos, mask, x, h = out
    _check("medusa_tree_embed", _lib.medusa_tree_embed(
        B, N, _p(parent), _p(rank), _p(root_tok), _p(topk_ids), _p(topk_vals), lists, K, topk,
        _p(ctx), _p(tokens),
        _p(pos), _p(mask), _p(table), V, H, _dt(table), _p(gain), float(eps), _p(x), _p(h),
        _stream()))
    return out
