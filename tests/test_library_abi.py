"""The C-ABI library on the host (no GPU): it loads, it exports every entry
point include/medusa.h declares, the Python binding's signature table names
exactly those, host-side validation rejects bad arguments before touching a
device, and the workspace queries follow the launch planner.  Also the
weight-layout helpers the fused projections rely on."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "medusa.h")
LIB = os.path.join(ROOT, "speculative_decoding_02_amd", "libmedusa.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    ret = r"(?:size_t|int32_t|void|const\s+char\s*\*)"
    return sorted(set(re.findall(r"^\s*" + ret + r"\s*(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def M():
    if not os.path.exists(LIB):  # a fresh checkout: build it (hipcc cross-compiles here)
        from speculative_decoding_02_amd import build as b
        b.build(verbose=False)
    from speculative_decoding_02_amd import medusa
    return medusa


def test_header_declares_the_entry_points():
    names = _declared()
    assert len(names) >= 20, names
    for must in ("medusa_linear", "medusa_tree_attention", "medusa_accept", "kv_compact",
                 "medusa_heads", "medusa_build_tree", "medusa_linear_rmsnorm",
                 "medusa_linear_qkv_rope"):
        assert must in names


def test_library_exports_every_declared_symbol(M):
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert missing == []


def test_binding_table_is_the_header(M):
    assert sorted(M.EXPORTS) == _declared()


def test_bad_arguments_are_rejected_on_the_host(M):
    lib = M._lib
    # unknown dtype, unknown epilogue, head dim outside the limits: status
    # codes from argument checks that run before any device call
    assert lib.medusa_linear(None, 0, 4, 8, None, 4, 1, 7, 0, None, None, None, 0, None, 0,
                             None) == 2
    assert lib.medusa_linear(None, 0, 4, 8, None, 4, 1, 1, 9, None, None, None, 0, None, 0,
                             None) == 1
    assert lib.medusa_linear_qkv_rope(None, 4, 64, None, 2, 2, 6, None, 10000.0, 1, None, None,
                                      None, None, 0, None) == 2
    assert lib.medusa_linear_rmsnorm(None, 4, 64, None, 10, 1, None, None, 1e-5, None, None, 0,
                                     None) == 2  # N not a multiple of 4
    assert lib.medusa_rmsnorm(None, 2, 64, None, -1.0, 1, None, None) == 1  # eps < 0
    # sampled acceptance: temperature must be positive; N outside [1, 64]
    assert lib.medusa_accept_sample(None, 100, None, None, 1, 9, 2, 0.0, None, None, None, None,
                                    None, 0, None) == 1
    assert lib.medusa_accept_sample(None, 100, None, None, 1, 65, 2, 1.0, None, None, None, None,
                                    None, 0, None) == 2
    assert lib.medusa_accept_sample(None, 100, None, None, 0, 9, 2, 1.0, None, None, None, None,
                                    None, 0, None) == 0  # empty batch
    # zero rows: nothing to do, success without pointers
    assert lib.medusa_linear(None, 0, 0, 8, None, 4, 1, 1, 0, None, None, None, 0, None, 0,
                             None) == 0
    # the fused decode tail: K above 8, unknown mode, sampled without a
    # positive temperature, head dim, hidden rows not whole 16-byte chunks,
    # an empty batch, and (with stand-in addresses that are never read) a
    # missing workspace
    vp = M.vp
    pools = (vp * 1)(256)

    def tail(K=5, mode=0, T=1.0, D=128, H=256, B=1, ws=None, nbytes=0, dt=1):
        a = 256
        return lib.medusa_decode_tail(a, 1000, a, a, B, 64, K, mode, T, 0.3, 0.09, a, pools, pools,
                                      1, a, 8, 16, 2, D, dt, a, H, a, a, a, a, a, a, a, 16, ws,
                                      nbytes, None)
    assert tail(K=9) == 2
    assert tail(mode=3) == 1
    assert tail(mode=2, T=0.0) == 1
    assert tail(D=96) == 2
    assert tail(H=4) == 1          # 8 bytes of bf16
    assert tail(B=0) == 0
    assert tail() == 3
    need = lib.medusa_decode_tail_ws(1, 64)
    assert need == lib.medusa_accept_ws(1, 64) + 256
    assert tail(ws=4096, nbytes=need - 1) == 3
    # the fused tree + embedding + norm: H not a multiple of 4, H above 8192,
    # N above 64, an empty batch
    emb = lambda B=1, N=9, H=256, lists=1: lib.medusa_tree_embed(
        B, N, None, None, None, None, None, lists, 2, 3, None, None, None, None, None, 100, H, 1,
        None, 1e-5, None, None, None)
    assert emb(H=250) == 2
    assert emb(H=8196) == 2
    assert emb(N=65) == 1
    assert emb(lists=0) == 1
    assert emb(lists=65) == 1
    assert emb(B=0) == 0
    # the per-chunk top-k list count: ceil(V / 4096)
    assert [lib.medusa_topk_lists(v) for v in (1, 4096, 4097, 32000, 0)] == [1, 1, 2, 8, 0]
    assert lib.medusa_heads_lists(None, 4, 256, 2, None, None, None, 1000, 1, 0, None, None, None,
                                  0, None) == 2  # topk below 1


def test_workspace_queries_follow_the_plan(M):
    lib, BF16 = M._lib, M.BF16
    # 64 rows: the 4096-wide projections split their contraction (fp32
    # partials: splits x M x N x 4 bytes), the wide ones do not
    assert lib.medusa_linear_ws(64, 4096, 4096, 1, BF16) == 2 * 64 * 4096 * 4
    assert lib.medusa_linear_ws(64, 11008, 4096, 1, BF16) == 4 * 64 * 4096 * 4
    assert lib.medusa_linear_ws(64, 4096, 22016, 1, BF16) == 0
    assert lib.medusa_linear_ws(64, 4096, 12288, 1, BF16) == 0
    # the fused QKV + rotary projection needs scratch only off the fused path
    assert lib.medusa_linear_qkv_rope_ws(64, 4096, 32, 32, 128, BF16) == 0
    assert lib.medusa_linear_qkv_rope_ws(1, 4096, 32, 32, 128, BF16) >= 12288 * 2
    # tree attention: partials for every split of the planned key range
    assert lib.medusa_tree_attention_ws(1, 64, 32, 32, 128, 2048, 16) > 0


def test_interleave_rope_pairs_definition(M):
    heads, D, K = 3, 8, 5
    w = np.arange(heads * D * K, dtype=np.float32).reshape(heads * D, K)
    p = M.interleave_rope_pairs(w, heads, D)
    for h in range(heads):
        for j in range(D // 2):
            np.testing.assert_array_equal(p[h * D + 2 * j], w[h * D + j])
            np.testing.assert_array_equal(p[h * D + 2 * j + 1], w[h * D + j + D // 2])
    import torch
    np.testing.assert_array_equal(M.interleave_rope_pairs(torch.tensor(w), heads, D).numpy(), p)


def test_attention_plans_reach_both_bf16_kernels(M):
    """The attention plan is a function of the shapes only: the one-launch
    kernel (plan 0) for bf16 calls of at most 256 (sequence, head, 16-node
    block) workgroups over at most 1024 planned keys (max_ctx + N), key
    splits otherwise and for fp32.  The parity cases
    of the GPU tests reach both bf16 kernels at both head dims and with
    power-of-two and other page sizes."""
    sp = M.tree_attention_splits
    assert sp(1, 64, 32, 32, 128, 928, 16) == 0               # one 7B sequence's decode step
    assert sp(1, 64, 32, 32, 128, 960, 16) == 0               # 1024 planned keys
    assert sp(1, 64, 32, 32, 128, 961, 16) > 0                # 1025
    assert sp(1, 64, 32, 32, 128, 2048, 16) > 0               # the 7B layer at 2048 cached keys
    assert sp(1, 64, 64, 8, 128, 900, 16) == 0                # exactly 256 workgroups
    assert sp(1, 64, 65, 65, 128, 900, 16) > 0                # 260
    assert sp(1, 65, 32, 32, 128, 100, 16) == -1              # N > 64: rejected
    assert sp(16, 64, 32, 32, 128, 1024, 16) > 0              # a 16-sequence batch
    assert sp(1, 64, 80, 80, 128, 1500, 16) > 0               # 320 workgroups
    assert sp(1, 64, 32, 32, 128, 2048, 16, bf16=False) > 0   # fp32
    assert sp(1, 64, 4, 4, 128, 4096 * 16, 16) > 0            # page table past the LDS window
    from tests.test_gpu_kernels import ATT_CASES
    import torch
    seen = set()
    for B, N, Hq, Hkv, D, ctx, P, _, dt in ATT_CASES:
        if dt != torch.bfloat16:
            continue
        plan = sp(B, N, Hq, Hkv, D, int(np.max(ctx)), P)
        assert plan >= 0
        seen.add((plan == 0, D, P & (P - 1) == 0))
    assert seen == {(z, D, p2) for z in (True, False) for D in (64, 128) for p2 in (True, False)}

