"""Helpers for the GPU parity tests (device transfer, tolerances, case logging)."""
import sys

import numpy as np
import torch

# Tolerances (max-abs), per the method's precision contract: bf16 storage with
# fp32 accumulation, or fp32 throughout.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def case(name):
    """Print and flush the case name before GPU work, so a failing run names it."""
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def dev(a, dtype=torch.float32):
    """numpy -> GPU tensor (float arrays cast to ``dtype``; ints kept)."""
    a = np.ascontiguousarray(a)
    if a.dtype.kind == "f":
        return torch.tensor(a.astype(np.float32)).to(device="cuda", dtype=dtype)
    if a.dtype == np.uint64:
        return torch.tensor(a.view(np.int64)).cuda()
    return torch.tensor(a).cuda()


def host(t):
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.cpu().numpy()


def assert_close(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    return err


def assert_close_stored(got, ref, tol, what="", dt=torch.bfloat16):
    """For outputs stored in the model dtype ``dt``.  bf16: the bound is
    ``tol`` absolute up to |ref| = 1 and relative beyond (bf16 storage alone
    rounds by up to 2^-8 |y|, well inside 2e-2 |y|).  fp32: the flat max-abs
    bound, as for any fp32 output."""
    if dt == torch.float32:
        return assert_close(got, ref, tol, what)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(1.0, np.abs(ref))
    return assert_close(np.asarray(got, np.float64) / scale, ref / scale, tol, what)
