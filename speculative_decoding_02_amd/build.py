"""Build libmedusa.so (HIP, gfx950) in-tree.

    python -m speculative_decoding_02_amd.build          # or __graft_entry__.build()

Each ``csrc/*.hip`` file is compiled separately by hipcc (in parallel) into
``_build/`` and linked into ``speculative_decoding_02_amd/libmedusa.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmedusa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True, out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile every HIP source and link ``out`` (default libmedusa.so).

    ``defines`` (NAME=VALUE strings) override the kernels' tuning constants;
    the default build uses none."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


# Host-only build with AddressSanitizer and UndefinedBehaviorSanitizer on the
# host code (the argument checks, workspace queries and host-side tree
# code), for CPU checks of those paths; its kernels are built as usual.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(build_dir: str, out: str) -> str:
    """Compile every source host-only with the sanitizers into ``out``."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = ["-O1", "-g", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", *SANITIZE,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

    def one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized host build) failed for {src}:\n{r.stderr}")
        return obj
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    r = subprocess.run([HIPCC, *flags, "-shared", *objs, "-o", out], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (sanitized host build) failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    build()
