"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer run of the C ABI.

A copy of libmedusa.so is built with both sanitizers on its host code (the
argument checks, workspace queries, launch planning and the host-only tree
code; the kernels are compiled as usual but never launched), and
tests/host_abi_check.c, built with the same sanitizers, drives it: status
strings, the tree-template check on valid and malformed templates, the
accuracy-driven sparse tree over a sweep of sizes, every workspace query at
ordinary, zero, negative and extreme sizes, and the rejection of bad
arguments by every device entry point.  Any sanitizer report aborts the
program; any wrong status code makes it exit 1.  No GPU is touched."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def b_hipcc():
    from speculative_decoding_02_amd import build as b
    return b.HIPCC


@pytest.mark.skipif(not (os.path.exists(CLANG) and os.path.exists(b_hipcc())),
                    reason="needs the ROCm toolchain")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from speculative_decoding_02_amd import build as b
    lib = b.build_host_sanitized(str(tmp_path / "obj"), str(tmp_path / "libmedusa_san.so"))
    exe = str(tmp_path / "host_abi_check")
    cc = subprocess.run([CLANG, "-g", "-O1", "-fsanitize=address,undefined",
                         "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                         os.path.join(ROOT, "tests", "host_abi_check.c"), "-o", exe,
                         "-L", str(tmp_path), "-lmedusa_san", f"-Wl,-rpath,{tmp_path}", "-lm"],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    assert os.path.exists(lib)
    env = dict(os.environ)
    # the HIP runtime keeps its allocations until exit; the order check would
    # trip on any library preloaded ahead of the sanitizer runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
