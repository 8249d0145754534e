"""The CPU ABI tests again, against the library whose host code (argument
checks, workspace layout arithmetic over multi-GB workspaces, launch
sequence) is built with AddressSanitizer and UBSan (libslr_hostsan.so, made
by the package build): any out-of-bounds access, overflow or other undefined
behaviour in that code aborts the run. No GPU is needed: every call the ABI
tests make is rejected, or sized, on the host."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "sparse_rank_attention_rope3d_amd", "libslr_hostsan.so")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists(SAN_LIB), reason="libslr_hostsan.so not built")
def test_abi_checks_under_address_and_undefined_behaviour_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this image")
    env = dict(os.environ, SLR_LIB=SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest; from sparse_rank_attention_rope3d_amd import binding as B; "
            f"assert B.LIB_PATH == {SAN_LIB!r}, B.LIB_PATH; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
