"""The C ABI's host layer (argument validation, workspace sizing, dispatch
up to the launch) under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is rebuilt with the host pass instrumented and the CPU boundary
tests run against it in a child process with the clang sanitizer runtime
preloaded.  Any sanitizer report fails the run.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not available")
def test_boundary_under_host_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("clang sanitizer runtime not found")
    from block_sparse_attention_amd import build as Bd
    lib = Bd.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, SPOT_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_boundary_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
