"""Builds libspot.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m block_sparse_attention_amd.build [-v] [--sanitize]

--sanitize builds _build_san/libspot_san.so instead: the same sources with
the host code (the C ABI's validation, sizing and dispatch) instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer; device code is compiled as
usual (the sanitizers are passed to the host pass only).  It runs the CPU
boundary tests with the clang sanitizer runtime preloaded
(tests/test_boundary_sanitized.py).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspot.so")
OBJDIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources() -> list[str]:
    out = [os.path.join(CSRC, "spot_api.cpp")]
    kdir = os.path.join(CSRC, "kernels")
    out += sorted(os.path.join(kdir, f) for f in os.listdir(kdir) if f.endswith(".hip"))
    return out


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose and res.stderr.strip():
        # the host pass does not know the packed-fp32 feature flag; that note is harmless
        lines = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


SAN_DIR = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_DIR, "libspot_san.so")


def host_sanitizer_flags() -> list[str]:
    """Host-pass-only sanitizer options (each one behind -Xarch_host)."""
    out = []
    for opt in ("-fsanitize=" + kind for kind in ("address", "undefined")):
        out += ["-Xarch_host", opt]
    return out + ["-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link libspot.so (or the host-sanitizer build); returns the library path."""
    objdir, lib = (SAN_DIR, SAN_LIB) if sanitize else (OBJDIR, LIB)
    flags = FLAGS + (host_sanitizer_flags() + ["-g"] if sanitize else [])
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    jobs = jobs or min(8, os.cpu_count() or 1)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *flags, "-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
    tmp = lib + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + (host_sanitizer_flags() if sanitize else [])
    _run(link + [*objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
