"""Register budgets and tile-loop schedules of the gfx950 kernels, checked at
compile time on the CPU.

No kernel spills VGPRs to scratch memory: the attention kernels run two waves
per SIMD at up to 256 registers (the early-stopped instantiation within about
ten of it), so a source change can push one of them into spilling inside its
tile loop, which keeps the output correct but costs a multiple of the time.

The MFMA block of each step of the d = 128 attention kernels (the code between
the raised and the restored wave priority) waits for all of its LDS reads
(`s_waitcnt lgkmcnt(0)`) at most a few times: when register pressure or the
loop's control flow leads the compiler to keep one K or V fragment in flight,
it waits before every MFMA (about 30 times per block), which cost the
early-stopped kernel 6% before its loop was restructured.  The bound is a
property of this compiler's schedule, checked so that a change that brings the
serialization back fails here rather than only in a timing run.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_attention_amd import build as BLD

SOURCES = sorted(f for f in os.listdir(os.path.join(BLD.CSRC, "kernels")) if f.endswith(".hip"))


def kernel_resources(asm: str):
    """(symbol, VGPRs, spilled VGPRs) for every kernel in the metadata of a device assembly listing."""
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = []
    for entry in re.split(r"\n  - ", meta)[1:]:
        sym = re.search(r"\.symbol:\s+(\S+)", entry)
        vg = re.search(r"\.vgpr_count:\s+(\d+)", entry)
        sp = re.search(r"\.vgpr_spill_count:\s+(\d+)", entry)
        if sym and vg and sp:
            out.append((sym.group(1), int(vg.group(1)), int(sp.group(1))))
    return out


def mfma_block_lds_waits(asm: str, symbol: str):
    """Full LDS waits in each MFMA block (s_setprio 1 .. s_setprio 0) of one kernel's code."""
    lines = asm.split("\n")
    start = next(i for i, line in enumerate(lines) if line.startswith(symbol + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].strip().startswith(".Lfunc_end"))
    counts, cur = [], None
    for line in lines[start:end]:
        if "s_setprio 1" in line:
            cur = 0
        elif cur is not None and "lgkmcnt(0)" in line:
            cur += 1
        if "s_setprio 0" in line and cur is not None:
            counts.append(cur)
            cur = None
    return counts


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    """Device assembly of every kernel source, compiled with the library's flags."""
    if not os.path.exists(BLD.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("no hipcc")
    tmp = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        out = tmp / (src + ".s")
        flags = [f for f in BLD.FLAGS if f != "-fPIC"]
        subprocess.run([BLD.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                        os.path.join(BLD.CSRC, "kernels", src)], check=True, capture_output=True)
        return src, out.read_text()

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        return dict(ex.map(compile_one, SOURCES))


def test_no_kernel_spills_vgprs(listings):
    kernels = [(src, sym, vg, sp) for src, asm in listings.items() for sym, vg, sp in kernel_resources(asm)]
    assert len(kernels) > 50                      # every instantiation was found in the metadata
    spilled = [(src, sym, vg, sp) for src, sym, vg, sp in kernels if sp]
    assert not spilled, spilled
    prefill = [k for k in kernels if "prefill_mfma_kernel" in k[1]]
    assert prefill and all(vg <= 256 for _, _, vg, _ in prefill)   # two waves per SIMD


def test_attention_mfma_blocks_keep_lds_reads_in_flight(listings):
    asm = listings["prefill.hip"]
    syms = [sym[:-3] if sym.endswith(".kd") else sym for sym, _, _ in kernel_resources(asm)
            if "prefill_mfma_kernel" in sym and "ILi128E" in sym]
    assert len(syms) >= 6                          # top-p, permuted, early-stopped; LDS and HBM lists
    for sym in syms:
        waits = mfma_block_lds_waits(asm, sym)
        assert len(waits) >= 3, (sym, waits)       # prologue tile and the two steps of the unrolled loop
        assert max(waits) <= 16, (sym, waits)      # serialized fragment reads wait about 30 times
