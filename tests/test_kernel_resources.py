"""Register budgets of the gfx950 kernels, checked at compile time on the CPU:
no kernel spills VGPRs to scratch memory.  The attention kernels run two
waves per SIMD at up to 256 registers (the early-stopped instantiation sits
at that limit), so a source change can push one of them into spilling inside
its tile loop, which keeps the output correct but costs a multiple of the
time; this test turns that into a failure."""
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


@pytest.mark.skipif(not os.path.exists(BLD.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_no_kernel_spills_vgprs(tmp_path):
    def compile_one(src):
        out = tmp_path / (src + ".s")
        flags = [f for f in BLD.FLAGS if f != "-fPIC"]
        subprocess.run([BLD.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                        os.path.join(BLD.CSRC, "kernels", src)], check=True, capture_output=True)
        return src, kernel_resources(out.read_text())

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        results = list(ex.map(compile_one, SOURCES))
    kernels = [(src, sym, vg, sp) for src, ks in results for sym, vg, sp in ks]
    assert len(kernels) > 50                      # every instantiation was found in the metadata
    spilled = [(src, sym, vg, sp) for src, sym, vg, sp in kernels if sp]
    assert not spilled, spilled
    prefill = [k for k in kernels if "prefill_mfma_kernel" in k[1]]
    assert prefill and all(vg <= 256 for _, _, vg, _ in prefill)   # two waves per SIMD
