"""The permuted gather path against the plain one ([PBS] §2 segmented
permutation, [S2O] §1 index-driven loading): with the identity permutation
every history row read through `perm` is the natural row, so block scores,
kept lists, outputs and LSE of the whole prefill pipeline, and the stop
points of the early-stopped attention, must be bit-identical to the call
without a permutation.  This pins the permuted instantiations of the kernels
(the row chosen when a tile is gathered, the permuted block means) to the
plain ones, which the oracle pins in turn."""
import numpy as np
import pytest
import torch

from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests.test_gpu_parity import log, upload_prefill

pytestmark = pytest.mark.gpu

CASES = [dict(L=5000, hq=8, hkv=2, d=128, block=128, segment=1024, top_p=0.9, heavy_hitters=True),
         dict(L=3001, hq=4, hkv=1, d=64, block=64, segment=512, top_p=0.8),
         dict(L=2048, hq=8, hkv=2, d=128, block=64, segment=2048 - 64 * 8, top_p=1.0),
         dict(L=700, hq=4, hkv=2, d=64, block=16, segment=128, top_p=0.9, dtype="f32")]


def identity_perm(cfg, device):
    perm = np.tile(np.arange(cfg.L, dtype=np.int32), (cfg.batch, cfg.hkv, 1))
    return torch.from_numpy(perm).to(device)


@pytest.mark.parametrize("kw", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_identity_permutation_is_the_plain_path(gpu, kw):
    cfg = I.small_prefill(name="perm-id", seed=47, **kw)
    _, (dq, dk, dv, _) = upload_prefill(cfg, gpu)
    perm = identity_perm(cfg, gpu)
    plain = B.prefill(dq, dk, dv, cfg.block, cfg.top_p)
    permuted = B.prefill(dq, dk, dv, cfg.block, cfg.top_p, perm=perm, segment=cfg.segment)
    torch.cuda.synchronize()
    assert torch.equal(plain.scores, permuted.scores)
    assert torch.equal(plain.cnt, permuted.cnt) and torch.equal(plain.idx, permuted.idx)
    assert torch.equal(plain.o, permuted.o)
    assert torch.equal(plain.lse, permuted.lse)
    log("identity permutation", kw, "kept blocks", int(plain.cnt.sum()), "bit-identical")


@pytest.mark.parametrize("kw", [c for c in CASES if c.get("dtype", "bf16") == "bf16" and c["block"] >= 64],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_identity_permutation_early_stop(gpu, kw):
    cfg = I.small_prefill(name="perm-id-es", seed=53, **kw)
    _, (dq, dk, dv, _) = upload_prefill(cfg, gpu)
    perm = identity_perm(cfg, gpu)
    for tau in (0.0, 0.01, 0.2):
        plain = B.prefill_early_stop(dq, dk, dv, cfg.block, cfg.segment, tau)
        permuted = B.prefill_early_stop(dq, dk, dv, cfg.block, cfg.segment, tau, perm=perm)
        torch.cuda.synchronize()
        assert torch.equal(plain.order, permuted.order) and torch.equal(plain.cnt, permuted.cnt)
        assert torch.equal(plain.nused, permuted.nused), tau
        assert torch.equal(plain.o, permuted.o) and torch.equal(plain.lse, permuted.lse), tau
        log("identity permutation, early stop", kw, "tau", tau, "mean history blocks",
            float(plain.nused.float().mean()), "bit-identical")
