"""GPU key permutation (importance from the last query block, sorted per
segment) against the float64 oracle, and the heavy-hitter prefill workload
run entirely on the device."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import log, pipeline_check, upload_prefill

pytestmark = pytest.mark.gpu

# Importance error relative to the row's largest importance.  Every
# probability is exp(x - lse) of a logit x that is a bf16 x bf16 dot product
# over d = 128 summed in fp32: at most d * 2^-24 * sum|q_c k_c| * scale, about
# 3.4e-4 for a heavy-hitter key (norm 4x, |q||k| about 500); exp2, the lse and
# the fp32 sums over the block's rows and the group's heads add about 1e-6.
IMP_RTOL = 1e-3
# Two keys may appear in either order only when their oracle importances are
# this close (the selection window of the block lists).
ORDER_RTOL = 1e-4


def check_permutation(cfg, q, k, perm_gpu, imp_gpu):
    scale = 1 / math.sqrt(cfg.d)
    worst_imp, swaps = 0.0, 0
    for b in range(cfg.batch):
        imp_ref = oracle.key_importance(q[b], k[b], cfg.block, scale)
        scale_imp = imp_ref.max(axis=1, keepdims=True)
        err = np.abs(imp_gpu[b] - imp_ref) / scale_imp
        worst_imp = max(worst_imp, float(err.max()))
        for g in range(cfg.hkv):
            for s0 in range(0, cfg.L, cfg.segment):
                seg = perm_gpu[b, g, s0:s0 + cfg.segment]
                assert sorted(seg.tolist()) == list(range(s0, s0 + seg.size)), (b, g, s0)
                # the GPU's own order is exactly non-increasing in its importance (ties by position)
                gi = imp_gpu[b, g, seg]
                assert np.all(np.diff(gi) <= 0)
                # against the oracle importance: out-of-order neighbours only within the tolerance
                ri = imp_ref[g, seg]
                bad = np.diff(ri) > ORDER_RTOL * np.maximum(ri[:-1], ri[1:]) + 1e-12
                swaps += int(bad.sum())
    log(cfg.name, f"max importance error {worst_imp:.3g} (relative to the row max), order violations {swaps}")
    assert worst_imp <= IMP_RTOL
    assert swaps == 0


@pytest.mark.parametrize("kw", [dict(L=1536, block=64, segment=256),
                                dict(L=1000, block=64, segment=256),        # ragged last block (40 rows)
                                dict(L=2048, block=128, segment=512, hq=8, hkv=8, d=64),
                                dict(L=777, block=16, segment=64, hq=4, hkv=1)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_key_permutation_matches_oracle(gpu, kw):
    base = dict(hq=8, hkv=2, d=128, heavy_hitters=True, seed=43, top_p=0.9)
    base.update(kw)
    cfg = I.small_prefill(name="perm", **base)
    q, k, v = I.prefill_inputs(cfg)
    dq, dk = P.to_dev(q, "bf16", gpu), P.to_dev(k, "bf16", gpu)
    perm, imp = B.key_permutation(dq, dk, cfg.block, cfg.segment, with_importance=True)
    torch.cuda.synchronize()
    check_permutation(cfg, q, k, perm.cpu().numpy(), imp.cpu().numpy())
    bad = torch.full((1,), -1, dtype=torch.int32, device=gpu)
    B.spot_validate_perm(B.prefill_desc(dq, dk, cfg.block, cfg.top_p, segment=cfg.segment), perm, bad)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("L,segment", [(1536, 256), (1000, 256), (777, 64), (16384 + 100, 16384)])
def test_validate_perm(gpu, L, segment):
    """The bijection check: random per-segment permutations (ragged last segments) pass; corruptions of
    known kind count one violation each (a repeated value, a value from another segment, values below 0
    or beyond L)."""
    batch, hkv = 2, 3
    rng = np.random.default_rng([L, segment])
    perm = np.empty((batch, hkv, L), dtype=np.int32)
    for b in range(batch):
        for g in range(hkv):
            for s0 in range(0, L, segment):
                perm[b, g, s0:s0 + segment] = rng.permutation(np.arange(s0, min(L, s0 + segment)))
    desc = B.make_desc(dtype=B.SPOT_BF16, batch=batch, hq=2 * hkv, hkv=hkv, d=128, q_len=L, kv_len=L, block=16,
                       segment=segment)
    bad = torch.full((1,), -1, dtype=torch.int32, device=gpu)

    def violations(p):
        B.spot_validate_perm(desc, torch.from_numpy(p).to(gpu), bad)
        torch.cuda.synchronize()
        return int(bad.item())

    assert violations(perm) == 0
    c = perm.copy()
    c[0, 0, 5] = c[0, 0, 6]                      # a value repeated inside segment 0
    assert violations(c) == 1
    c = perm.copy()
    c[1, 2, L - 1] = perm[1, 2, 0]               # the last position takes a value of segment 0
    assert violations(c) == 1
    c = perm.copy()
    c[0, 1, 3] = -5                              # below every segment
    c[1, 0, L - 2] = L + 7                       # beyond L
    c[1, 1, 2] = c[1, 1, 1]                      # and a repeat
    assert violations(c) == 3
    assert violations(perm) == 0                 # the count starts from zero on every call


def test_c3_heavy_hitter_prefill_on_device(gpu):
    """The heavy-hitter workload with the permutation generated on the GPU:
    permutation checked against the oracle importance, then the whole prefill
    checked against the oracle using that permutation."""
    cfg = I.C3
    host, dev = upload_prefill(cfg, gpu)
    q, k, v = host
    perm, imp = B.key_permutation(dev[0], dev[1], cfg.block, cfg.segment, with_importance=True)
    torch.cuda.synchronize()
    perm_np = perm.cpu().numpy()
    check_permutation(cfg, q, k, perm_np, imp.cpu().numpy())
    bufs = B.prefill(dev[0], dev[1], dev[2], cfg.block, cfg.top_p, perm=perm, segment=cfg.segment)
    torch.cuda.synchronize()
    rng = np.random.default_rng([cfg.seed, 7])
    blocks = sorted({0, 1, cfg.nb - 1} | set(rng.choice(cfg.nb, 13, replace=False).tolist()))
    pairs = [(0, int(rng.integers(cfg.hkv)), int(i)) for i in blocks]
    pipeline_check(cfg, host, bufs, perm=perm_np.astype(np.int64), pairs=pairs)
