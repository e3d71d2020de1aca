"""Representative-query history maps ([S2O] §1) and the early-stopped
attention walking them ([S2O] §2-3) on the GPU against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests.test_gpu_early_stop import es_check
from tests.test_gpu_parity import log, upload_prefill

pytestmark = pytest.mark.gpu

# Neighbours in the GPU's map may be out of the oracle's order only where
# their oracle scores agree to this (fp32 means and dot products).
MAP_TOL = 2e-5


def check_map(cfg, q, k, hmap_gpu):
    scale = 1 / math.sqrt(cfg.d)
    swaps = exact = rows = 0
    for b in range(cfg.batch):
        ref, score = oracle.history_map(q[b], k[b], cfg.segment, scale)
        for g in range(cfg.hkv):
            assert np.all(hmap_gpu[b, g, 0] == -1)
            for sg in range(1, ref.shape[1]):
                n = sg * cfg.segment
                m = hmap_gpu[b, g, sg, :n].astype(np.int64)
                assert sorted(m.tolist()) == list(range(n)), (b, g, sg)
                assert np.all(hmap_gpu[b, g, sg, n:] == -1)
                c = score[g, sg, m]
                tol = MAP_TOL * np.abs(score[g, sg, :n]).max() + 1e-7
                bad = np.diff(c) > tol
                swaps += int(bad.sum())
                exact += int(np.array_equal(m, ref[g, sg, :n]))
                rows += 1
    log(cfg.name, f"map rows {rows}, identical to the oracle's {exact}, order violations beyond tolerance {swaps}")
    assert swaps == 0


MAP_CASES = [
    dict(L=1536, segment=256, hq=8, hkv=2, d=128),
    dict(L=1000, segment=128, hq=4, hkv=2, d=64),                # ragged last segment
    dict(L=24576, segment=4096, hq=4, hkv=1, d=64),              # prefix above 16384: two-level sort
]


@pytest.mark.parametrize("kw", MAP_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_history_map_matches_oracle(gpu, kw):
    cfg = I.small_prefill(name="hmap", block=64, top_p=1.0, seed=71, heavy_hitters=True, **kw)
    q, k, v = I.prefill_inputs(cfg)
    host, dev = upload_prefill(cfg, gpu)
    hmap = B.history_map(dev[0], dev[1], cfg.segment)
    torch.cuda.synchronize()
    check_map(cfg, q, k, hmap.cpu().numpy())


ATT_CASES = [
    dict(L=1536, block=64, segment=256, tau=0.01),
    dict(L=2048, block=128, segment=512, tau=0.02, hq=8, hkv=8, d=64),
    dict(L=1280, block=64, segment=256, tau=0.0),               # the whole prefix: dense causal
    dict(L=1280, block=64, segment=128, tau=2.0, hq=16, hkv=2),  # one run per row
    dict(L=1100, block=64, segment=256, tau=0.01, batch=2),      # two sequences, ragged
]


@pytest.mark.parametrize("case", ATT_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_attention_on_gpu_maps(gpu, case):
    case = dict(case)
    tau = case.pop("tau")
    base = dict(hq=8, hkv=2, d=128, heavy_hitters=True, seed=73)
    base.update(case)
    cfg = I.small_prefill(name="hmap-attn", top_p=1.0, **base)
    host, dev = upload_prefill(cfg, gpu)
    hmap = B.history_map(dev[0], dev[1], cfg.segment)
    bufs = B.prefill_history_map(dev[0], dev[1], dev[2], cfg.block, cfg.segment, tau, hmap=hmap)
    torch.cuda.synchronize()
    hm = hmap.cpu().numpy()
    check_map(cfg, host[0], host[1], hm)
    es_check(cfg, host, None, None, bufs, tau, hmap=hm)
    nz = bufs.nused.cpu().numpy()
    if tau == 0.0:
        for i in range(cfg.nb):
            rows = slice(i * cfg.block, min((i + 1) * cfg.block, cfg.L))
            assert np.all(nz[:, :, rows] == (i * cfg.block // cfg.segment) * cfg.segment // cfg.block)
    if tau >= 1.0:
        assert set(np.unique(nz).tolist()) <= {0, 1}


def test_c3_history_map_on_device(gpu):
    """The heavy-hitter workload (L=32768, segment 2048) with maps and
    early stopping at tau = 0.01 on the GPU: maps of every segment checked,
    stops and outputs on sampled query blocks."""
    cfg = I.C3
    host, dev = upload_prefill(cfg, gpu)
    hmap = B.history_map(dev[0], dev[1], cfg.segment)
    bufs = B.prefill_history_map(dev[0], dev[1], dev[2], cfg.block, cfg.segment, 0.01, hmap=hmap)
    torch.cuda.synchronize()
    hm = hmap.cpu().numpy()
    check_map(cfg, host[0], host[1], hm)
    rng = np.random.default_rng([cfg.seed, 23])
    blocks = sorted({0, 16, cfg.nb - 1} | set(rng.choice(cfg.nb, 4, replace=False).tolist()))
    pairs = [(0, int(rng.integers(cfg.hkv)), int(i)) for i in blocks]
    es_check(cfg, host, None, None, bufs, 0.01, pairs=pairs, hmap=hm)
    log(cfg.name, "mean runs taken per row", float(bufs.nused.float().mean()))
