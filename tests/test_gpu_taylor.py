"""Second-order Taylor block score ([SPLA] §2.1) on the GPU: scores,
selection and attention output of the whole prefill path against the float64
oracle."""
import math

import numpy as np
import pytest

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests.test_gpu_parity import gpu_prefill, log, pipeline_check, upload_prefill

pytestmark = pytest.mark.gpu

TAYLOR = B.SPOT_SCORE_TAYLOR

CASES = [
    dict(L=1000, hq=8, hkv=2, d=128, block=64, top_p=0.9),
    dict(L=700, hq=8, hkv=2, d=64, block=32, top_p=0.8, heavy_hitters=True),
    dict(L=513, hq=4, hkv=4, d=128, block=16, top_p=0.7),
    dict(L=2048, hq=16, hkv=2, d=128, block=128, top_p=0.95, heavy_hitters=True),
    dict(L=300, hq=2, hkv=2, d=64, block=16, top_p=0.9, dtype="f32"),
    dict(L=900, hq=8, hkv=2, d=128, block=64, top_p=0.9, batch=2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_taylor_pipeline_small(gpu, case):
    cfg = I.small_prefill(name="taylor", seed=23, **case)
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev, score_kind=TAYLOR)
    pipeline_check(cfg, host, bufs, score="taylor")


def test_taylor_pipeline_with_permutation(gpu):
    """History blocks are scored with the statistics of the permuted rows."""
    cfg = I.small_prefill(name="taylor-perm", L=2048, hq=8, hkv=2, d=128, block=64, top_p=0.9, seed=29,
                          heavy_hitters=True, segment=512)
    q, k, v = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    host, dev = upload_prefill(cfg, gpu, perm[None])
    bufs = gpu_prefill(cfg, dev, perm_dev=dev[3], score_kind=TAYLOR)
    pipeline_check(cfg, host, bufs, perm=perm[None], score="taylor")


def test_taylor_c2_sampled(gpu):
    """The GQA workload (L=8192, 32/8 heads, block 64) with the Taylor score:
    scores everywhere, selection and output on a seeded sample of query
    blocks of every KV head."""
    cfg = I.C2
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev, score_kind=TAYLOR)
    rng = np.random.default_rng([cfg.seed, 41])
    blocks = sorted({0, 1, cfg.nb - 1} | set(rng.choice(cfg.nb, 9, replace=False).tolist()))
    pairs = [(0, g, i) for g in range(cfg.hkv) for i in blocks]
    rep, err = pipeline_check(cfg, host, bufs, pairs=pairs, score="taylor")
    cnt = bufs.cnt.cpu().numpy()
    log("taylor c2 mean kept blocks per row", float(cnt.mean()))
