"""Early-stopped prefill ([S2O] §2 early-stopping rule, §3 kernel passes) on
the GPU against the float64 oracle: the visiting order of the history blocks,
each row's stop point and the attention output at that stop point."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import log, upload_prefill

pytestmark = pytest.mark.gpu

# A row's stop point may differ from the exact rule only where the oracle's
# gain ratio lies within this relative distance of tau.  The kernel's ratio
# is (sum of the block's P) / (sum of all P so far), every P rounded to bf16
# (relative error at most 2^-8 per term, so at most 2^-8 on each sum; one
# heavy key can carry a whole block's mass, so the bound is reached) and the
# sums kept in fp32 (at most a few hundred tiles: below 1e-4 relative).  The
# ratio is therefore within (1 + 2^-8) / (1 - 2^-8) - 1 + 1e-4 = 7.9e-3 of
# the exact one.
RATIO_REL = (1 + 2.0 ** -8) / (1 - 2.0 ** -8) - 1 + 1e-4


def order_nested(order_np, cnt_np, b, hkv, blocks):
    out = [dict() for _ in range(hkv)]
    for g in range(hkv):
        for i in blocks:
            out[g][i] = order_np[b, g, i, :cnt_np[b, g, i]].astype(np.int64)
    return out


def es_check(cfg, host, order_np, cnt_np, bufs, tau, perm=None, pairs=None, hmap=None):
    """Stop points and outputs of an early-stopped GPU prefill against the oracle.

    pairs: (b, g, i) query blocks to check (default: all); hmap (batch, hkv,
    nseg, L): the history maps the GPU walked (order_np and cnt_np unused)."""
    q, k, v = host
    scale = 1.0 / math.sqrt(cfg.d)
    G = cfg.hq // cfg.hkv
    go = bufs.o.float().cpu().numpy()
    glse = bufs.lse.cpu().numpy()
    gn = bufs.nused.cpu().numpy()
    pairs = [(b, g, i) for b in range(cfg.batch) for g in range(cfg.hkv) for i in range(cfg.nb)] \
        if pairs is None else pairs
    rows_total = exact = near = 0
    worst = worst_lse = 0.0
    near_dev = 0.0   # largest |ratio / tau - 1| at a row whose stop point differs
    taken = 0
    for b, g, i in pairs:
        n_hist = ((i * cfg.block) // cfg.segment) * cfg.segment // cfg.block
        if hmap is None:
            assert cnt_np[b, g, i] == n_hist
            hist = order_np[b, g, i, :n_hist].astype(np.int64)
            assert np.all(order_np[b, g, i, n_hist:] == -1)
        else:
            hist = None
        hm = None if hmap is None else hmap[b].astype(np.int64)
        pb = None if perm is None else perm[b]
        rows = oracle.block_rows(i, cfg.block, cfg.L)
        for h in range(g * G, (g + 1) * G):
            ratio = oracle.es_gain_ratios(q[b], k[b], i, g, h, hist, cfg.block, cfg.segment, scale, pb, hm)
            for ri, r in enumerate(rows):
                n = int(gn[b, h, r])
                rows_total += 1
                assert 0 <= n <= n_hist, (b, h, r, n, n_hist)
                below = np.nonzero(ratio[ri] < tau)[0]
                n_exact = int(below[0]) + 1 if below.size else n_hist
                if n == n_exact:
                    exact += 1
                else:
                    near += 1
                    # the first block where the two decisions part: one side stops there, the other goes on
                    k_part = max(min(n, n_exact) - 1, 0)
                    near_dev = max(near_dev, abs(float(ratio[ri, k_part]) / tau - 1.0))
                    # did not stop earlier than allowed, and stopped where the ratio was (nearly) below tau
                    assert np.all(ratio[ri, :max(n - 1, 0)] >= tau * (1 - RATIO_REL)), (b, h, r, n, n_exact)
                    assert n == n_hist or ratio[ri, n - 1] < tau * (1 + RATIO_REL), (b, h, r, n, n_exact)
                taken += n
        # output and LSE: the oracle evaluated at the GPU's stop points
        ords = [dict() for _ in range(cfg.hkv)]
        ords[g][i] = hist
        o_ref, lse_ref, used_ref = oracle.attend_prefill_es(
            q[b, g * G:(g + 1) * G], k[b, g:g + 1], v[b, g:g + 1], None if hm is not None else [ords[g]],
            cfg.block, cfg.segment, scale, tau, perm=None if pb is None else pb[g:g + 1], qblocks=[i],
            nused=gn[b, g * G:(g + 1) * G], hmap=None if hm is None else hm[g:g + 1])
        rs = slice(rows[0], rows[-1] + 1)
        worst = max(worst, P.max_abs(go[b, g * G:(g + 1) * G, rs], o_ref[:, rs]))
        worst_lse = max(worst_lse, P.max_abs(glse[b, g * G:(g + 1) * G, rs], lse_ref[:, rs]))
    log(cfg.name, f"tau={tau} rows={rows_total} exact stops={exact} within-rounding={near} "
        f"history blocks taken={taken} max|dO|={worst:.3g} max|dLSE|={worst_lse:.3g} "
        f"largest |ratio/tau-1| at a differing stop={near_dev:.3g} (window {RATIO_REL:.3g})")
    assert worst <= P.BF16_ATOL, worst
    assert worst_lse <= P.BF16_LSE_ATOL, worst_lse
    assert near <= max(2, rows_total // 100)
    return taken


def gpu_es(cfg, dev, order_dev, cnt_dev, tau, perm_dev=None):
    dq, dk, dv = dev[:3]
    desc = B.prefill_desc(dq, dk, cfg.block, 1.0, segment=cfg.segment)
    bufs = B.alloc_prefill_early_stop(desc, dq.device)
    B.spot_sparse_attn_prefill_early_stop(desc, tau, dq, dk, dv, perm_dev, order_dev, cnt_dev, bufs.o, bufs.lse,
                                          bufs.nused)
    torch.cuda.synchronize()
    return bufs


def test_order_history_on_oracle_scores(gpu):
    """Same fp32 scores on both sides: the visiting order must match exactly
    (scores rounded to one decimal so that many are tied)."""
    rng = np.random.default_rng(21)
    for (L, block, segment, hkv) in ((640, 16, 64, 2), (4096 * 16, 16, 2048, 1), (9000, 64, 512, 3)):
        nb = -(-L // block)
        s = np.round(rng.standard_normal((1, hkv, nb, nb)), 1).astype(np.float32)
        desc = B.make_desc(dtype=B.SPOT_BF16, batch=1, hq=hkv, hkv=hkv, d=128, q_len=L, kv_len=L, block=block,
                           segment=segment)
        ds = torch.from_numpy(s).to(gpu)
        order = torch.empty(1, hkv, nb, nb, dtype=torch.int32, device=gpu)
        cnt = torch.empty(1, hkv, nb, dtype=torch.int32, device=gpu)
        B.spot_order_history(desc, ds, order, cnt)
        torch.cuda.synchronize()
        on, cn = order.cpu().numpy(), cnt.cpu().numpy()
        rows = range(nb) if nb <= 700 else sorted(set(rng.choice(nb, 64, replace=False).tolist()) | {nb - 1})
        ref = oracle.history_order(s[0].astype(np.float64), block, segment, rows=rows)
        for g in range(hkv):
            for i in rows:
                n = len(ref[g][i])
                assert cn[0, g, i] == n
                assert np.array_equal(on[0, g, i, :n], ref[g][i]), (L, g, i)
                assert np.all(on[0, g, i, n:] == -1)
        log("order", L, block, segment, "rows checked", len(rows) * hkv)


ES_CASES = [
    dict(L=1536, block=64, segment=256, tau=0.01, perm=True),
    dict(L=1000, block=64, segment=256, tau=0.05, perm=False),          # ragged last block
    dict(L=2048, block=128, segment=512, tau=0.02, perm=True, hq=8, hkv=8, d=64),
    dict(L=1280, block=128, segment=256, tau=0.0, perm=True),           # dense causal
    dict(L=1280, block=64, segment=128, tau=2.0, perm=True, hq=16, hkv=2),  # one history block per row
    dict(L=900, block=64, segment=64, tau=0.003, perm=False, hq=6, hkv=3, d=64),
    dict(L=1100, block=64, segment=256, tau=0.01, perm=True, batch=2),     # two sequences, ragged
]


@pytest.mark.parametrize("case", ES_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_early_stop_on_oracle_order(gpu, case):
    case = dict(case)
    tau, use_perm = case.pop("tau"), case.pop("perm")
    base = dict(hq=8, hkv=2, d=128, heavy_hitters=True, seed=61)
    base.update(case)
    cfg = I.small_prefill(name="es", top_p=1.0, **base)
    q, k, v = I.prefill_inputs(cfg)
    scale = 1 / math.sqrt(cfg.d)
    perm = None
    if use_perm:
        perm = np.stack([oracle.key_permutation(q[b], k[b], cfg.block, cfg.segment, scale)[0]
                         for b in range(cfg.batch)])
    host, dev = upload_prefill(cfg, gpu, perm)
    order_np = np.full((cfg.batch, cfg.hkv, cfg.nb, cfg.nb), -1, dtype=np.int32)
    cnt_np = np.zeros((cfg.batch, cfg.hkv, cfg.nb), dtype=np.int32)
    for b in range(cfg.batch):
        qbar, kn, kp = oracle.pool_blocks(q[b], k[b], cfg.block, None if perm is None else perm[b])
        s = oracle.meanpool_scores(qbar, kn, kp, cfg.block, cfg.segment if use_perm else 0, scale)
        od = oracle.history_order(s, cfg.block, cfg.segment)
        for g in range(cfg.hkv):
            for i in range(cfg.nb):
                order_np[b, g, i, :len(od[g][i])] = od[g][i]
                cnt_np[b, g, i] = len(od[g][i])
    bufs = gpu_es(cfg, dev, torch.from_numpy(order_np).to(gpu), torch.from_numpy(cnt_np).to(gpu), tau, dev[3])
    taken = es_check(cfg, host, order_np, cnt_np, bufs, tau, perm=perm)
    total_hist = sum(int(cnt_np[b, g, i]) * min(cfg.block, cfg.L - i * cfg.block) * (cfg.hq // cfg.hkv)
                     for b in range(cfg.batch) for g in range(cfg.hkv) for i in range(cfg.nb))
    if tau == 0.0:
        assert taken == total_hist      # every history block
    if tau >= 1.0:
        nz = bufs.nused.cpu().numpy()
        assert set(np.unique(nz).tolist()) <= {0, 1}


def test_early_stop_pipeline_on_device(gpu):
    """Scores, order and early-stopped attention all on the GPU, with the
    permutation generated on the GPU: scores against the oracle, the order
    against the oracle's ordering of the GPU's own scores, then stops and
    outputs."""
    cfg = I.small_prefill(name="es-pipe", L=3072, hq=8, hkv=2, d=128, block=128, segment=512, heavy_hitters=True,
                          seed=62, top_p=1.0)
    host, dev = upload_prefill(cfg, gpu)
    q, k, v = host
    perm = B.key_permutation(dev[0], dev[1], cfg.block, cfg.segment)
    tau = 0.01
    bufs = B.prefill_early_stop(dev[0], dev[1], dev[2], cfg.block, cfg.segment, tau, perm=perm)
    torch.cuda.synchronize()
    perm_np = perm.cpu().numpy().astype(np.int64)
    gs = bufs.scores.cpu().numpy()
    qbar, kn, kp = oracle.pool_blocks(q[0], k[0], cfg.block, perm_np[0])
    s = oracle.meanpool_scores(qbar, kn, kp, cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    fin = np.isfinite(s)
    assert np.all(np.abs(gs[0][fin] - s[fin]) <= 1e-5 * np.abs(s[fin]) + 2e-6)
    on, cn = bufs.order.cpu().numpy(), bufs.cnt.cpu().numpy()
    ref = oracle.history_order(gs[0].astype(np.float64), cfg.block, cfg.segment)
    for g in range(cfg.hkv):
        for i in range(cfg.nb):
            assert np.array_equal(on[0, g, i, :cn[0, g, i]], ref[g][i])
    es_check(cfg, host, on, cn, bufs, tau, perm=perm_np)


def test_c3_early_stop_on_device(gpu):
    """The heavy-hitter workload (L=32768, segment 2048) early-stopped at
    tau = 0.01 with the device permutation; stops and outputs checked on
    sampled query blocks, the order checked on the same blocks."""
    cfg = I.C3
    host, dev = upload_prefill(cfg, gpu)
    perm = B.key_permutation(dev[0], dev[1], cfg.block, cfg.segment)
    tau = 0.01
    bufs = B.prefill_early_stop(dev[0], dev[1], dev[2], cfg.block, cfg.segment, tau, perm=perm)
    torch.cuda.synchronize()
    perm_np = perm.cpu().numpy().astype(np.int64)
    gs = bufs.scores.cpu().numpy()
    on, cn = bufs.order.cpu().numpy(), bufs.cnt.cpu().numpy()
    rng = np.random.default_rng([cfg.seed, 17])
    blocks = sorted({0, 16, cfg.nb - 1} | set(rng.choice(cfg.nb, 5, replace=False).tolist()))
    pairs = [(0, int(rng.integers(cfg.hkv)), int(i)) for i in blocks]
    for _, g, i in pairs:
        ref = oracle.history_order(gs[0, g:g + 1].astype(np.float64), cfg.block, cfg.segment, rows=[i])
        assert np.array_equal(on[0, g, i, :cn[0, g, i]], ref[0][i])
    es_check(cfg, host, on, cn, bufs, tau, perm=perm_np, pairs=pairs)
    nz = bufs.nused.cpu().numpy()
    log(cfg.name, "mean history blocks taken per row", float(nz.mean()))
