"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Selection: kept lists identical except for blocks within 1e-4 of the top-p
cutoff (see parity.compare_selection).  Outputs: compared with the oracle's
attention evaluated on the GPU's own kept lists, max-abs 2e-2 in bf16 and
1e-4 in fp32.  Large workloads are checked on seeded samples of (KV head,
query block) rows."""
import math
import time

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu


def log(*a):
    print("[parity]", *a, flush=True)


# ----------------------------------------------------------------- helpers
def upload_prefill(cfg, device, perm=None):
    q, k, v = I.prefill_inputs(cfg)
    dq = P.to_dev(q, cfg.dtype, device)
    dk = P.to_dev(k, cfg.dtype, device)
    dv = P.to_dev(v, cfg.dtype, device)
    dp = None if perm is None else torch.from_numpy(perm.astype(np.int32)).to(device).contiguous()
    return (q, k, v), (dq, dk, dv, dp)


def gpu_prefill(cfg, dev_inputs, perm_dev=None, top_p=None, score_kind=B.SPOT_SCORE_MEANPOOL, **kw):
    dq, dk, dv, _ = dev_inputs
    bufs = B.prefill(dq, dk, dv, cfg.block, cfg.top_p if top_p is None else top_p, perm=perm_dev,
                     segment=cfg.segment if perm_dev is not None else 0, n_sink=kw.get("n_sink", cfg.n_sink),
                     n_recent=kw.get("n_recent", cfg.n_recent), k_min=kw.get("k_min", cfg.k_min),
                     score_kind=score_kind)
    torch.cuda.synchronize()
    return bufs


def pipeline_check(cfg, host, bufs, perm=None, pairs=None, top_p=None, n_sink=None, n_recent=None, k_min=None,
                   check_scores=True, score="meanpool"):
    """Scores, selection and output of a GPU prefill against the oracle.

    pairs: list of (b, g, i) rows to check (default: all); score: "meanpool"
    or "taylor" (the block score the GPU used)."""
    q, k, v = host
    top_p = cfg.top_p if top_p is None else top_p
    n_sink = cfg.n_sink if n_sink is None else n_sink
    n_recent = cfg.n_recent if n_recent is None else n_recent
    k_min = cfg.k_min if k_min is None else k_min
    d = cfg.d
    scale = 1.0 / math.sqrt(d)
    G = cfg.hq // cfg.hkv
    seg = cfg.segment if perm is not None else 0
    gs = bufs.scores.cpu().numpy()
    gl = P.kept_lists(bufs.idx, bufs.cnt)
    go = bufs.o.float().cpu().numpy()
    glse = bufs.lse.cpu().numpy()
    P.check_list_format(bufs.idx, bufs.cnt, lambda i: i + 1)
    atol = P.BF16_ATOL if cfg.dtype == "bf16" else P.F32_ATOL
    lse_atol = P.BF16_LSE_ATOL if cfg.dtype == "bf16" else P.F32_LSE_ATOL
    rep = P.SelectionReport()
    worst = 0.0
    worst_lse = 0.0
    for b in range(cfg.batch):
        pb = None if perm is None else perm[b]
        qbar, kn, kp = oracle.pool_blocks(q[b], k[b], cfg.block, pb)
        if score == "taylor":
            vn, vp = oracle.key_block_variance(k[b], cfg.block, pb)
            s = oracle.taylor_scores(qbar, kn, kp, vn, vp, cfg.block, seg, scale)
        else:
            s = oracle.meanpool_scores(qbar, kn, kp, cfg.block, seg, scale)
        if check_scores:
            fin = np.isfinite(s)
            assert np.array_equal(fin, np.isfinite(gs[b]))
            err = np.abs(gs[b][fin] - s[fin])
            assert np.all(err <= 1e-5 * np.abs(s[fin]) + 2e-6), float(err.max())
        rows = [(g, i) for g in range(cfg.hkv) for i in range(cfg.nb)] if pairs is None else \
            [(g, i) for (bb, g, i) in pairs if bb == b]
        for g, i in rows:
            forced = oracle.prefill_forced(i, n_sink, n_recent)
            P.compare_selection(rep, gl[b][g][i], s[g, i, :i + 1], forced, top_p, k_min, (b, g, i))
            o_ref, lse_ref = oracle.attend_prefill(q[b, g * G:(g + 1) * G], k[b, g:g + 1], v[b, g:g + 1],
                                                   [{i: gl[b][g][i]}], cfg.block, scale, seg,
                                                   None if pb is None else pb[g:g + 1], qblocks=[i])
            rs = slice(i * cfg.block, min((i + 1) * cfg.block, cfg.L))
            worst = max(worst, P.max_abs(go[b, g * G:(g + 1) * G, rs], o_ref[:, rs]))
            worst_lse = max(worst_lse, P.max_abs(glse[b, g * G:(g + 1) * G, rs], lse_ref[:, rs]))
    log(cfg.name, "selection", rep, f"max|dO|={worst:.3g} max|dLSE|={worst_lse:.3g}")
    assert not rep.violations, rep.violations[:10]
    assert worst <= atol, worst
    assert worst_lse <= lse_atol, worst_lse
    return rep, worst


# ----------------------------------------------------------------- attention kernel on oracle lists
ATTN_CASES = [
    dict(L=1000, hq=8, hkv=2, d=128, block=64, top_p=0.9),
    dict(L=1000, hq=8, hkv=2, d=128, block=128, top_p=0.8),
    dict(L=700, hq=8, hkv=2, d=64, block=32, top_p=0.9),
    dict(L=513, hq=4, hkv=4, d=128, block=16, top_p=0.7),
    dict(L=1024, hq=16, hkv=2, d=128, block=64, top_p=0.9),
    dict(L=777, hq=6, hkv=3, d=64, block=64, top_p=0.5),
    dict(L=640, hq=8, hkv=2, d=128, block=64, top_p=1.0),
    dict(L=640, hq=8, hkv=2, d=128, block=64, top_p=0.0),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_prefill_attention_on_oracle_lists(gpu, case):
    cfg = I.small_prefill(name="attn", seed=31, **case)
    log("case", case)
    host, dev = upload_prefill(cfg, gpu)
    q, k, v = host
    ref = oracle.prefill(q[0], k[0], v[0], cfg.block, cfg.top_p)
    nb = cfg.nb
    idx = np.full((1, cfg.hkv, nb, nb), -1, np.int32)
    cnt = np.zeros((1, cfg.hkv, nb), np.int32)
    for g in range(cfg.hkv):
        for i in range(nb):
            kl = ref["kept"][g][i]
            idx[0, g, i, :len(kl)] = kl
            cnt[0, g, i] = len(kl)
    desc = B.prefill_desc(dev[0], dev[1], cfg.block, cfg.top_p)
    o = torch.full_like(dev[0], float("nan"))
    lse = torch.full((1, cfg.hq, cfg.L), float("nan"), device=gpu)
    B.spot_sparse_attn_prefill(desc, dev[0], dev[1], dev[2], None, torch.from_numpy(idx).to(gpu),
                               torch.from_numpy(cnt).to(gpu), o, lse)
    torch.cuda.synchronize()
    err = P.max_abs(o.float().cpu().numpy()[0], ref["o"])
    err_lse = P.max_abs(lse.cpu().numpy()[0], ref["lse"])
    log("max|dO|", err, "max|dLSE|", err_lse)
    assert err <= P.BF16_ATOL
    assert err_lse <= 1e-2


def test_prefill_attention_with_permutation_on_oracle_lists(gpu):
    cfg = I.small_prefill(name="attn-perm", L=1536, hq=8, hkv=2, d=128, block=64, top_p=0.6, seed=41,
                          heavy_hitters=True, segment=256)
    host, dev = upload_prefill(cfg, gpu)
    q, k, v = host
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    dperm = torch.from_numpy(perm[None].astype(np.int32)).to(gpu)
    ref = oracle.prefill(q[0], k[0], v[0], cfg.block, cfg.top_p, segment=cfg.segment, perm=perm)
    nb = cfg.nb
    idx = np.full((1, cfg.hkv, nb, nb), -1, np.int32)
    cnt = np.zeros((1, cfg.hkv, nb), np.int32)
    for g in range(cfg.hkv):
        for i in range(nb):
            kl = ref["kept"][g][i]
            idx[0, g, i, :len(kl)] = kl
            cnt[0, g, i] = len(kl)
    desc = B.prefill_desc(dev[0], dev[1], cfg.block, cfg.top_p, segment=cfg.segment)
    o = torch.full_like(dev[0], float("nan"))
    B.spot_sparse_attn_prefill(desc, dev[0], dev[1], dev[2], dperm, torch.from_numpy(idx).to(gpu),
                               torch.from_numpy(cnt).to(gpu), o)
    torch.cuda.synchronize()
    err = P.max_abs(o.float().cpu().numpy()[0], ref["o"])
    log("perm max|dO|", err)
    assert err <= P.BF16_ATOL


LONG_LIST_CASES = [
    dict(d=64, hq=2, perm=False),
    dict(d=128, hq=4, perm=True),
]


@pytest.mark.parametrize("case", LONG_LIST_CASES, ids=lambda c: f"d{c['d']}-perm{int(c['perm'])}")
def test_prefill_attention_lists_longer_than_lds_copy(gpu, case):
    """2055 blocks per sequence (block 16, ragged last block): more than the
    kept-list entries the kernel copies to LDS (2048), so its lists are read
    from HBM.  Kept lists are drawn on the host (sink, about 2% of the earlier
    blocks, diagonal); the oracle evaluates sampled query blocks on both
    sides of the 2048 boundary."""
    block, nb = 16, 2055
    L = nb * block - 7
    segment = 4096 if case["perm"] else 0
    cfg = I.small_prefill(name="long-lists", L=L, hq=case["hq"], hkv=1, d=case["d"], block=block, top_p=0.9,
                          seed=53, segment=segment)
    host, dev = upload_prefill(cfg, gpu)
    q, k, v = host
    perm = None
    dperm = None
    if case["perm"]:
        perm, _ = oracle.key_permutation(q[0], k[0], block, segment, 1 / math.sqrt(cfg.d))
        dperm = torch.from_numpy(perm[None].astype(np.int32)).to(gpu)
    rng = np.random.default_rng(53)
    idx = np.full((1, 1, nb, nb), -1, np.int32)
    cnt = np.zeros((1, 1, nb), np.int32)
    kept = [[None] * nb]
    for i in range(nb):
        mid = np.flatnonzero(rng.random(max(i - 1, 0)) < 0.02) + 1 if i > 1 else np.zeros(0, np.int64)
        kl = np.unique(np.concatenate([[0], mid, [i]])).astype(np.int64)
        kept[0][i] = kl
        idx[0, 0, i, :len(kl)] = kl
        cnt[0, 0, i] = len(kl)
    desc = B.prefill_desc(dev[0], dev[1], block, cfg.top_p, segment=segment)
    o = torch.full_like(dev[0], float("nan"))
    lse = torch.full((1, cfg.hq, L), float("nan"), device=gpu)
    B.spot_sparse_attn_prefill(desc, dev[0], dev[1], dev[2], dperm, torch.from_numpy(idx).to(gpu),
                               torch.from_numpy(cnt).to(gpu), o, lse)
    torch.cuda.synchronize()
    qb = [0, 1, 700, 2046, 2047, 2048, 2053, 2054]
    o_ref, lse_ref = oracle.attend_prefill(q[0], k[0], v[0], kept, block, 1 / math.sqrt(cfg.d), segment=segment,
                                           perm=perm, qblocks=qb)
    rows = np.concatenate([np.arange(i * block, min((i + 1) * block, L)) for i in qb])
    err = P.max_abs(o.float().cpu().numpy()[0][:, rows], o_ref[:, rows])
    err_lse = P.max_abs(lse.cpu().numpy()[0][:, rows], lse_ref[:, rows])
    log("long lists", case, "max|dO|", err, "max|dLSE|", err_lse)
    assert err <= P.BF16_ATOL
    assert err_lse <= 1e-2


# ----------------------------------------------------------------- scores and selection kernels
def test_select_kernel_on_oracle_scores(gpu):
    """Selection kernel alone: both sides see the same fp32 scores."""
    cfg = I.small_prefill(name="sel", L=2048, hq=4, hkv=2, d=64, block=16, top_p=0.9, seed=5)
    q, k, v = I.prefill_inputs(cfg)
    qbar, kn, kp = oracle.pool_blocks(q[0], k[0], cfg.block)
    s = oracle.meanpool_scores(qbar, kn, kp, cfg.block, 0, 1 / 8).astype(np.float32)
    nb = cfg.nb
    for top_p, k_min, n_sink, n_recent in [(0.9, 0, 1, 1), (0.5, 3, 2, 1), (0.99, 0, 0, 2), (1.0, 0, 1, 1),
                                           (0.0, 0, 1, 1), (0.0, 5, 1, 0)]:
        desc = B.make_desc(dtype=B.SPOT_F32, batch=1, hq=4, hkv=2, d=64, q_len=cfg.L, kv_len=cfg.L, block=16,
                           top_p=top_p, k_min=k_min, n_sink=n_sink, n_recent=n_recent)
        ds = torch.from_numpy(s[None]).to(gpu)
        idx = torch.full((1, 2, nb, nb), -7, dtype=torch.int32, device=gpu)
        cnt = torch.full((1, 2, nb), -7, dtype=torch.int32, device=gpu)
        B.spot_select_topp(desc, ds, idx, cnt)
        torch.cuda.synchronize()
        gl = P.kept_lists(idx, cnt)
        rep = P.SelectionReport()
        s64 = s.astype(np.float64)
        for g in range(2):
            for i in range(nb):
                P.compare_selection(rep, gl[0][g][i], s64[g, i, :i + 1],
                                    oracle.prefill_forced(i, n_sink, n_recent), top_p, k_min, (g, i))
        log("select", top_p, k_min, n_sink, n_recent, rep)
        assert not rep.violations, rep.violations[:5]
        assert rep.mismatched_rows == 0 or top_p not in (0.0, 1.0)


LONG_ROWS = [
    # (name, candidates, score recipe): flat and narrow rows leave more than 2048 candidates after the
    # histogram narrowing (cutoff search), N(0, 2.5) leaves about a thousand (bitonic sort), N(0, 4) a
    # few dozen (ranking by counting); 5001 candidates put every row after the first off 16-byte alignment
    ("flat", 8192, lambda r, n: np.zeros(n)),
    ("narrow", 8192, lambda r, n: r.normal(0.0, 0.05, n)),
    ("wide", 8192, lambda r, n: r.normal(0.0, 2.5, n)),
    ("ties", 8192, lambda r, n: np.round(r.normal(0.0, 2.5, n), 1)),
    ("peaked", 5001, lambda r, n: r.normal(0.0, 4.0, n)),
    ("widest", 16384, lambda r, n: r.normal(0.0, 2.5, n)),
]


@pytest.mark.parametrize("case", LONG_ROWS, ids=lambda c: f"{c[0]}-{c[1]}")
def test_select_long_decode_rows(gpu, case):
    """Selection kernel on long decode rows, both sides on the same fp32 scores.  Besides the
    cutoff rule (parity.compare_selection), the kept residual blocks must be exactly a prefix of
    the oracle's order (score descending, ties to the lower block id)."""
    name, nk, recipe = case
    rng = np.random.default_rng([31, nk, len(name)])
    rows = 4
    s = np.stack([recipe(rng, nk) for _ in range(rows)]).astype(np.float32)
    top_p = float(np.float32(0.9))
    desc = B.make_desc(dtype=B.SPOT_BF16, batch=rows, hq=32, hkv=8, d=128, q_len=1, kv_len=16 * nk, block=16,
                       top_p=top_p, n_sink=1, n_recent=1, score_kind=B.SPOT_SCORE_RELU_INDEXER, h_idx=4, d_idx=64)
    idx = torch.full((rows, 1, 1, nk), -7, dtype=torch.int32, device=gpu)
    cnt = torch.full((rows, 1, 1), -7, dtype=torch.int32, device=gpu)
    B.spot_select_topp(desc, torch.from_numpy(s[:, None, None]).to(gpu), idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy()[:, 0, 0], cnt.cpu().numpy()[:, 0, 0]
    rep = P.SelectionReport()
    forced = oracle.decode_forced(nk, 1, 1)
    for r in range(rows):
        kept = gi[r, :gc[r]]
        assert np.all(gi[r, gc[r]:] == -1) and np.all(np.diff(kept) > 0)
        det = oracle.topp_detail(s[r].astype(np.float64), forced, top_p, 0)
        resid = kept[~forced[kept]]
        assert set(resid.tolist()) == set(det["order"][:resid.size].tolist()), (name, r)
        if name == "flat":   # equal masses are exact on both sides: the same count
            assert np.array_equal(kept, det["kept"]), (name, r, kept.size, det["kept"].size)
        P.compare_selection(rep, kept, s[r].astype(np.float64), forced, top_p, 0, r)
    log("long rows", name, nk, rep, "kept", gc.tolist())
    assert not rep.violations, rep.violations[:5]


def test_indexer_scores_and_decode_select(gpu):
    cfg = I.C4.with_(batch=3, T=16 * 3000 + 7, name="dec-small")
    D = I.decode_inputs(cfg)
    desc = B.decode_desc(P.to_dev(D["q"], "bf16", gpu), P.to_dev(D["k_cache"], "bf16", gpu), cfg.block,
                         cfg.top_p, cfg.h_idx, cfg.d_idx)
    scores = torch.empty(cfg.batch, 1, 1, cfg.nt, device=gpu)
    B.spot_block_score(desc, None, None, None, P.to_dev(D["idx_q"], "bf16", gpu),
                       torch.from_numpy(D["idx_w"]).to(gpu), P.to_dev(D["idx_k"], "bf16", gpu), scores)
    idx = torch.empty(cfg.batch, 1, 1, cfg.nt, dtype=torch.int32, device=gpu)
    cnt = torch.empty(cfg.batch, 1, 1, dtype=torch.int32, device=gpu)
    B.spot_select_topp(desc, scores, idx, cnt)
    torch.cuda.synchronize()
    gs = scores.cpu().numpy()[:, 0, 0]
    gl = idx.cpu().numpy()[:, 0, 0]
    gc = cnt.cpu().numpy()[:, 0, 0]
    rep = P.SelectionReport()
    for b in range(cfg.batch):
        s = oracle.indexer_scores(D["idx_q"][b], D["idx_w"][b], D["idx_k"][b])
        err = np.abs(gs[b] - s)
        assert np.all(err <= 1e-5 * np.abs(s) + 1e-5), float(err.max())
        P.compare_selection(rep, gl[b, :gc[b]], s, oracle.decode_forced(cfg.nt, 1, 1), cfg.top_p, 0, b)
        assert np.all(gl[b, gc[b]:] == -1)
    log("decode select", rep, "kept", gc.tolist(), "of", cfg.nt)
    assert not rep.violations, rep.violations[:5]


# ----------------------------------------------------------------- whole prefill pipeline
PIPE_SMALL = [
    dict(L=1000, hq=8, hkv=2, d=128, block=64, top_p=0.9),
    dict(L=1000, hq=8, hkv=2, d=128, block=128, top_p=0.95, heavy_hitters=True),
    dict(L=523, hq=4, hkv=1, d=64, block=16, top_p=0.8),
    dict(L=40, hq=4, hkv=2, d=128, block=64, top_p=0.9),        # one partial block
    dict(L=1, hq=2, hkv=1, d=64, block=16, top_p=0.9),          # a single token
    dict(L=300, hq=2, hkv=2, d=64, block=16, top_p=0.9, dtype="f32"),
    dict(L=333, hq=4, hkv=2, d=128, block=32, top_p=0.85, dtype="f32"),   # fp32 rows kernel at d = 128
    dict(L=900, hq=16, hkv=4, d=128, block=64, top_p=0.9, batch=2),   # 8 (batch, KV head) pairs: XCD-pinned order
    dict(L=600, hq=8, hkv=2, d=64, block=32, top_p=0.85, batch=3),
]


@pytest.mark.parametrize("case", PIPE_SMALL, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_prefill_pipeline_small(gpu, case):
    cfg = I.small_prefill(name="pipe", seed=7, **case)
    log("case", case)
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev)
    pipeline_check(cfg, host, bufs)


@pytest.mark.parametrize("kw", [dict(top_p=0.0), dict(top_p=1.0), dict(top_p=0.6, k_min=4),
                                dict(top_p=0.9, n_sink=2, n_recent=2), dict(top_p=0.9, n_sink=0, n_recent=1),
                                dict(top_p=0.9, n_sink=1, n_recent=0)])
def test_prefill_pipeline_selection_parameters(gpu, kw):
    cfg = I.small_prefill(name="params", L=900, hq=8, hkv=2, d=128, block=64, seed=9, batch=2)
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev, top_p=kw.get("top_p"), **{k: v for k, v in kw.items() if k != "top_p"})
    pipeline_check(cfg, host, bufs, top_p=kw.get("top_p"), n_sink=kw.get("n_sink"), n_recent=kw.get("n_recent"),
                   k_min=kw.get("k_min"))


def test_prefill_pipeline_with_permutation(gpu):
    cfg = I.small_prefill(name="pipe-perm", L=2048, hq=8, hkv=2, d=128, block=64, top_p=0.9, seed=13,
                          heavy_hitters=True, segment=512)
    q, k, v = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    host, dev = upload_prefill(cfg, gpu, perm[None])
    bufs = gpu_prefill(cfg, dev, perm_dev=dev[3])
    pipeline_check(cfg, host, bufs, perm=perm[None])


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_pipeline_fp32_with_permutation(gpu, d):
    """fp32 inputs with a segment permutation: pooling through the permutation and the fp32 rows
    kernel's permuted history reads."""
    cfg = I.small_prefill(name=f"pipe-perm-f32-d{d}", L=700, hq=4, hkv=2, d=d, block=32, top_p=0.9, seed=37,
                          heavy_hitters=True, segment=128, dtype="f32")
    q, k, v = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    host, dev = upload_prefill(cfg, gpu, perm[None])
    bufs = gpu_prefill(cfg, dev, perm_dev=dev[3])
    pipeline_check(cfg, host, bufs, perm=perm[None])


def test_keep_all_is_dense(gpu):
    cfg = I.small_prefill(name="dense", L=1024, hq=8, hkv=2, d=128, block=64, top_p=1.0, seed=17)
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev)
    assert torch.equal(bufs.cnt.cpu(), torch.arange(1, cfg.nb + 1, dtype=torch.int32).expand(1, 2, cfg.nb))
    q, k, v = host
    o_ref, _ = oracle.attend_prefill(q[0], k[0], v[0], [{i: np.arange(i + 1) for i in range(cfg.nb)}] * 2,
                                     cfg.block, 1 / math.sqrt(cfg.d))
    err = P.max_abs(bufs.o.float().cpu().numpy()[0], o_ref)
    log("dense max|dO|", err)
    assert err <= P.BF16_ATOL


def test_deterministic_and_in_bounds(gpu):
    cfg = I.small_prefill(name="det", L=1500, hq=8, hkv=2, d=128, block=64, top_p=0.9, seed=19)
    host, dev = upload_prefill(cfg, gpu)
    desc = B.prefill_desc(dev[0], dev[1], cfg.block, cfg.top_p)
    runs = []
    for _ in range(2):
        bufs = B.alloc_prefill(desc, gpu)
        pad = 4096
        o_full = torch.full((bufs.o.numel() + pad,), 7.0, dtype=torch.bfloat16, device=gpu)
        bufs.o = o_full[:bufs.o.numel()].view(bufs.o.shape)
        i_full = torch.full((bufs.idx.numel() + pad,), 12345, dtype=torch.int32, device=gpu)
        bufs.idx = i_full[:bufs.idx.numel()].view(bufs.idx.shape)
        B.prefill(dev[0], dev[1], dev[2], cfg.block, cfg.top_p, bufs=bufs)
        torch.cuda.synchronize()
        assert torch.all(o_full[-pad:] == 7.0) and torch.all(i_full[-pad:] == 12345)
        runs.append((bufs.o.clone(), bufs.idx.clone(), bufs.cnt.clone(), bufs.lse.clone()))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


# ----------------------------------------------------------------- the five workloads
def test_c1_tiny_fp32(gpu):
    cfg = I.C1
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev)
    rep, err = pipeline_check(cfg, host, bufs)
    assert err <= P.F32_ATOL


def test_c2_gqa_prefill_full(gpu):
    cfg = I.C2
    t0 = time.time()
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev)
    # every KV head, a seeded sample of query blocks (always the first two and the last)
    rng = np.random.default_rng([cfg.seed, 5])
    blocks = sorted({0, 1, cfg.nb - 1} | set(rng.choice(cfg.nb, 29, replace=False).tolist()))
    pairs = [(0, g, i) for g in range(cfg.hkv) for i in blocks]
    pipeline_check(cfg, host, bufs, pairs=pairs)
    log("c2 seconds", time.time() - t0)


def _sample_pairs(cfg, n):
    rng = np.random.default_rng([cfg.seed, 99])
    blocks = I.oracle_query_blocks(cfg) if cfg.oracle_qblocks else np.arange(cfg.nb)
    out = []
    for j, i in enumerate(blocks):
        out.append((0, int(rng.integers(cfg.hkv)), int(i)))
    if n < len(out):
        keep = rng.choice(len(out), n, replace=False)
        must = [k for k, p in enumerate(out) if p[2] in (0, 1, cfg.nb - 1)]
        out = [out[k] for k in sorted(set(keep.tolist()) | set(must))]
    return out


def test_c3_heavy_hitter_permuted_prefill(gpu):
    cfg = I.C3
    t0 = time.time()
    q, k, v = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    log("perm seconds", time.time() - t0)
    host, dev = upload_prefill(cfg, gpu, perm[None])
    bufs = gpu_prefill(cfg, dev, perm_dev=dev[3])
    pairs = _sample_pairs(cfg.with_(oracle_qblocks=24), 24)
    pipeline_check(cfg, host, bufs, perm=perm[None], pairs=pairs)
    log("c3 seconds", time.time() - t0)


def test_c5_long_prefill_sampled(gpu):
    cfg = I.C5
    t0 = time.time()
    host, dev = upload_prefill(cfg, gpu)
    bufs = gpu_prefill(cfg, dev)
    log("c5 gpu done", time.time() - t0)
    # scores on 64 seeded query blocks (all KV heads) are checked inside; outputs on one KV head each
    pairs = _sample_pairs(cfg, 64)
    pipeline_check(cfg, host, bufs, pairs=pairs, check_scores=True)
    log("c5 seconds", time.time() - t0)


# ----------------------------------------------------------------- decode
def decode_check(cfg, D, bufs):
    go = bufs.o.float().cpu().numpy()
    glse = bufs.lse.cpu().numpy()
    gl = bufs.idx.cpu().numpy()[:, 0, 0]
    gc = bufs.cnt.cpu().numpy()[:, 0, 0]
    rep = P.SelectionReport()
    worst = worst_lse = 0.0
    scale = 1 / math.sqrt(cfg.d)
    for b in range(cfg.batch):
        s = oracle.indexer_scores(D["idx_q"][b], D["idx_w"][b], D["idx_k"][b])
        P.compare_selection(rep, gl[b, :gc[b]], s, oracle.decode_forced(cfg.nt, cfg.n_sink, cfg.n_recent),
                            cfg.top_p, cfg.k_min, b)
        o_ref, lse_ref = oracle.attend_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], gl[b, :gc[b]],
                                              cfg.block, cfg.T, scale)
        worst = max(worst, P.max_abs(go[b], o_ref))
        worst_lse = max(worst_lse, P.max_abs(glse[b], lse_ref))
    log(cfg.name, rep, "kept", gc.tolist(), "of", cfg.nt, f"max|dO|={worst:.3g} max|dLSE|={worst_lse:.3g}")
    assert not rep.violations, rep.violations[:5]
    assert worst <= P.BF16_ATOL
    assert worst_lse <= 1e-2


def run_decode(cfg, D, gpu):
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], dev["idx_k"], cfg.block,
                    cfg.top_p, n_sink=cfg.n_sink, n_recent=cfg.n_recent, k_min=cfg.k_min)
    torch.cuda.synchronize()
    return bufs


@pytest.mark.parametrize("kw", [dict(batch=2, T=16 * 1000 + 5), dict(batch=3, T=4096, hq=16, hkv=2, d=64),
                                dict(batch=2, T=2000, hq=8, hkv=8), dict(batch=1, T=10),
                                dict(batch=2, T=5000, top_p=1.0), dict(batch=2, T=5000, top_p=0.0, k_min=7),
                                # 400 kept blocks x 64 (sequence, KV head) pairs: more work units than the
                                # workgroups launched, several blocks per wave
                                dict(batch=8, T=16 * 400, top_p=1.0),
                                dict(batch=2, T=64 * 300 + 17, block=64),    # larger blocks, ragged last block
                                dict(batch=3, T=32 * 500, block=32, top_p=0.8),
                                dict(batch=2, T=3000, hq=8, hkv=4),              # two query heads per KV head
                                dict(batch=2, T=16 * 700 + 3, n_sink=2, n_recent=3, top_p=0.7),
                                dict(batch=2, T=4000, n_sink=0, n_recent=1, hq=16, hkv=2),
                                dict(batch=2, T=4000, n_sink=1, n_recent=0, top_p=0.5)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_decode_small(gpu, kw):
    cfg = I.C4.with_(name="dec", seed=23, **kw)
    D = I.decode_inputs(cfg)
    bufs = run_decode(cfg, D, gpu)
    decode_check(cfg, D, bufs)


def test_decode_attention_on_host_lists(gpu):
    """Decode attention on kept lists drawn on the host (not by the select
    kernel): an empty list (O = 0, LSE = -inf by the library's convention), the
    ragged last block alone, a sparse random list and every block."""
    cfg = I.C4.with_(name="declists", seed=29, batch=4, T=16 * 300 + 9)
    D = I.decode_inputs(cfg)
    nt = cfg.nt
    rng = np.random.default_rng(31)
    lists = [np.zeros(0, np.int64), np.array([nt - 1]), np.sort(rng.choice(nt, 37, replace=False)), np.arange(nt)]
    dev = {k: P.to_dev(D[k], "bf16", gpu) for k in ("q", "k_cache", "v_cache")}
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.alloc_decode(desc, gpu)
    idx = np.full((cfg.batch, 1, 1, nt), -1, np.int32)
    for b, kl in enumerate(lists):
        idx[b, 0, 0, :len(kl)] = kl
    bufs.idx.copy_(torch.from_numpy(idx))
    bufs.cnt.copy_(torch.tensor([len(kl) for kl in lists], dtype=torch.int32).view(cfg.batch, 1, 1))
    B.spot_sparse_attn_decode(desc, dev["q"], dev["k_cache"], dev["v_cache"], bufs.idx, bufs.cnt, bufs.o, bufs.lse,
                              bufs.workspace)
    torch.cuda.synchronize()
    go, glse = bufs.o.float().cpu().numpy(), bufs.lse.cpu().numpy()
    assert (go[0] == 0).all() and np.isneginf(glse[0]).all()
    scale = 1 / math.sqrt(cfg.d)
    for b in range(1, cfg.batch):
        o_ref, lse_ref = oracle.attend_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], lists[b], cfg.block,
                                              cfg.T, scale)
        err_o, err_l = P.max_abs(go[b], o_ref), P.max_abs(glse[b], lse_ref)
        log("declists", b, len(lists[b]), f"max|dO|={err_o:.3g} max|dLSE|={err_l:.3g}")
        assert err_o <= P.BF16_ATOL and err_l <= 1e-2


def test_c4_decode_full(gpu):
    cfg = I.C4
    t0 = time.time()
    D = I.decode_inputs(cfg)
    log("c4 inputs", time.time() - t0)
    bufs = run_decode(cfg, D, gpu)
    decode_check(cfg, D, bufs)
    log("c4 seconds", time.time() - t0)
