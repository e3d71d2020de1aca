"""Residual linear attention ([SPLA] §2.2-2.3) on the GPU against the float64
oracle, evaluated on the GPU's own kept lists (and, with a permutation, the
oracle's permutation given to both sides).

Window: the GPU sums in fp32 in a fixed order: a block (or cache chunk) state
over its keys, the residual over the block states, the output over d.  With
unit roundoff u = 2^-24 the error of such a sum of n terms is at most about
n u times the sum of the terms' magnitudes, and every term here is
phi(q).phi(k_t) * |v_t| summed over the keys involved (phi > 0), so
    |o_gpu - o| <= (n_terms * u + 2^-20) * sum_t (phi(q).phi(k_t)) |v_t|
per element, with n_terms the longest chain of additions and 2^-20 covering
the two fp32 exponentials (a few ulp each).  The magnitude sum is the oracle
run on |v|.  A block added or dropped changes the output by about
1/(blocks in the sum) of that magnitude, far above the window (in decode the
magnitude is that of the whole cache: on the short caches below a block of 16
keys is 0.16-5% of it, against windows of 2.7-3.3e-4)."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P
from tests.test_gpu_parity import gpu_prefill, log, upload_prefill

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
EXP_SLACK = 2.0 ** -20
SPAN = 4096   # keys per cache chunk state in decode


def _check(name, got, ref, mag, n_terms):
    tol = n_terms * U + EXP_SLACK
    err = np.abs(np.asarray(got, np.float64) - ref)
    assert np.isfinite(got).all(), name
    ratio = float(np.max(err / np.maximum(mag, 1e-300))) if err.size else 0.0
    log(name, f"max|d|={float(err.max()) if err.size else 0.0:.3g}", f"max |d|/mag={ratio:.3g}", f"window {tol:.3g}")
    assert np.all(err <= tol * mag), (name, ratio, tol)


def _prefill_case(cfg, gpu, top_p=None, perm=None, qblocks=None, **sel):
    """GPU pipeline lists, then the residual on the GPU and in the oracle for every sequence of the batch."""
    host, dev = upload_prefill(cfg, gpu, perm)
    bufs = gpu_prefill(cfg, dev, perm_dev=dev[3], top_p=top_p, **sel)
    desc = B.prefill_desc(dev[0], dev[1], cfg.block, cfg.top_p if top_p is None else top_p,
                          segment=cfg.segment if perm is not None else 0, n_sink=sel.get("n_sink", cfg.n_sink),
                          n_recent=sel.get("n_recent", cfg.n_recent))
    rb = B.rla_prefill(desc, dev[0], dev[1], dev[2], bufs.idx, bufs.cnt, perm=dev[3])
    torch.cuda.synchronize()
    q, k, v = host
    all_lists = P.kept_lists(bufs.idx, bufs.cnt)
    o_all = rb.o_rla.cpu().numpy()
    qb = np.arange(cfg.nb) if qblocks is None else np.asarray(qblocks)
    seg = cfg.segment if perm is not None else 0
    rows = np.concatenate([np.arange(i * cfg.block, min((i + 1) * cfg.block, cfg.L)) for i in qb])
    got, ref, mag = [], [], []
    for b in range(cfg.batch):
        pm = None if perm is None else perm[b]
        r = oracle.spot_oracle.rla_prefill(q[b], k[b], v[b], all_lists[b], cfg.block, segment=seg, perm=pm,
                                           qblocks=qb)
        m = oracle.spot_oracle.rla_prefill(q[b], k[b], np.abs(v[b]), all_lists[b], cfg.block, segment=seg,
                                           perm=pm, qblocks=qb)
        got.append(o_all[b][:, rows])
        ref.append(r[:, rows])
        mag.append(m[:, rows])
    return np.stack(got), np.stack(ref), np.stack(mag), all_lists


@pytest.mark.parametrize("kw", [dict(L=256, hq=1, hkv=1, d=64, dtype="f32", block=16, seed=1),
                                dict(L=1000, hq=8, hkv=2, d=128, block=64, seed=21),
                                dict(L=777, hq=4, hkv=1, d=64, block=32, seed=22),
                                dict(L=640, hq=16, hkv=2, d=128, block=128, seed=23, top_p=0.6)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_rla_prefill_small(gpu, kw):
    cfg = I.small_prefill(name="rla", **kw)
    got, ref, mag, _ = _prefill_case(cfg, gpu)
    _check(cfg.name + str(kw), got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_with_permutation(gpu):
    cfg = I.small_prefill(name="rla-perm", L=2048, hq=8, hkv=2, d=128, block=64, segment=512, seed=24,
                          heavy_hitters=True)
    q, k, _ = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    got, ref, mag, _ = _prefill_case(cfg, gpu, perm=perm[None])
    _check("rla permuted", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_batch_and_sink(gpu):
    """Two sequences (batch indexing of states, lists and outputs) and no sink block."""
    cfg = I.small_prefill(name="rla-b2", L=900, hq=8, hkv=2, d=128, block=64, seed=26, batch=2)
    got, ref, mag, _ = _prefill_case(cfg, gpu, n_sink=0)
    _check("rla batch 2, no sink", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_fp32_with_permutation(gpu):
    cfg = I.small_prefill(name="rla-f32-perm", L=512, hq=4, hkv=2, d=64, dtype="f32", block=32, segment=128,
                          seed=27, heavy_hitters=True)
    q, k, _ = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    got, ref, mag, _ = _prefill_case(cfg, gpu, perm=perm[None])
    _check("rla fp32 permuted", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_c3_sampled(gpu):
    """The heavy-hitter workload with its segment permutation at full size, three query blocks of later
    segments checked."""
    cfg = I.C3
    q, k, _ = I.prefill_inputs(cfg)
    perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, 1 / math.sqrt(cfg.d))
    del q, k
    got, ref, mag, _ = _prefill_case(cfg, gpu, perm=perm[None], qblocks=[17, 40, 63])
    _check("rla C3 permuted", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_keep_all_is_zero(gpu):
    cfg = I.small_prefill(name="rla-all", L=512, hq=8, hkv=2, d=128, block=64, seed=25)
    got, ref, mag, _ = _prefill_case(cfg, gpu, top_p=1.0)
    assert np.all(ref == 0.0) and np.all(got == 0.0)


def test_rla_prefill_c2_sampled(gpu):
    """The GQA workload at full size (every block state and residual on the
    GPU), checked on four query blocks."""
    cfg = I.C2
    got, ref, mag, _ = _prefill_case(cfg, gpu, qblocks=[0, 1, 64, cfg.nb - 1])
    _check("rla C2", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def test_rla_prefill_c5_sampled(gpu):
    """The long-context workload at full size, checked on three early query
    blocks (the oracle's cost grows with the prefix)."""
    cfg = I.C5
    got, ref, mag, _ = _prefill_case(cfg, gpu, qblocks=[1, 2, 21])
    _check("rla C5", got, ref, mag, cfg.block + cfg.nb + cfg.d)


def _decode_case(cfg, gpu, seqs=None, top_p=None):
    D = I.decode_inputs(cfg)
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    p = cfg.top_p if top_p is None else top_p
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], dev["idx_k"], cfg.block, p)
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, p, cfg.h_idx, cfg.d_idx)
    state = B.rla_decode_state(desc, dev["k_cache"], dev["v_cache"])
    o = B.rla_decode(desc, dev["q"], dev["k_cache"], dev["v_cache"], state, bufs.idx, bufs.cnt)
    torch.cuda.synchronize()
    got = o.cpu().numpy()
    gl, gc = bufs.idx.cpu().numpy()[:, 0, 0], bufs.cnt.cpu().numpy()[:, 0, 0]
    n_terms = SPAN + -(-cfg.T // SPAN) + 2 * cfg.d + int(gc.max()) * cfg.block + 64   # + the split partials
    for b in (range(cfg.batch) if seqs is None else seqs):
        kept = gl[b, :gc[b]]
        ref = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], kept, cfg.block, cfg.T)
        mag = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], np.abs(D["v_cache"][b]), [], cfg.block,
                                            cfg.T)
        _check(f"{cfg.name} seq {b} kept {len(kept)}", got[b], ref, mag, n_terms)
    return got


@pytest.mark.parametrize("kw", [dict(batch=2, T=2000), dict(batch=2, T=10000 + 7, hq=16, hkv=2),
                                dict(batch=1, T=4096 * 2, hq=8, hkv=8, d=64), dict(batch=3, T=300, top_p=0.5)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_rla_decode_small(gpu, kw):
    cfg = I.C4.with_(name="rla-dec", seed=41, **kw)
    _decode_case(cfg, gpu)


def test_rla_decode_c4(gpu):
    """The decode workload (batch 16, context 131072): the whole-cache state
    and the residual of every sequence on the GPU, three sequences checked."""
    _decode_case(I.C4, gpu, seqs=[0, 7, 15])


def _fused_case(cfg, gpu, seqs=None):
    """The decode attention with the residual in the same pass: O and LSE equal to the plain call's bit for
    bit, the residual against the oracle on the same lists."""
    D = I.decode_inputs(cfg)
    dev = {k: (torch.from_numpy(v).to(gpu) if k == "idx_w" else P.to_dev(v, "bf16", gpu)) for k, v in D.items()}
    bufs = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], dev["idx_k"], cfg.block,
                    cfg.top_p)
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    state = B.rla_decode_state(desc, dev["k_cache"], dev["v_cache"])
    ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_DECODE_RLA), dtype=torch.uint8, device=gpu)
    o2, lse2 = torch.empty_like(bufs.o), torch.empty_like(bufs.lse)
    o_rla = torch.empty(cfg.batch, cfg.hq, cfg.d, dtype=torch.float32, device=gpu)
    B.spot_sparse_attn_decode_rla(desc, dev["q"], dev["k_cache"], dev["v_cache"], bufs.idx, bufs.cnt, state, o2,
                                  lse2, o_rla, ws)
    torch.cuda.synchronize()
    assert torch.equal(o2, bufs.o) and torch.equal(lse2, bufs.lse)
    got = o_rla.cpu().numpy()
    gl, gc = bufs.idx.cpu().numpy()[:, 0, 0], bufs.cnt.cpu().numpy()[:, 0, 0]
    n_terms = SPAN + -(-cfg.T // SPAN) + 2 * cfg.d + int(gc.max()) * cfg.block + 64
    for b in (range(cfg.batch) if seqs is None else seqs):
        kept = gl[b, :gc[b]]
        ref = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], kept, cfg.block, cfg.T)
        mag = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], np.abs(D["v_cache"][b]), [], cfg.block,
                                            cfg.T)
        _check(f"fused {cfg.name} seq {b} kept {len(kept)}", got[b], ref, mag, n_terms)


@pytest.mark.parametrize("kw", [dict(batch=2, T=2000), dict(batch=2, T=10000 + 7, hq=16, hkv=2),
                                dict(batch=1, T=4096 * 2, hq=8, hkv=8, d=64), dict(batch=3, T=300, top_p=0.5)],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_rla_decode_fused_small(gpu, kw):
    _fused_case(I.C4.with_(name="rla-fused", seed=43, **kw), gpu)


def test_rla_decode_fused_c4(gpu):
    _fused_case(I.C4, gpu, seqs=[0, 9, 15])


def test_rla_decode_on_host_lists(gpu):
    """Both decode forms of the residual on lists drawn on the host: an empty list (the whole cache is the
    rest), the ragged last block alone, a sparse random list and every block (nothing is left: zero up to
    the window)."""
    cfg = I.C4.with_(name="rla-lists", seed=29, batch=4, T=16 * 300 + 9)
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
    state = B.rla_decode_state(desc, dev["k_cache"], dev["v_cache"])
    sep = B.rla_decode(desc, dev["q"], dev["k_cache"], dev["v_cache"], state, bufs.idx, bufs.cnt)
    ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_DECODE_RLA), dtype=torch.uint8, device=gpu)
    fused = torch.empty_like(sep)
    B.spot_sparse_attn_decode_rla(desc, dev["q"], dev["k_cache"], dev["v_cache"], bufs.idx, bufs.cnt, state, bufs.o,
                                  bufs.lse, fused, ws)
    torch.cuda.synchronize()
    n_terms = SPAN + -(-cfg.T // SPAN) + 2 * cfg.d + nt * cfg.block + 64
    for name, out in (("own pass", sep.cpu().numpy()), ("fused", fused.cpu().numpy())):
        for b, kl in enumerate(lists):
            ref = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], D["v_cache"][b], kl, cfg.block, cfg.T)
            mag = oracle.spot_oracle.rla_decode(D["q"][b], D["k_cache"][b], np.abs(D["v_cache"][b]), [], cfg.block,
                                                cfg.T)
            _check(f"host lists {name} seq {b} kept {len(kl)}", out[b], ref, mag, n_terms)
