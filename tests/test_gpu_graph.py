"""The prefill and decode steps captured in a HIP graph: every replay, with
eager work and synchronisations in between, equals the eager result bit for
bit (the library issues no memset nodes and its kernels are deterministic)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_amd import binding as B
from block_sparse_attention_amd import inputs as I
from tests import parity as P

pytestmark = pytest.mark.gpu


def test_prefill_step_graph_replays_match_eager(gpu):
    cfg = I.small_prefill(name="graph", L=1500, hq=8, hkv=2, d=128, block=64, top_p=0.9, seed=29)
    q, k, v = I.prefill_inputs(cfg)
    dq, dk, dv = (P.to_dev(x, "bf16", gpu) for x in (q, k, v))
    desc = B.prefill_desc(dq, dk, cfg.block, cfg.top_p)
    eager = B.prefill(dq, dk, dv, cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (eager.scores, eager.idx, eager.cnt, eager.o, eager.lse)]
    bufs = B.alloc_prefill(desc, gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.prefill(dq, dk, dv, cfg.block, cfg.top_p, bufs=bufs)
    for rep in range(3):
        for t in (bufs.scores, bufs.o, bufs.lse):
            t.fill_(float("nan"))
        bufs.idx.fill_(-7)
        bufs.cnt.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = (bufs.scores, bufs.idx, bufs.cnt, bufs.o, bufs.lse)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"
        _ = (dq.float() * 2).sum().item()        # unrelated eager work between replays


def test_decode_step_graph_replays_match_eager(gpu):
    cfg = I.C4.with_(name="graph-dec", batch=3, T=16 * 700 + 9, seed=31)
    D = I.decode_inputs(cfg)
    dev = {kk: (torch.from_numpy(vv).to(gpu) if kk == "idx_w" else P.to_dev(vv, "bf16", gpu)) for kk, vv in D.items()}
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], dev["idx_k"], cfg.block, cfg.top_p)
    eager = B.decode(*args)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (eager.scores, eager.idx, eager.cnt, eager.o, eager.lse)]
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.alloc_decode(desc, gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.decode(*args, bufs=bufs)
    for rep in range(3):
        bufs.o.fill_(float("nan"))
        bufs.idx.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = (bufs.scores, bufs.idx, bufs.cnt, bufs.o, bufs.lse)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep}"
        _ = dev["q"].float().sum().item()


def _replay_matches(graph, outs, ref, scrub, between):
    for rep in range(3):
        scrub()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(), ref):
            assert torch.equal(a, b), f"replay {rep}"
        between()


def test_early_stop_step_graph_replays_match_eager(gpu):
    """Key permutation, mean-pooled block scores, history order and the
    early-stopped attention captured together."""
    cfg = I.small_prefill(name="graph-es", L=2048, hq=8, hkv=2, d=128, block=128, top_p=1.0, seed=37,
                          heavy_hitters=True, segment=512)
    q, k, v = I.prefill_inputs(cfg)
    dq, dk, dv = (P.to_dev(x, "bf16", gpu) for x in (q, k, v))
    perm_e = B.key_permutation(dq, dk, cfg.block, cfg.segment)
    eager = B.prefill_early_stop(dq, dk, dv, cfg.block, cfg.segment, 0.01, perm=perm_e)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (perm_e, eager.scores, eager.order, eager.cnt, eager.o, eager.lse, eager.nused)]
    desc = B.prefill_desc(dq, dk, cfg.block, 1.0, segment=cfg.segment)
    bufs = B.alloc_prefill_early_stop(desc, gpu)
    perm = torch.empty_like(perm_e)
    ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_KEY_PERMUTATION), dtype=torch.uint8, device=gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.spot_key_permutation(desc, dq, dk, perm, None, ws)
        B.prefill_early_stop(dq, dk, dv, cfg.block, cfg.segment, 0.01, perm=perm, bufs=bufs)

    def scrub():
        perm.fill_(-3)
        bufs.o.fill_(float("nan"))
        bufs.nused.fill_(-7)
        bufs.order.fill_(-7)

    _replay_matches(graph, lambda: (perm, bufs.scores, bufs.order, bufs.cnt, bufs.o, bufs.lse, bufs.nused), ref,
                    scrub, lambda: (dq.float() * 3).sum().item())


def test_taylor_prefill_graph_replays_match_eager(gpu):
    cfg = I.small_prefill(name="graph-taylor", L=1200, hq=8, hkv=2, d=64, block=32, top_p=0.8, seed=41)
    q, k, v = I.prefill_inputs(cfg)
    dq, dk, dv = (P.to_dev(x, "bf16", gpu) for x in (q, k, v))
    kind = B.SPOT_SCORE_TAYLOR
    eager = B.prefill(dq, dk, dv, cfg.block, cfg.top_p, score_kind=kind)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (eager.scores, eager.idx, eager.cnt, eager.o, eager.lse)]
    desc = B.prefill_desc(dq, dk, cfg.block, cfg.top_p, score_kind=kind)
    bufs = B.alloc_prefill(desc, gpu)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.prefill(dq, dk, dv, cfg.block, cfg.top_p, score_kind=kind, bufs=bufs)

    def scrub():
        bufs.scores.fill_(float("nan"))
        bufs.o.fill_(float("nan"))
        bufs.idx.fill_(-7)

    _replay_matches(graph, lambda: (bufs.scores, bufs.idx, bufs.cnt, bufs.o, bufs.lse), ref, scrub,
                    lambda: dq.float().sum().item())


def test_mxfp4_decode_graph_replays_match_eager(gpu):
    """Encoding of the indexer keys and the decode step on the encoding,
    captured together."""
    cfg = I.C4.with_(name="graph-mx", batch=2, T=16 * 900 + 3, seed=43)
    D = I.decode_inputs(cfg)
    dev = {kk: (torch.from_numpy(vv).to(gpu) if kk == "idx_w" else P.to_dev(vv, "bf16", gpu)) for kk, vv in D.items()}
    codes_e, scales_e = B.quantize_indexer_keys(dev["idx_k"], cfg.block, cfg.T)
    eager = B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes_e, scales_e),
                     cfg.block, cfg.top_p)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (codes_e, scales_e, eager.scores, eager.idx, eager.cnt, eager.o, eager.lse)]
    desc = B.decode_desc(dev["q"], dev["k_cache"], cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.alloc_decode(desc, gpu)
    codes, scales = torch.empty_like(codes_e), torch.empty_like(scales_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.spot_quantize_indexer_keys(desc, dev["idx_k"], codes, scales)
        B.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["idx_q"], dev["idx_w"], (codes, scales), cfg.block,
                 cfg.top_p, bufs=bufs)

    def scrub():
        codes.fill_(0xAA)
        scales.fill_(0)
        bufs.o.fill_(float("nan"))
        bufs.idx.fill_(-7)

    _replay_matches(graph, lambda: (codes, scales, bufs.scores, bufs.idx, bufs.cnt, bufs.o, bufs.lse), ref, scrub,
                    lambda: dev["q"].float().sum().item())
