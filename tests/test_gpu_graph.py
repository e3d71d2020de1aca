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
