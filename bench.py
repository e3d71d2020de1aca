"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = the whole prefill path on the GQA workload (L=8192, 32 query / 8 KV
heads, d=128, bf16, block 64, top-p 0.9): mean-pool block scores, top-p
selection, sparse attention.  Inputs are resident in HBM before timing.  The
step is timed two ways over K steps: its four launches issued call by call on
the stream, and captured once as a HIP graph and replayed; `ms_per_step` is
the faster of the two (`config.step_launch` names it, both times are in
`config`).

Prints one JSON line.  `value` is effective TFLOP/s over kept blocks
(4*d*visible query-key pairs per step / step time).  The line also carries the
roofline of the dominant kernel (the attention kernel, bf16 MFMA bound), a
decode measurement on the sparse-decode workload (batch 16, context 131072,
KV GB/s against HBM) and the float64 oracle timed on a bounded sample on the
host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "effective TFLOP/s sparse prefill (kept blocks); decode KV GB/s; % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-early-stop", action="store_true", help="skip the early-stopping measurement")
    ap.add_argument("--es-tau", type=float, default=0.01, help="early-stopping threshold tau")
    ap.add_argument("--no-taylor", action="store_true", help="skip the Taylor-score measurement")
    ap.add_argument("--cpu-sample-blocks", type=int, default=0, help="0: every query block")
    ap.add_argument("--workload", default="gqa-bf16-L8192",
                    help="prefill workload of the step: gqa-bf16-L8192 (default), heavy-perm-bf16-L32768 "
                         "(permutation generated on the GPU inside the step), long-bf16-L131072, tiny-fp32-L256")
    return ap.parse_args()


# ----------------------------------------------------------------- work accounting
def prefill_visible_pairs(idx: np.ndarray, cnt: np.ndarray, L: int, B: int, G: int) -> np.ndarray:
    """Visible (query, key) pairs per (batch, KV head, query block), summed over
    the G query heads: kept blocks before the diagonal count |blk(j)| keys per
    row, the diagonal counts r - iB + 1 keys for row r."""
    nb = idx.shape[-1]
    bs = np.minimum(B, L - np.arange(nb) * B).astype(np.int64)
    bs_ext = np.concatenate([bs, [0]])
    safe = np.where(idx >= 0, idx, nb)
    keys = bs_ext[safe].sum(axis=-1)                                   # keys of all kept blocks
    i_of_row = np.arange(nb)
    diag_kept = (idx == i_of_row[:, None]).any(axis=-1)
    nrow = bs                                                          # rows of query block i
    full = keys - np.where(diag_kept, nrow, 0)
    pairs = nrow * full + np.where(diag_kept, nrow * (nrow + 1) // 2, 0)
    return G * pairs


def source_digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file: str, key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(key)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest(kernel_file):
        return None
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------- prefill
def prefill_data(args, torch, I):
    """Host and device inputs of the prefill workload (made once, shared by its measurements)."""
    cfg = {c.name: c for c in (I.C1, I.C2, I.C3, I.C5)}[args.workload]
    q, k, v = I.prefill_inputs(cfg)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    dq, dk, dv = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    return cfg, (q, k), (dq, dk, dv)


def settle(torch, fn, ms=30.0):
    """Run fn untimed until about `ms` of GPU time has passed: after the host has kept the GPU idle (input
    generation), its clock takes some milliseconds of work to come back up."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done = 0.0
    while done < ms:
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)


def bench_prefill(args, torch, B, I, data, score_kind=None, top_p=None):
    cfg, (q, k), (dq, dk, dv) = data
    if top_p is not None:
        cfg = cfg.with_(top_p=top_p)
    score_kind = B.SPOT_SCORE_MEANPOOL if score_kind is None else score_kind
    dev = torch.device("cuda:0")
    desc = B.prefill_desc(dq, dk, cfg.block, cfg.top_p, segment=cfg.segment, score_kind=score_kind)
    bufs = B.alloc_prefill(desc, dev)
    perm = perm_ws = None
    if cfg.segment:
        perm = torch.empty(dk.shape[0], dk.shape[1], dk.shape[2], dtype=torch.int32, device=dev)
        perm_ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_KEY_PERMUTATION), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if perm is not None:
            B.spot_key_permutation(desc, dq, dk, perm, None, perm_ws)
        if ev is not None:
            ev[3].record()
        B.spot_block_score(desc, dq, dk, perm, None, None, None, bufs.scores, bufs.workspace)
        B.spot_select_topp(desc, bufs.scores, bufs.idx, bufs.cnt)
        if ev is not None:
            ev[1].record()
        B.spot_sparse_attn_prefill(desc, dq, dk, dv, perm, bufs.idx, bufs.cnt, bufs.o, bufs.lse)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # K steps back to back, launched one call at a time
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_step_eager = t0.elapsed_time(t1) / args.steps

    # the same step captured once as a HIP graph and replayed K times
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step_graph = t0.elapsed_time(t1) / args.steps
    # the same work either way: report the faster launch mode
    ms_step = min(ms_step_graph, ms_step_eager)
    step_launch = "hip_graph_replay" if ms_step_graph <= ms_step_eager else "stream_launches"

    # per-kernel split with events on the launch stream (same work again)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms_perm = float(np.mean([e[0].elapsed_time(e[3]) for e in evs])) if perm is not None else 0.0
    ms_sel = float(np.mean([e[3].elapsed_time(e[1]) for e in evs]))
    ms_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    idx = bufs.idx.cpu().numpy()
    cnt = bufs.cnt.cpu().numpy()
    G = cfg.hq // cfg.hkv
    pairs = prefill_visible_pairs(idx, cnt, cfg.L, cfg.block, G)
    flops = 4.0 * cfg.d * float(pairs.sum())
    dense_pairs = G * cfg.hkv * cfg.L * (cfg.L + 1) / 2
    kept_fraction = float(pairs.sum()) / dense_pairs

    attn_file = os.path.join(ROOT, "block_sparse_attention_amd", "csrc", "kernels", "prefill.hip")
    achieved = flops / (ms_attn * 1e-3) / 1e12
    if cfg.dtype == "bf16":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                "traffic": load_traffic(attn_file, f"prefill_mfma_kernel@{cfg.name}"),
                "kernel": f"prefill_mfma_kernel<{cfg.d},8,1,{'true' if cfg.segment else 'false'},false,"
                          f"{'true' if cfg.nb <= 2048 else 'false'}>",
                "flop_per_launch": flops, "avg_launch_ms": round(ms_attn, 4)}
    else:   # the fp32 row kernel on a 256-token input is launch-latency bound
        roof = {"bound": "latency", "achieved": round(achieved, 4), "peak": None, "unit": "TFLOP/s", "frac": None,
                "traffic": None, "kernel": "prefill_rows_kernel<float,64>", "flop_per_launch": flops,
                "avg_launch_ms": round(ms_attn, 4)}
    res = dict(
        cfg=cfg, ms_step=ms_step, ms_step_eager=ms_step_eager, ms_step_graph=ms_step_graph, step_launch=step_launch,
        ms_perm=ms_perm, ms_sel=ms_sel, ms_attn=ms_attn,
        flops=flops, kept_fraction=kept_fraction, value=flops / (ms_step * 1e-3) / 1e12, roofline=roof,
        host=(q, k, None), idx=idx, cnt=cnt,
    )
    return res


# ----------------------------------------------------------------- decode
def bench_decode(args, torch, B, I, mxfp4=False):
    cfg = I.C4
    dev = torch.device("cuda:0")
    D = I.decode_inputs(cfg)
    up = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
    q, kc, vc = up(D["q"]), up(D["k_cache"]), up(D["v_cache"])
    iq, ik = up(D["idx_q"]), up(D["idx_k"])
    iw = torch.from_numpy(D["idx_w"]).to(dev)
    del D
    desc = B.decode_desc(q, kc, cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.alloc_decode(desc, dev)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    if mxfp4:   # the cache is encoded once, when keys are appended (outside the step)
        kcodes, kscales = B.quantize_indexer_keys(ik, cfg.block, cfg.T)
        torch.cuda.synchronize()
        del ik

    def score():
        if mxfp4:
            B.spot_indexer_score_mxfp4(desc, iq, iw, kcodes, kscales, bufs.scores)
        else:
            B.spot_block_score(desc, None, None, None, iq, iw, ik, bufs.scores)

    def step(ev):
        ev[0].record()
        score()
        ev[3].record()
        B.spot_select_topp(desc, bufs.scores, bufs.idx, bufs.cnt)
        ev[1].record()
        B.spot_sparse_attn_decode(desc, q, kc, vc, bufs.idx, bufs.cnt, bufs.o, bufs.lse, bufs.workspace)
        ev[2].record()

    settle(torch, lambda: step([torch.cuda.Event(enable_timing=True) for _ in range(4)]))
    for _ in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(4)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        flush.sum()               # read 512 MB between steps (outside the events): evicts the 256 MB last-level cache
        step(e)
    torch.cuda.synchronize()
    ms_front = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_scan = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    ms_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_step_eager = ms_front + ms_attn

    # the step's four launches as one HIP graph, replayed with a cold cache each time
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        score()
        B.spot_select_topp(desc, bufs.scores, bufs.idx, bufs.cnt)
        B.spot_sparse_attn_decode(desc, q, kc, vc, bufs.idx, bufs.cnt, bufs.o, bufs.lse, bufs.workspace)
    graph.replay()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in gev:
        flush.sum()
        e[0].record()
        graph.replay()
        e[1].record()
    torch.cuda.synchronize()
    ms_step_graph = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]))
    # the same work either way: report the faster launch mode
    ms_step = min(ms_step_graph, ms_step_eager)
    step_launch = "hip_graph_replay" if ms_step_graph <= ms_step_eager else "stream_launches"
    cnt = bufs.cnt.cpu().numpy()[:, 0, 0]
    idx = bufs.idx.cpu().numpy()[:, 0, 0]
    bs = np.minimum(cfg.block, cfg.T - np.arange(cfg.nt) * cfg.block)
    kept_keys = np.array([bs[idx[b, :cnt[b]]].sum() for b in range(cfg.batch)], dtype=np.float64)
    kv_bytes = float(kept_keys.sum()) * cfg.hkv * cfg.d * 2 * 2
    scan_bytes = cfg.batch * cfg.nt * cfg.h_idx * cfg.d_idx * (0.5 + 1.0 / 32 if mxfp4 else 2.0)
    qo_bytes = cfg.batch * cfg.hq * cfg.d * 2 * 2.0 + cfg.batch * cfg.h_idx * (cfg.d_idx * 2 + 4)
    step_bytes = kv_bytes + scan_bytes + qo_bytes
    attn_gbs = (kv_bytes + qo_bytes) / (ms_attn * 1e-3) / 1e9
    return dict(
        workload=cfg.name, indexer_cache="mxfp4" if mxfp4 else "bf16",
        value=round(step_bytes / (ms_step * 1e-3) / 1e9, 1), unit="GB/s",
        ms_per_step=round(ms_step, 4), step_launch=step_launch, ms_per_step_stream_launches=round(ms_step_eager, 4),
        ms_per_step_graph_replay=round(ms_step_graph, 4), ms_score_select=round(ms_front, 4), ms_indexer_scan=round(ms_scan, 4),
        indexer_scan_gbs=round(scan_bytes / (ms_scan * 1e-3) / 1e9, 1), indexer_scan_bytes=scan_bytes,
        ms_attention=round(ms_attn, 4),
        kept_fraction=round(float(kept_keys.sum()) / (cfg.batch * cfg.T), 4), bytes_per_step=step_bytes,
        roofline={"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "kernel": "decode_split_kernel<128,4>+combine",
                  "traffic": load_traffic(os.path.join(ROOT, "block_sparse_attention_amd", "csrc", "kernels",
                                                       "decode.hip"), f"decode_split_kernel@{cfg.name}"),
                  "bytes_per_launch": kv_bytes + qo_bytes},
    )


# ----------------------------------------------------------------- early stopping
def bench_early_stop(args, torch, B, I):
    """Early-stopped prefill on the heavy-hitter workload (L=32768, segment
    2048): key permutation, block scores, history visiting order and the
    early-stopped attention, captured as one HIP graph."""
    cfg = I.C3
    dev = torch.device("cuda:0")
    q, k, v = I.prefill_inputs(cfg)
    dq = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    dk = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    dv = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    del q, k, v
    tau = args.es_tau
    desc = B.prefill_desc(dq, dk, cfg.block, 1.0, segment=cfg.segment)
    bufs = B.alloc_prefill_early_stop(desc, dev)
    perm = torch.empty(dk.shape[0], dk.shape[1], dk.shape[2], dtype=torch.int32, device=dev)
    perm_ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_KEY_PERMUTATION), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        B.spot_key_permutation(desc, dq, dk, perm, None, perm_ws)
        if ev is not None:
            ev[1].record()
        B.spot_block_score(desc, dq, dk, perm, None, None, None, bufs.scores, bufs.workspace)
        B.spot_order_history(desc, bufs.scores, bufs.order, bufs.cnt)
        if ev is not None:
            ev[2].record()
        B.spot_sparse_attn_prefill_early_stop(desc, tau, dq, dk, dv, perm, bufs.order, bufs.cnt, bufs.o, bufs.lse,
                                              bufs.nused)
        if ev is not None:
            ev[3].record()

    settle(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms_perm = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_front = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_attn = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    # work: each row's own-segment keys (causal) plus the history blocks it took
    nused = bufs.nused.cpu().numpy()[0].astype(np.int64)          # (hq, L)
    L, Bk, S = cfg.L, cfg.block, cfg.segment
    r = np.arange(L)
    own = r - (r // S) * S + 1
    pairs_row = own[None, :] + nused * Bk
    flops = 4.0 * cfg.d * float(pairs_row.sum())
    dense_pairs = cfg.hq * L * (L + 1) / 2
    # keys the workgroups walked: a workgroup (256 packed rows of one KV head
    # and query block) runs until its last row has stopped
    G = cfg.hq // cfg.hkv
    packed = nused.reshape(cfg.hkv, G, cfg.nb, Bk).transpose(0, 2, 1, 3).reshape(cfg.hkv, cfg.nb, G * Bk)
    own_packed = np.tile(own.reshape(cfg.nb, Bk), (1, G))                 # (nb, G*Bk)
    walked = 0.0
    for c0 in range(0, G * Bk, 256):
        part = packed[..., c0:c0 + 256]
        walked += float((own_packed[None, :, c0:c0 + 256] + part.max(axis=-1, keepdims=True) * Bk).sum())
    achieved = flops / (ms_attn * 1e-3) / 1e12

    # top-p selection at the workload's p with history means over the permuted keys and without the
    # permutation: how many blocks the same mass needs in each case (outside the timed steps)
    kept = {}
    for name, seg, pm in (("with_permutation", cfg.segment, perm), ("without_permutation", 0, None)):
        d2 = B.prefill_desc(dq, dk, cfg.block, cfg.top_p, segment=seg)
        b2 = B.alloc_prefill(d2, dev)
        B.spot_block_score(d2, dq, dk, pm, None, None, None, b2.scores, b2.workspace)
        B.spot_select_topp(d2, b2.scores, b2.idx, b2.cnt)
        torch.cuda.synchronize()
        kept[name] = int(b2.cnt.cpu().numpy().astype(np.int64).sum())
        del b2
    cand = cfg.hkv * cfg.nb * (cfg.nb + 1) // 2
    top_p_blocks = {"top_p": cfg.top_p, "candidate_blocks": cand, **kept,
                    "change": round(kept["with_permutation"] / kept["without_permutation"] - 1.0, 4)}
    return dict(
        workload=cfg.name, tau=tau, value=round(flops / (ms_step * 1e-3) / 1e12, 2), unit="TFLOP/s",
        top_p_kept_blocks=top_p_blocks,
        ms_per_step=round(ms_step, 4), ms_key_permutation=round(ms_perm, 4), ms_score_order=round(ms_front, 4),
        ms_attention=round(ms_attn, 4), taken_fraction=round(float(pairs_row.sum()) / dense_pairs, 4),
        walked_fraction=round(walked / dense_pairs, 4), mean_history_blocks=round(float(nused.mean()), 2),
        flop_per_step=flops,
        roofline={"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                  "kernel": "prefill_mfma_kernel<128,8,1,true,true,true> (early stop)", "avg_launch_ms": round(ms_attn, 4),
                  "traffic": load_traffic(os.path.join(ROOT, "block_sparse_attention_amd", "csrc", "kernels",
                                                       "prefill.hip"),
                                          f"prefill_mfma_kernel_early_stop@{cfg.name}"),
                  "walked_tflops": round(4.0 * cfg.d * walked / (ms_attn * 1e-3) / 1e12, 2)},
    )


def bench_history_map(args, torch, B, I):
    """Early-stopped prefill on representative-query history maps on the
    heavy-hitter workload: maps of every segment, then the attention walking
    them, captured as one HIP graph."""
    cfg = I.C3
    dev = torch.device("cuda:0")
    q, k, v = I.prefill_inputs(cfg)
    dq = torch.from_numpy(q).to(torch.bfloat16).to(dev)
    dk = torch.from_numpy(k).to(torch.bfloat16).to(dev)
    dv = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    del q, k, v
    tau = args.es_tau
    desc = B.prefill_desc(dq, dk, cfg.block, 1.0, segment=cfg.segment)
    bufs = B.alloc_prefill_early_stop(desc, dev)
    nseg = -(-cfg.L // cfg.segment)
    hmap = torch.empty(dk.shape[0], dk.shape[1], nseg, cfg.L, dtype=torch.int32, device=dev)
    ws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_HISTORY_MAP), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        B.spot_history_map(desc, dq, dk, hmap, ws)
        if ev is not None:
            ev[1].record()
        B.spot_sparse_attn_prefill_history_map(desc, tau, dq, dk, dv, hmap, bufs.o, bufs.lse, bufs.nused)
        if ev is not None:
            ev[2].record()

    settle(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms_map = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    nused = bufs.nused.cpu().numpy()[0].astype(np.int64)
    r = np.arange(cfg.L)
    own = r - (r // cfg.segment) * cfg.segment + 1
    flops = 4.0 * cfg.d * float((own[None, :] + nused * cfg.block).sum())
    dense_pairs = cfg.hq * cfg.L * (cfg.L + 1) / 2
    achieved = flops / (ms_attn * 1e-3) / 1e12
    return dict(
        workload=cfg.name, tau=tau, value=round(flops / (ms_step * 1e-3) / 1e12, 2), unit="TFLOP/s",
        ms_per_step=round(ms_step, 4), ms_history_map=round(ms_map, 4), ms_attention=round(ms_attn, 4),
        taken_fraction=round(flops / (4.0 * cfg.d) / dense_pairs, 4), mean_history_runs=round(float(nused.mean()), 2),
        flop_per_step=flops,
        roofline={"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                  "kernel": "prefill_mfma_kernel<128,8,1,true,true,true> (early stop, history maps)",
                  "avg_launch_ms": round(ms_attn, 4)},
    )


# ----------------------------------------------------------------- measured ceilings
def measured_ceilings(torch):
    """Context for the rooflines: a dense bf16 GEMM (8192^3, the vendor BLAS
    through torch) and a 1 GiB device-to-device copy on the same GPU."""
    dev = torch.device("cuda:0")
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
    del a, b, c
    src = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9
    return {"bf16_gemm_8192_tflops": round(gemm, 1), "device_copy_1gib_gbs": round(copy, 1)}


# ----------------------------------------------------------------- oracle on the host
def cpu_baseline(res, I, sample_blocks: int):
    """The float64 oracle on the host over the workload (or a seeded sample of
    query blocks on the long ones): pool and score every block, select and
    attend the sampled query blocks, permutation included when the workload
    uses one."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    cfg = res["cfg"]
    q, k, v = I.prefill_inputs(cfg)
    if sample_blocks <= 0 and cfg.L > 16384:
        sample_blocks = 8
    if sample_blocks <= 0 or sample_blocks >= cfg.nb:
        blocks = list(range(cfg.nb))
    else:
        rng = np.random.default_rng([cfg.seed, 1234])
        blocks = sorted({cfg.nb - 1} | set(rng.choice(cfg.nb, sample_blocks - 1, replace=False).tolist()))
    scale = 1 / math.sqrt(cfg.d)
    t0 = time.time()
    perm = None
    if cfg.segment:
        perm, _ = oracle.key_permutation(q[0], k[0], cfg.block, cfg.segment, scale)
    out = oracle.prefill(q[0], k[0], v[0], cfg.block, cfg.top_p, qblocks=blocks, segment=cfg.segment, perm=perm)
    dt = time.time() - t0
    G = cfg.hq // cfg.hkv
    nb = cfg.nb
    idx = np.full((1, cfg.hkv, nb, nb), -1, np.int64)
    sel = np.zeros((1, cfg.hkv, nb), bool)
    for g in range(cfg.hkv):
        for i in blocks:
            kl = out["kept"][g][i]
            idx[0, g, i, :len(kl)] = kl
            sel[0, g, i] = True
    pairs = prefill_visible_pairs(idx, None, cfg.L, cfg.block, G)
    flops = 4.0 * cfg.d * float(pairs[sel].sum())
    what = "every query block" if len(blocks) == nb else f"{len(blocks)} seeded query blocks"
    cpu_model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2), "cpu_model": cpu_model, "blas_threads": int(threads),
            "sample": f"float64 NumPy oracle, whole pipeline ({'permutation, ' if cfg.segment else ''}pool and "
                      f"score every block, select and attend {what} x {cfg.hkv} KV heads of {cfg.name})"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (prefill would shard by KV head "
              "and decode by sequence, with no exchange; one GPU's share is what is timed)", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_attention_amd import binding as B
    from block_sparse_attention_amd import inputs as I
    B.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    data = prefill_data(args, torch, I)
    # the ceilings are measured first: their GEMMs and copies also bring the GPU to its working clock after the
    # host-side input generation, before the warm-up steps of the prefill step
    ceil = measured_ceilings(torch)
    print(f"[bench] measured ceilings: {ceil}", file=sys.stderr, flush=True)
    pre = bench_prefill(args, torch, B, I, data)
    # the same kernels keeping every block (p = 1): an in-house dense reference
    dense = bench_prefill(args, torch, B, I, data, top_p=1.0)
    dense_ref = {"workload": dense["cfg"].name, "top_p": 1.0, "ms_per_step": round(dense["ms_step"], 4),
                 "ms_attention": round(dense["ms_attn"], 4), "value": round(dense["value"], 2), "unit": "TFLOP/s",
                 "kept_fraction": round(dense["kept_fraction"], 4),
                 "sparse_speedup_step": round(dense["ms_step"] / pre["ms_step"], 3),
                 "sparse_speedup_attention": round(dense["ms_attn"] / pre["ms_attn"], 3)}
    del dense
    tay = None
    if not args.no_taylor:
        t = bench_prefill(args, torch, B, I, data, score_kind=B.SPOT_SCORE_TAYLOR)
        tay = {"workload": t["cfg"].name, "score": "second-order Taylor", "value": round(t["value"], 2),
               "unit": "TFLOP/s", "ms_per_step": round(t["ms_step"], 4), "ms_score_select": round(t["ms_sel"], 4),
               "ms_attention": round(t["ms_attn"], 4), "kept_fraction": round(t["kept_fraction"], 4),
               "flop_per_step": t["flops"]}
        del t
    print(f"[bench] prefill {pre['cfg'].name}: {pre['ms_step_graph']:.4f} ms/step (graph), "
          f"{pre['ms_step_eager']:.4f} ms/step (eager), attention {pre['ms_attn']:.4f} ms, "
          f"score+select {pre['ms_sel']:.4f} ms, kept {pre['kept_fraction']:.4f}", file=sys.stderr, flush=True)
    dec = dec_mx = None
    if not args.no_decode:
        dec = bench_decode(args, torch, B, I)
        print(f"[bench] decode: {dec}", file=sys.stderr, flush=True)
        dec_mx = bench_decode(args, torch, B, I, mxfp4=True)
        print(f"[bench] decode mxfp4: {dec_mx}", file=sys.stderr, flush=True)
    print(f"[bench] dense reference: {dense_ref}", file=sys.stderr, flush=True)
    if tay:
        print(f"[bench] taylor: {tay}", file=sys.stderr, flush=True)
    es = es_map = None
    if not args.no_early_stop:
        es = bench_early_stop(args, torch, B, I)
        print(f"[bench] early stop: {es}", file=sys.stderr, flush=True)
        es_map = bench_history_map(args, torch, B, I)
        print(f"[bench] early stop on history maps: {es_map}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(pre, I, args.cpu_sample_blocks)
        print(f"[bench] cpu baseline: {cpu}", file=sys.stderr, flush=True)

    cfg = pre["cfg"]
    line = {
        "metric": METRIC, "value": round(pre["value"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.L, "hq": cfg.hq, "hkv": cfg.hkv,
                   "d": cfg.d, "block": cfg.block, "top_p": cfg.top_p, "n_sink": cfg.n_sink,
                   "n_recent": cfg.n_recent, "kept_fraction": round(pre["kept_fraction"], 4),
                   "ms_attention": round(pre["ms_attn"], 4), "ms_score_select": round(pre["ms_sel"], 4),
                   "ms_per_step_stream_launches": round(pre["ms_step_eager"], 4),
                   "ms_per_step_graph_replay": round(pre["ms_step_graph"], 4), "step_launch": pre["step_launch"],
                   "segment": cfg.segment, "ms_key_permutation": round(pre["ms_perm"], 4),
                   "flop_per_step": pre["flops"]},
        "roofline": dict(pre["roofline"], measured_ceilings=ceil,
                         frac_of_measured_gemm=round(pre["roofline"]["achieved"] / ceil["bf16_gemm_8192_tflops"], 4)
                         if pre["roofline"]["peak"] else None),
        "cpu_baseline": cpu,
        "dense_reference": dense_ref,
        "decode": dec,
        "decode_mxfp4_indexer": dec_mx,
        "taylor_score": tay,
        "early_stop": es,
        "early_stop_history_map": es_map,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
