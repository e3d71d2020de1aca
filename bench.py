"""Benchmark of the block-sparse attention hot path on one MI355X.

Headline step = the whole prefill path on the long-context workload
(L=131072, 32 query / 8 KV heads, d=128, bf16, block 128, top-p 0.9, 2% planted
heavy hitters): mean-pool block scores, top-p selection, sparse attention.
Inputs are resident in HBM before timing.  The step is timed two ways over K
steps: its launches issued call by call on the stream, and captured once as a
HIP graph and replayed; `ms_per_step` is the faster of the two
(`config.step_launch` names it, both times are in `config`).

Prints one JSON line.  `value` is effective TFLOP/s over kept blocks
(4*d*visible query-key pairs per step / step time).  The line also carries the
roofline of the dominant kernel (the attention kernel, bf16 MFMA bound), the
float64 oracle timed on the host cores over 64 seeded query blocks of the same
workload, and under `configs` one object per synthetic workload: the tiny fp32
prefill (time only), the GQA prefill (with the keep-all reference and the
Taylor score), the heavy-hitter prefill with the GPU key permutation inside
the step (plus the early-stopping variants), the sparse decode step (bf16,
MXFP4 and INT4 indexer caches, and a keep-all run that streams the whole KV
cache) and
the long prefill's keep-all reference.
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
HEADLINE = "long-bf16-L131072"
KDIR = os.path.join(ROOT, "block_sparse_attention_amd", "csrc", "kernels")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE,
                    help="prefill workload of the headline step: long-bf16-L131072 (default), gqa-bf16-L8192, "
                         "heavy-perm-bf16-L32768 (permutation generated on the GPU inside the step), tiny-fp32-L256")
    ap.add_argument("--headline-only", action="store_true", help="time the headline workload only")
    ap.add_argument("--configs", default="",
                    help="comma-separated workloads to time besides the headline (default: every one)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-early-stop", action="store_true", help="skip the early-stopping measurements")
    ap.add_argument("--es-tau", type=float, default=0.01, help="early-stopping threshold tau")
    ap.add_argument("--no-taylor", action="store_true", help="skip the Taylor-score measurement")
    ap.add_argument("--cpu-blocks", type=int, default=0,
                    help="query blocks the oracle covers (0: the workload's seeded sample, or every block)")
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
def prefill_host(I, name):
    cfg = {c.name: c for c in (I.C1, I.C2, I.C3, I.C5)}[name]
    return cfg, I.prefill_inputs(cfg)


def prefill_device(torch, cfg, host):
    """Device copies of the workload's inputs (made once, shared by its measurements)."""
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    return tuple(torch.from_numpy(x).to(tdt).to(dev) for x in host)


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


def bench_prefill(args, torch, B, cfg, dev_in, score_kind=None, top_p=None):
    """Times the prefill step (key permutation when the workload has segments, block scores, top-p
    selection, sparse attention) on resident inputs."""
    dq, dk, dv = dev_in
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
    del graph
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

    attn_file = os.path.join(KDIR, "prefill.hip")
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
                "traffic": None, "kernel": f"prefill_rows_kernel<float,{cfg.d}>", "flop_per_launch": flops,
                "avg_launch_ms": round(ms_attn, 4)}
    perm_blocks = None
    if perm is not None and score_kind == B.SPOT_SCORE_MEANPOOL:
        # top-p at the workload's p with history means over the permuted keys and without the permutation:
        # how many blocks the same mass needs in each case (outside the timed steps)
        kept = {}
        for name, seg, pm in (("with_permutation", cfg.segment, perm), ("without_permutation", 0, None)):
            d2 = B.prefill_desc(dq, dk, cfg.block, cfg.top_p, segment=seg)
            b2 = B.alloc_prefill(d2, dev)
            B.spot_block_score(d2, dq, dk, pm, None, None, None, b2.scores, b2.workspace)
            B.spot_select_topp(d2, b2.scores, b2.idx, b2.cnt)
            torch.cuda.synchronize()
            kept[name] = int(b2.cnt.cpu().numpy().astype(np.int64).sum())
            del b2
        cand = cfg.batch * cfg.hkv * cfg.nb * (cfg.nb + 1) // 2
        perm_blocks = {"top_p": cfg.top_p, "candidate_blocks": cand, **kept,
                       "change": round(kept["with_permutation"] / kept["without_permutation"] - 1.0, 4)}
    return dict(
        cfg=cfg, ms_step=ms_step, ms_step_eager=ms_step_eager, ms_step_graph=ms_step_graph, step_launch=step_launch,
        ms_perm=ms_perm, ms_sel=ms_sel, ms_attn=ms_attn,
        flops=flops, kept_fraction=kept_fraction, value=flops / (ms_step * 1e-3) / 1e12, roofline=roof,
        perm_blocks=perm_blocks,
    )


def prefill_object(res, headline=False):
    """JSON object of one prefill measurement."""
    cfg = res["cfg"]
    out = {"workload": cfg.name, "dtype": cfg.dtype, "seq_len": cfg.L, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d,
           "block": cfg.block, "top_p": cfg.top_p, "segment": cfg.segment,
           "value": round(res["value"], 4 if cfg.dtype != "bf16" else 2), "unit": "TFLOP/s",
           "ms_per_step": round(res["ms_step"], 4), "step_launch": res["step_launch"],
           "ms_per_step_stream_launches": round(res["ms_step_eager"], 4),
           "ms_per_step_graph_replay": round(res["ms_step_graph"], 4),
           "ms_key_permutation": round(res["ms_perm"], 4), "ms_score_select": round(res["ms_sel"], 4),
           "ms_attention": round(res["ms_attn"], 4), "kept_fraction": round(res["kept_fraction"], 4),
           "flop_per_step": res["flops"]}
    if not headline:
        out["roofline"] = res["roofline"]
    if res.get("perm_blocks"):
        out["top_p_kept_blocks"] = res["perm_blocks"]
    return out


def dense_object(sparse, dense):
    return {"workload": dense["cfg"].name, "top_p": 1.0, "ms_per_step": round(dense["ms_step"], 4),
            "ms_attention": round(dense["ms_attn"], 4), "value": round(dense["value"], 2), "unit": "TFLOP/s",
            "kept_fraction": round(dense["kept_fraction"], 4),
            "attention_frac_of_peak": dense["roofline"]["frac"],
            "sparse_speedup_step": round(dense["ms_step"] / sparse["ms_step"], 3),
            "sparse_speedup_attention": round(dense["ms_attn"] / sparse["ms_attn"], 3)}


# ----------------------------------------------------------------- decode
def decode_device(torch, B, I):
    """Device inputs of the sparse-decode workload (made once, shared by its measurements), with the
    MXFP4 encoding of the indexer keys (made once, when keys are appended; outside every step)."""
    cfg = I.C4
    dev = torch.device("cuda:0")
    D = I.decode_inputs(cfg)
    up = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
    t = dict(q=up(D["q"]), kc=up(D["k_cache"]), vc=up(D["v_cache"]), iq=up(D["idx_q"]), ik=up(D["idx_k"]),
             iw=torch.from_numpy(D["idx_w"]).to(dev))
    del D
    t["codes"], t["scales"] = B.quantize_indexer_keys(t["ik"], cfg.block, cfg.T)
    t["codes4"], t["scales4"] = B.quantize_indexer_keys_int4(t["ik"], cfg.block, cfg.T)
    torch.cuda.synchronize()
    return cfg, t


def bench_decode(args, torch, B, cfg, t, cache="bf16", top_p=None):
    dev = torch.device("cuda:0")
    top_p = cfg.top_p if top_p is None else top_p
    q, kc, vc, iq, iw = t["q"], t["kc"], t["vc"], t["iq"], t["iw"]
    desc = B.decode_desc(q, kc, cfg.block, top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.alloc_decode(desc, dev)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

    def score():
        if cache == "mxfp4":
            B.spot_indexer_score_mxfp4(desc, iq, iw, t["codes"], t["scales"], bufs.scores)
        elif cache == "int4":
            B.spot_indexer_score_int4(desc, iq, iw, t["codes4"], t["scales4"], bufs.scores)
        else:
            B.spot_block_score(desc, None, None, None, iq, iw, t["ik"], bufs.scores)

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

    # the step's launches as one HIP graph, replayed with a cold cache each time
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
    del graph
    # the same work either way: report the faster launch mode
    ms_step = min(ms_step_graph, ms_step_eager)
    step_launch = "hip_graph_replay" if ms_step_graph <= ms_step_eager else "stream_launches"
    cnt = bufs.cnt.cpu().numpy()[:, 0, 0]
    idx = bufs.idx.cpu().numpy()[:, 0, 0]
    bs = np.minimum(cfg.block, cfg.T - np.arange(cfg.nt) * cfg.block)
    kept_keys = np.array([bs[idx[b, :cnt[b]]].sum() for b in range(cfg.batch)], dtype=np.float64)
    kv_bytes = float(kept_keys.sum()) * cfg.hkv * cfg.d * 2 * 2
    scan_bytes = cfg.batch * cfg.nt * cfg.h_idx * cfg.d_idx * {"bf16": 2.0, "mxfp4": 0.5 + 1.0 / 32,
                                                                "int4": 0.5 + 2.0 / 32}[cache]
    qo_bytes = cfg.batch * cfg.hq * cfg.d * 2 * 2.0 + cfg.batch * cfg.h_idx * (cfg.d_idx * 2 + 4)
    step_bytes = kv_bytes + scan_bytes + qo_bytes
    attn_gbs = (kv_bytes + qo_bytes) / (ms_attn * 1e-3) / 1e9
    return dict(
        workload=cfg.name, indexer_cache=cache, top_p=top_p,
        value=round(step_bytes / (ms_step * 1e-3) / 1e9, 1), unit="GB/s",
        frac_of_hbm_peak=round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        ms_per_step=round(ms_step, 4), step_launch=step_launch, ms_per_step_stream_launches=round(ms_step_eager, 4),
        ms_per_step_graph_replay=round(ms_step_graph, 4), ms_score_select=round(ms_front, 4), ms_indexer_scan=round(ms_scan, 4),
        indexer_scan_gbs=round(scan_bytes / (ms_scan * 1e-3) / 1e9, 1), indexer_scan_bytes=scan_bytes,
        ms_select=round(ms_front - ms_scan, 4), ms_attention=round(ms_attn, 4),
        kept_fraction=round(float(kept_keys.sum()) / (cfg.batch * cfg.T), 4), bytes_per_step=step_bytes,
        roofline={"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                  "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "kernel": "decode attention (split + combine)",
                  "traffic": load_traffic(os.path.join(KDIR, "decode.hip"), f"decode_split_kernel@{cfg.name}"
                                          + ("" if top_p < 1.0 else "-keep-all")),
                  "bytes_per_launch": kv_bytes + qo_bytes},
    )


# ----------------------------------------------------------------- residual linear attention
def _event_ms(torch, fn, n):
    times = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def bench_rla_prefill(args, torch, B, cfg, dev_in):
    """Residual linear attention ([SPLA] §2.2) beside the prefill step: the
    block states (once per K/V) and the residual of every query block over
    the blocks its list does not keep, on the lists of one pipeline step."""
    dq, dk, dv = dev_in
    dev = torch.device("cuda:0")
    desc = B.prefill_desc(dq, dk, cfg.block, cfg.top_p)
    bufs = B.prefill(dq, dk, dv, cfg.block, cfg.top_p)
    rb = B.rla_prefill(desc, dq, dk, dv, bufs.idx, bufs.cnt)
    torch.cuda.synchronize()
    n = max(args.steps // 2, 3)
    ms_states = _event_ms(torch, lambda: B.spot_rla_block_states(desc, dk, dv, None, rb.states), n)
    ms_res = _event_ms(torch, lambda: B.spot_rla_prefill(desc, dq, rb.states, None, bufs.idx, bufs.cnt, rb.o_rla), n)
    cnt = bufs.cnt.cpu().numpy().astype(np.int64)                      # (batch, hkv, nb), own block included
    rest_blocks = float((np.arange(cfg.nb)[None, None, :] + 1 - cnt).clip(min=0).sum())
    d2 = cfg.d * cfg.d
    state_flop = 2.0 * d2 * cfg.L * cfg.hkv * cfg.batch
    out_flop = 2.0 * d2 * cfg.L * cfg.hq * cfg.batch
    res_bytes = rest_blocks * d2 * 4.0
    del rb, bufs
    return {"workload": cfg.name, "ms_block_states": round(ms_states, 4), "ms_residual": round(ms_res, 4),
            "block_states_tflops": round(state_flop / (ms_states * 1e-3) / 1e12, 2),
            "residual_state_reads_gb": round(res_bytes / 1e9, 3),
            "residual_gbs": round(res_bytes / (ms_res * 1e-3) / 1e9, 1),
            "residual_output_tflops": round(out_flop / (ms_res * 1e-3) / 1e12, 2),
            "blocks_outside_lists": int(rest_blocks)}


def bench_rla_decode(args, torch, B, cfg, t):
    """Residual linear attention of the decode step: the whole-cache state is
    built once (it changes only with the cache); per step the state's
    contribution minus the kept keys', on the lists of the bf16-indexer step,
    as its own pass and inside the attention pass."""
    dev = torch.device("cuda:0")
    q, kc, vc = t["q"], t["kc"], t["vc"]
    desc = B.decode_desc(q, kc, cfg.block, cfg.top_p, cfg.h_idx, cfg.d_idx)
    bufs = B.decode(q, kc, vc, t["iq"], t["iw"], t["ik"], cfg.block, cfg.top_p)
    ws = torch.empty(max(B.spot_workspace_size(desc, B.SPOT_OP_RLA_DECODE_STATE), 1), dtype=torch.uint8, device=dev)
    state = torch.empty(cfg.batch, cfg.hkv, cfg.d, cfg.d, dtype=torch.float32, device=dev)
    o = torch.empty(cfg.batch, cfg.hq, cfg.d, dtype=torch.float32, device=dev)
    dws = torch.empty(max(B.spot_workspace_size(desc, B.SPOT_OP_RLA_DECODE), 1), dtype=torch.uint8, device=dev)
    ms_state = _event_ms(torch, lambda: B.spot_rla_decode_state(desc, kc, vc, state, ws), 2)
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    times = []
    for _ in range(max(args.steps, 3)):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.spot_rla_decode(desc, q, kc, vc, state, bufs.idx, bufs.cnt, o, dws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    # the same term inside the attention pass (the kept tiles it already reads), against the plain attention
    fws = torch.empty(B.spot_workspace_size(desc, B.SPOT_OP_DECODE_RLA), dtype=torch.uint8, device=dev)
    o2, lse2 = torch.empty_like(bufs.o), torch.empty_like(bufs.lse)

    def timed(fn):
        ts = []
        for _ in range(max(args.steps, 3)):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    ms_plain = timed(lambda: B.spot_sparse_attn_decode(desc, q, kc, vc, bufs.idx, bufs.cnt, o2, lse2,
                                                       bufs.workspace))
    ms_fused = timed(lambda: B.spot_sparse_attn_decode_rla(desc, q, kc, vc, bufs.idx, bufs.cnt, state, o2, lse2, o,
                                                           fws))
    cnt = bufs.cnt.cpu().numpy()[:, 0, 0].astype(np.int64)
    kv_bytes = float(cnt.sum()) * cfg.block * cfg.hkv * cfg.d * 2 * 2
    st_bytes = cfg.batch * cfg.hkv * cfg.d * cfg.d * 4.0
    del ws, fws, flush
    return {"workload": cfg.name, "ms_cache_state": round(ms_state, 4), "ms_per_step": round(ms, 4),
            "bytes_per_step": kv_bytes + st_bytes, "gbs": round((kv_bytes + st_bytes) / (ms * 1e-3) / 1e9, 1),
            "fused_with_attention": {"ms_attention": round(ms_plain, 4), "ms_attention_and_residual": round(ms_fused, 4)}}


# ----------------------------------------------------------------- early stopping
def bench_early_stop(args, torch, B, cfg, dev_in):
    """Early-stopped prefill on the heavy-hitter workload (L=32768, segment
    2048): key permutation, block scores, history visiting order and the
    early-stopped attention, captured as one HIP graph."""
    dev = torch.device("cuda:0")
    dq, dk, dv = dev_in
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

    return dict(
        workload=cfg.name, tau=tau, value=round(flops / (ms_step * 1e-3) / 1e12, 2), unit="TFLOP/s",
        ms_per_step=round(ms_step, 4), ms_key_permutation=round(ms_perm, 4), ms_score_order=round(ms_front, 4),
        ms_attention=round(ms_attn, 4), taken_fraction=round(float(pairs_row.sum()) / dense_pairs, 4),
        walked_fraction=round(walked / dense_pairs, 4), mean_history_blocks=round(float(nused.mean()), 2),
        flop_per_step=flops,
        roofline={"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                  "kernel": "prefill_mfma_kernel<128,8,1,true,true,true> (early stop)", "avg_launch_ms": round(ms_attn, 4),
                  "traffic": load_traffic(os.path.join(KDIR, "prefill.hip"),
                                          f"prefill_mfma_kernel_early_stop@{cfg.name}"),
                  "walked_tflops": round(4.0 * cfg.d * walked / (ms_attn * 1e-3) / 1e12, 2)},
    )


def bench_history_map(args, torch, B, cfg, dev_in):
    """Early-stopped prefill on representative-query history maps on the
    heavy-hitter workload: maps of every segment, then the attention walking
    them, captured as one HIP graph."""
    dev = torch.device("cuda:0")
    dq, dk, dv = dev_in
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
_ORC = {}   # inputs of the oracle's per-unit work, inherited by the forked workers


def _oracle_worker_init():
    try:   # one BLAS thread per worker process: the pool supplies the parallelism
        from threadpoolctl import threadpool_limits
        _ORC["limit"] = threadpool_limits(1)
    except Exception:
        pass


def _oracle_unit(unit):
    """Select and attend one (KV head, query block) with the float64 oracle; returns its visible
    (query, key) pairs summed over the group's heads and the seconds it took."""
    import oracle
    g, i = unit
    c = _ORC
    t0 = time.perf_counter()
    kept = oracle.topp_keep(c["scores"][g, i, :i + 1], oracle.prefill_forced(i, c["n_sink"], c["n_recent"]),
                            c["top_p"], c["k_min"])
    G = c["G"]
    oracle.attend_prefill(c["q"][g * G:(g + 1) * G], c["k"][g:g + 1], c["v"][g:g + 1], [{i: kept}], c["block"],
                          c["scale"], c["segment"], None if c["perm"] is None else c["perm"][g:g + 1], qblocks=[i])
    dt = time.perf_counter() - t0
    L, B = c["L"], c["block"]
    bs = [min(B, L - j * B) for j in range(i + 1)]
    nrow = bs[i]
    full = sum(bs[int(j)] for j in kept if int(j) != i)
    diag = i in set(int(j) for j in kept)
    return G * (nrow * full + (nrow * (nrow + 1) // 2 if diag else 0)), dt


def cpu_baseline(cfg, host, I, n_blocks: int = 0):
    """The float64 oracle on the host over the workload's seeded sample of query blocks (every block
    on the short workloads): widen the inputs, permutation when the workload uses one, pool and score
    every block (one process), then select and attend each (KV head, sampled query block) in a pool
    of forked worker processes with one BLAS thread each.  Runs before the process touches the GPU."""
    import multiprocessing as mp

    import oracle
    if n_blocks > 0:
        blocks = I.oracle_query_blocks(cfg.with_(oracle_qblocks=n_blocks))
    else:
        blocks = I.oracle_query_blocks(cfg)
    blocks = [int(b) for b in blocks]
    ncpu = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = ncpu
    workers = max(1, min(ncpu, avail, 16))
    q, k, v = host
    t0 = time.perf_counter()
    q64, k64, v64 = (np.asarray(x[0], dtype=np.float64) for x in (q, k, v))
    scale = 1.0 / math.sqrt(cfg.d)
    perm = None
    if cfg.segment:
        perm, _ = oracle.key_permutation(q64, k64, cfg.block, cfg.segment, scale)
    qbar, kn, kp = oracle.pool_blocks(q64, k64, cfg.block, perm)
    scores = oracle.meanpool_scores(qbar, kn, kp, cfg.block, cfg.segment, scale)
    t_front = time.perf_counter() - t0
    _ORC.update(q=q64, k=k64, v=v64, perm=perm, scores=scores, block=cfg.block, segment=cfg.segment, L=cfg.L,
                G=cfg.hq // cfg.hkv, scale=scale, top_p=cfg.top_p, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                k_min=cfg.k_min)
    units = [(g, i) for i in sorted(blocks, reverse=True) for g in range(cfg.hkv)]   # longest first
    with mp.get_context("fork").Pool(workers, initializer=_oracle_worker_init) as pool:
        res = pool.map(_oracle_unit, units, chunksize=1)
    dt = time.perf_counter() - t0
    _ORC.clear()
    pairs = float(sum(r[0] for r in res))
    unit_s = float(sum(r[1] for r in res))
    flops = 4.0 * cfg.d * pairs
    cpu_model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = "every query block" if len(blocks) == cfg.nb else \
        f"{len(blocks)} seeded query blocks ({', '.join(str(b) for b in blocks[:3])}, ..., {blocks[-1]})"
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"float64 NumPy oracle on {cfg.name}: widen inputs, "
                      f"{'key permutation, ' if cfg.segment else ''}pool and score every block (one process), "
                      f"then select and attend {what} x {cfg.hkv} KV heads in {workers} worker processes",
            "workers": workers, "blas_threads_per_worker": 1, "os_cpu_count": ncpu, "cpus_available": avail,
            "cpu_model": cpu_model, "seconds": round(dt, 2), "seconds_pool_and_score": round(t_front, 2),
            "query_blocks": len(blocks), "units": len(units),
            "seconds_per_query_block": round(dt / len(blocks), 4),
            "cpu_seconds_per_unit": round(unit_s / len(units), 4), "flop": flops}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (prefill would shard by KV head "
              "and decode by sequence, with no exchange; one GPU's share is what is timed)", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_attention_amd import binding as B
    from block_sparse_attention_amd import inputs as I

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    head_cfg, head_host = prefill_host(I, args.workload)
    say(f"inputs of {head_cfg.name} generated")
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's worker processes are forked before this process touches the GPU
        cpu = cpu_baseline(head_cfg, head_host, I, args.cpu_blocks)
        say(f"cpu baseline: {cpu}")

    B.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    head_dev = prefill_device(torch, head_cfg, head_host)
    del head_host
    # the ceilings are measured first: their GEMMs and copies also bring the GPU to its working clock after the
    # host-side input generation, before the warm-up steps of the prefill step
    ceil = measured_ceilings(torch)
    say(f"measured ceilings: {ceil}")
    pre = bench_prefill(args, torch, B, head_cfg, head_dev)
    say(f"headline {head_cfg.name}: {prefill_object(pre)}")
    # the same kernels keeping every block (p = 1): an in-house dense reference
    dense = bench_prefill(args, torch, B, head_cfg, head_dev, top_p=1.0)
    configs = {head_cfg.name: dict(prefill_object(pre, headline=True), headline=True,
                                   dense_reference=dense_object(pre, dense))}
    say(f"dense reference: {configs[head_cfg.name]['dense_reference']}")
    del dense
    if args.headline_only:
        del head_dev
    else:
        del head_dev
        torch.cuda.empty_cache()
        wanted = set(x for x in args.configs.split(",") if x) or None
        for c in (I.C1, I.C2, I.C3, I.C5):
            if c.name == head_cfg.name or (wanted is not None and c.name not in wanted):
                continue
            cfg, host = prefill_host(I, c.name)
            dev_in = prefill_device(torch, cfg, host)
            del host
            r = bench_prefill(args, torch, B, cfg, dev_in)
            obj = prefill_object(r)
            if cfg.dtype == "bf16":
                obj["dense_reference"] = dense_object(r, bench_prefill(args, torch, B, cfg, dev_in, top_p=1.0))
            if cfg.name == I.C2.name and not args.no_taylor:
                t = bench_prefill(args, torch, B, cfg, dev_in, score_kind=B.SPOT_SCORE_TAYLOR)
                obj["taylor_score"] = {"score": "second-order Taylor", "value": round(t["value"], 2),
                                       "unit": "TFLOP/s", "ms_per_step": round(t["ms_step"], 4),
                                       "ms_score_select": round(t["ms_sel"], 4),
                                       "ms_attention": round(t["ms_attn"], 4),
                                       "kept_fraction": round(t["kept_fraction"], 4), "flop_per_step": t["flops"]}
            if cfg.name == I.C2.name:
                obj["residual_linear_attention"] = bench_rla_prefill(args, torch, B, cfg, dev_in)
            if cfg.name == I.C3.name and not args.no_early_stop:
                obj["early_stop"] = bench_early_stop(args, torch, B, cfg, dev_in)
                obj["early_stop_history_map"] = bench_history_map(args, torch, B, cfg, dev_in)
            configs[cfg.name] = obj
            say(f"{cfg.name}: {obj}")
            del dev_in
            torch.cuda.empty_cache()
        if not args.no_decode and (wanted is None or I.C4.name in wanted):
            dcfg, t = decode_device(torch, B, I)
            dec = {"bf16_indexer": bench_decode(args, torch, B, dcfg, t)}
            say(f"decode: {dec['bf16_indexer']}")
            dec["mxfp4_indexer"] = bench_decode(args, torch, B, dcfg, t, cache="mxfp4")
            say(f"decode mxfp4: {dec['mxfp4_indexer']}")
            dec["int4_indexer"] = bench_decode(args, torch, B, dcfg, t, cache="int4")
            say(f"decode int4: {dec['int4_indexer']}")
            # every block kept (p = 1): the attention streams the whole 8 GiB KV cache
            dec["keep_all"] = bench_decode(args, torch, B, dcfg, t, top_p=1.0)
            say(f"decode keep-all: {dec['keep_all']}")
            dec["residual_linear_attention"] = bench_rla_decode(args, torch, B, dcfg, t)
            say(f"decode residual linear attention: {dec['residual_linear_attention']}")
            configs[dcfg.name] = dict(dec, workload=dcfg.name, batch=dcfg.batch, context=dcfg.T, hq=dcfg.hq,
                                      hkv=dcfg.hkv, d=dcfg.d, block=dcfg.block, h_idx=dcfg.h_idx, d_idx=dcfg.d_idx,
                                      top_p=dcfg.top_p)
            del t

    cfg = pre["cfg"]
    line = {
        "metric": METRIC, "value": round(pre["value"], 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(pre["ms_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.L, "hq": cfg.hq, "hkv": cfg.hkv,
                   "d": cfg.d, "block": cfg.block, "top_p": cfg.top_p, "n_sink": cfg.n_sink,
                   "n_recent": cfg.n_recent, "heavy_hitters": cfg.heavy_hitters, "segment": cfg.segment,
                   "kept_fraction": round(pre["kept_fraction"], 4),
                   "ms_attention": round(pre["ms_attn"], 4), "ms_score_select": round(pre["ms_sel"], 4),
                   "ms_key_permutation": round(pre["ms_perm"], 4),
                   "ms_per_step_stream_launches": round(pre["ms_step_eager"], 4),
                   "ms_per_step_graph_replay": round(pre["ms_step_graph"], 4), "step_launch": pre["step_launch"],
                   "flop_per_step": pre["flops"]},
        "roofline": dict(pre["roofline"], measured_ceilings=ceil,
                         frac_of_measured_gemm=round(pre["roofline"]["achieved"] / ceil["bf16_gemm_8192_tflops"], 4)
                         if pre["roofline"]["peak"] else None),
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
