"""Fixed workload for rocprofv3 runs (kernel trace and hardware counters).

Runs, on cuda:0, in this order: `--steps` prefill steps of the long-context
workload (L=131072, 32/8 heads, d=128, bf16, block 128, top-p 0.9), `--steps`
prefill steps of the GQA workload (L=8192, block 64, top-p 0.9), `--steps`
decode steps of the sparse decode workload (batch 16, context 131072) with the
bf16 indexer cache, then with the MXFP4 indexer cache, then with the INT4
indexer cache, then keeping every block (p = 1), `--steps` early-stopped prefill steps of the heavy-hitter
workload (L=32768, segment 2048, tau 0.01, permutation on the GPU), `--steps`
top-p prefill steps of that workload through the same permutation, and
`--steps` plain device copies of 1 GiB, whose counter readings calibrate
FETCH_SIZE / WRITE_SIZE against a known byte count.  The summariser
attributes launches of a kernel that several parts use by this order.

  rocprofv3 --kernel-trace --stats -d OUT -o run -- python -m block_sparse_attention_amd.prof_workload
  rocprofv3 --pmc FETCH_SIZE -d OUT -o fetch -- python -m block_sparse_attention_amd.prof_workload
  rocprofv3 --pmc WRITE_SIZE -d OUT -o write -- python -m block_sparse_attention_amd.prof_workload
"""
from __future__ import annotations

import argparse
import sys

import torch

from . import binding as B
from . import inputs as I

COPY_BYTES = 1 << 30


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-early-stop", action="store_true")
    args = ap.parse_args()
    B.load_library()
    dev = torch.device("cuda:0")

    for cfg in (I.C5, I.C2):
        q, k, v = I.prefill_inputs(cfg)
        dq, dk, dv = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
        del q, k, v
        desc = B.prefill_desc(dq, dk, cfg.block, cfg.top_p)
        bufs = B.alloc_prefill(desc, dev)
        for _ in range(args.steps):
            B.prefill(dq, dk, dv, cfg.block, cfg.top_p, bufs=bufs)
        torch.cuda.synchronize()
        print(f"prefill steps of {cfg.name} done: {args.steps}", flush=True)
        del dq, dk, dv, bufs

    if not args.no_decode:
        dc = I.C4
        D = I.decode_inputs(dc)
        up = lambda x: torch.from_numpy(x).to(torch.bfloat16).to(dev)
        t = {kk: (torch.from_numpy(vv).to(dev) if kk == "idx_w" else up(vv)) for kk, vv in D.items()}
        del D
        dbufs = None
        for _ in range(args.steps):
            dbufs = B.decode(t["q"], t["k_cache"], t["v_cache"], t["idx_q"], t["idx_w"], t["idx_k"], dc.block,
                             dc.top_p, bufs=dbufs)
        torch.cuda.synchronize()
        print(f"decode steps done: {args.steps}", flush=True)
        codes, scales = B.quantize_indexer_keys(t["idx_k"], dc.block, dc.T)
        for _ in range(args.steps):
            dbufs = B.decode(t["q"], t["k_cache"], t["v_cache"], t["idx_q"], t["idx_w"], (codes, scales),
                             dc.block, dc.top_p, bufs=dbufs)
        torch.cuda.synchronize()
        print(f"decode steps with the MXFP4 indexer cache done: {args.steps}", flush=True)
        codes4, scales4 = B.quantize_indexer_keys_int4(t["idx_k"], dc.block, dc.T)
        for _ in range(args.steps):
            dbufs = B.decode(t["q"], t["k_cache"], t["v_cache"], t["idx_q"], t["idx_w"], (codes4, scales4),
                             dc.block, dc.top_p, bufs=dbufs)
        torch.cuda.synchronize()
        print(f"decode steps with the INT4 indexer cache done: {args.steps}", flush=True)
        abufs = None
        for _ in range(args.steps):
            abufs = B.decode(t["q"], t["k_cache"], t["v_cache"], t["idx_q"], t["idx_w"], t["idx_k"], dc.block, 1.0,
                             bufs=abufs)
        torch.cuda.synchronize()
        print(f"decode steps keeping every block done: {args.steps}", flush=True)
        del t, codes, scales, codes4, scales4, dbufs, abufs

    if not args.no_early_stop:
        ec = I.C3
        q, k, v = I.prefill_inputs(ec)
        eq, ek, ev = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
        del q, k, v
        perm = B.key_permutation(eq, ek, ec.block, ec.segment)
        ebufs = None
        for _ in range(args.steps):
            ebufs = B.prefill_early_stop(eq, ek, ev, ec.block, ec.segment, 0.01, perm=perm, bufs=ebufs)
        torch.cuda.synchronize()
        print(f"early-stopped prefill steps done: {args.steps}", flush=True)
        pbufs = None
        for _ in range(args.steps):
            pbufs = B.prefill(eq, ek, ev, ec.block, ec.top_p, perm=perm, segment=ec.segment, bufs=pbufs)
        torch.cuda.synchronize()
        print(f"top-p prefill steps through the permutation done: {args.steps}", flush=True)
        del eq, ek, ev, perm, ebufs, pbufs

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy steps done: {args.steps} x {COPY_BYTES} bytes", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
