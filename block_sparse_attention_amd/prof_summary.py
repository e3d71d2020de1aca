"""Summarise rocprofv3 databases into the text records kept under profiles/.

  python -m block_sparse_attention_amd.prof_summary --trace T.db --fetch F.db --write W.db \
      --cmd-trace "..." --cmd-pmc "..." --out profiles

* kernel table: calls, total / average / min / max duration per kernel (trace run);
* HBM traffic per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
  each scaled by what the same counter reads for the plain 1 GiB device copy
  the profiling workload runs (known bytes); written to traffic.json together
  with a digest of the kernel source, so a stale record is ignored;
* with --pmc DB ... --kernel K: the other counters of those runs for the first
  --steps launches of kernel K, summed over the GPU's instances, and the
  derived clock, MFMA occupancy, VALU mix and wave residency.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sqlite3
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KDIR = os.path.join(PKG, "csrc", "kernels")
COPY_BYTES = 1 << 30

# (kernel-name fragment, source file, workload key, first, count): the launches
# of that kernel from position first * steps to (first + count) * steps - 1,
# in the profiling workload's fixed order (long-context prefill, GQA prefill,
# decode with the bf16 indexer cache, with the MXFP4 cache, with the INT4
# cache, keeping every block, early-stopped heavy-hitter prefill, top-p
# heavy-hitter prefill through the permutation); count 0 takes every launch.
TRACKED = [
    ("prefill_mfma_kernel<128, 8, 1, false, false, true>", "prefill.hip", "prefill_mfma_kernel@long-bf16-L131072", 0, 1),
    ("prefill_mfma_kernel<128, 8, 1, false, false, true>", "prefill.hip", "prefill_mfma_kernel@gqa-bf16-L8192", 1, 1),
    ("prefill_mfma_kernel<128, 8, 1, true, true, true>", "prefill.hip",
     "prefill_mfma_kernel_early_stop@heavy-perm-bf16-L32768", 0, 0),
    ("prefill_mfma_kernel<128, 8, 1, true, false, true>", "prefill.hip", "prefill_mfma_kernel@heavy-perm-bf16-L32768",
     0, 0),
    ("decode_split_kernel<128, 4", "decode.hip", "decode_split_kernel@decode-b16-T131072", 0, 1),
    ("decode_split_kernel<128, 4", "decode.hip", "decode_split_kernel@decode-b16-T131072-keep-all", 3, 1),
    ("indexer_score_kernel<", "score.hip", "indexer_score_kernel@decode-b16-T131072", 0, 1),
    ("indexer_score_mxfp4_kernel", "score.hip", "indexer_score_mxfp4_kernel@decode-b16-T131072", 0, 0),
    ("indexer_score_int4_kernel", "score.hip", "indexer_score_int4_kernel@decode-b16-T131072", 0, 0),
    ("pool_blocks_kernel<unsigned short>", "score.hip", "pool_blocks_kernel@long-bf16-L131072", 0, 1),
    ("pool_blocks_kernel<unsigned short>", "score.hip", "pool_blocks_kernel@gqa-bf16-L8192", 1, 1),
]


def digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def kernel_durations(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels order by start").fetchall() if _has(con, "kernels") else []
    if not rows:
        rows = con.execute(
            "select s.string, (k.end - k.start) from rocpd_kernel_dispatch k join rocpd_info_kernel_symbol ks "
            "on k.kernel_id = ks.id join rocpd_string s on ks.kernel_name_id = s.id order by k.start").fetchall()
    out = defaultdict(list)
    for name, dur in rows:
        out[name].append(float(dur))
    return out


def _has(con, name):
    return con.execute("select 1 from sqlite_master where name=?", (name,)).fetchone() is not None


def counter_values(db: str):
    con = sqlite3.connect(db)
    out = defaultdict(list)
    for name, v in con.execute("select kernel_name, value from counters_collection order by dispatch_id"):
        out[name].append(float(v))
    return out


def counters_of(dbs, frag: str, steps: int):
    """counter -> per-launch values (summed over instances) of the first `steps` launches of kernel `frag`."""
    out = defaultdict(list)
    for db in dbs:
        con = sqlite3.connect(db)
        per = defaultdict(lambda: defaultdict(float))
        order = []
        for did, name, cn, v in con.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection order by dispatch_id"):
            if frag in name:
                if did not in per:
                    order.append(did)
                per[did][cn] += float(v)
        for did in order[:steps]:
            for cn, v in per[did].items():
                out[cn].append(v)
    return {cn: statistics.mean(vs) for cn, vs in out.items()}


def counter_lines(c: dict, trace_us: float, ncu: int, nse: int, nxcd: int):
    """Derived figures; SQ_* are per-SE or per-SIMD sums over the GPU, GRBM_GUI_ACTIVE per XCD."""
    simds = 4 * ncu
    out = []
    if "GRBM_GUI_ACTIVE" in c:
        cyc = c["GRBM_GUI_ACTIVE"] / nxcd
        out.append(f"* cycles per launch (GRBM_GUI_ACTIVE per XCD): {cyc:.4g}; over the traced launch time of "
                   f"{trace_us:.1f} us that is a clock of {cyc / trace_us / 1e3:.2f} GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out.append(f"* MFMA unit busy: {c['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / cyc:.1%} of SIMD cycles "
                       f"(SQ_VALU_MFMA_BUSY_CYCLES / (4 x {ncu} CUs x cycles))")
        if "SQ_WAVE_CYCLES" in c:
            out.append(f"* waves resident per SIMD on average: {4 * c['SQ_WAVE_CYCLES'] / simds / cyc:.2f} "
                       f"(SQ_WAVE_CYCLES, quad-cycles)")
    if "SQ_INSTS_MFMA" in c and "SQ_INSTS_VALU" in c:
        out.append(f"* VALU instructions per MFMA (the count includes the MFMA itself): "
                   f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f}")
    if "SQ_INSTS_VALU_TRANS_F32" in c and "SQ_INSTS_MFMA" in c:
        out.append(f"* fp32 transcendentals per MFMA: {c['SQ_INSTS_VALU_TRANS_F32'] / c['SQ_INSTS_MFMA']:.2f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and "SQ_VALU_MFMA_BUSY_CYCLES" in c:
        out.append(f"* cycles with a VALU instruction issued beside a busy MFMA: "
                   f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1%} of MFMA-busy cycles")
    if "SQ_WAVE_CYCLES" in c:
        for k, what in (("SQ_WAIT_ANY", "waiting on a counter (s_waitcnt)"),
                        ("SQ_WAIT_INST_ANY", "waiting to issue"), ("SQ_WAIT_INST_LDS", "waiting to issue an LDS op")):
            if k in c:
                out.append(f"* wave-cycles {what}: {c[k] / c['SQ_WAVE_CYCLES']:.1%} ({k} / SQ_WAVE_CYCLES)")
    if "SQ_LDS_IDX_ACTIVE" in c and "GRBM_GUI_ACTIVE" in c:
        out.append(f"* LDS busy with indexed accesses: {c['SQ_LDS_IDX_ACTIVE'] / ncu / (c['GRBM_GUI_ACTIVE'] / nxcd):.1%} "
                   f"of CU cycles; bank-conflict cycles: {c.get('SQ_LDS_BANK_CONFLICT', float('nan')):.4g}")
    return out


def copy_factor(vals) -> float:
    """counter KiB read for the 1 GiB copy / true KiB."""
    copies = [v for name, vs in vals.items() if "copyBuffer" in name or "copy" in name.lower()
              for v in vs if v > 0.25 * COPY_BYTES / 1024]
    if not copies:
        raise SystemExit("no 1 GiB copy dispatch found for calibration")
    return statistics.median(copies) / (COPY_BYTES / 1024)


def short(name: str) -> str:
    return name.replace("void ", "").replace("spot::", "").split("(")[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--cmd-trace", default="")
    ap.add_argument("--cmd-pmc", default="")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--name", default="kernels")
    ap.add_argument("--steps", type=int, default=3, help="--steps of the profiling workload")
    ap.add_argument("--pmc", nargs="*", default=[], help="databases of counter runs (any counters)")
    ap.add_argument("--kernel", default="", help="kernel-name fragment the --pmc summary covers")
    ap.add_argument("--cmd-counters", default="")
    ap.add_argument("--groups", default="", help="KERNEL=N:label,N:label,...: split that kernel's launches, in "
                                                 "order, into consecutive groups and report each group's mean")
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--ses", type=int, default=32)
    ap.add_argument("--xcds", type=int, default=8)
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)

    durs = kernel_durations(args.trace)
    lines = [f"# rocprofv3 kernel trace: {args.name}", "", "Command:", "", "```", args.cmd_trace, "```", "",
             "| kernel | calls | total us | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short(name)}` | {len(ds)} | {sum(ds) / 1e3:.1f} | {statistics.mean(ds) / 1e3:.2f} | "
                     f"{min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")

    if args.groups:
        frag, spec = args.groups.split("=", 1)
        ds = next((v for k, v in durs.items() if frag in k), [])
        lines += ["", f"Launches of `{frag}` in order, by the part of the command that made them:", "",
                  "| launches | part | avg us | min us | max us |", "|---|---|---:|---:|---:|"]
        at = 0
        for part in spec.split(","):
            n, label = part.split(":", 1)
            g = ds[at:at + int(n)]
            at += int(n)
            if g:
                lines.append(f"| {at - len(g)}..{at - 1} | {label} | {statistics.mean(g) / 1e3:.2f} | "
                             f"{min(g) / 1e3:.2f} | {max(g) / 1e3:.2f} |")

    traffic = {}
    if args.fetch and args.write:
        fv, wv = counter_values(args.fetch), counter_values(args.write)
        ff, wf = copy_factor(fv), copy_factor(wv)
        lines += ["", "HBM traffic per launch (rocprofv3 --pmc, one counter per run):", "", "```", args.cmd_pmc, "```",
                  "", f"Calibration on a 1 GiB device copy: FETCH_SIZE reads {ff:.4f} x the bytes moved, "
                  f"WRITE_SIZE {wf:.4f} x; measured values below are divided by these factors.", "",
                  "| kernel | launches | fetch MB | write MB | total MB |", "|---|---:|---:|---:|---:|"]
        for frag, src, key, first, count in TRACKED:
            fk = [k for k in fv if frag in k]
            wk = [k for k in wv if frag in k]
            if not fk or not wk:
                continue
            fl, wl = fv[fk[0]], wv[wk[0]]
            if count:
                fl = fl[first * args.steps:(first + count) * args.steps]
                wl = wl[first * args.steps:(first + count) * args.steps]
            if not fl or not wl:
                continue
            fetch = statistics.median(fl) * 1024 / ff
            write = statistics.median(wl) * 1024 / wf
            lines.append(f"| `{frag}` ({key.split('@')[1]}) | {len(fl)} | {fetch / 1e6:.2f} | {write / 1e6:.2f} | "
                         f"{(fetch + write) / 1e6:.2f} |")
            traffic[key] = {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
                            "write_bytes": round(write), "source_sha256_16": digest(os.path.join(KDIR, src)),
                            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
    if args.pmc and args.kernel:
        c = counters_of(args.pmc, args.kernel, args.steps)
        kd = [statistics.mean(ds[:args.steps]) / 1e3 for name, ds in durs.items() if args.kernel in name]
        lines += ["", f"Counters of `{args.kernel}` (mean of its first {args.steps} launches, each summed over the "
                  "GPU's instances):", "", "```", args.cmd_counters, "```", "",
                  "| counter | value |", "|---|---:|"]
        lines += [f"| {cn} | {v:.4g} |" for cn, v in sorted(c.items())]
        lines += [""] + counter_lines(c, kd[0] if kd else float("nan"), args.cus, args.ses, args.xcds)
    path = os.path.join(args.out, f"{args.name}.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)
    if traffic:
        tpath = os.path.join(args.out, "traffic.json")
        old = json.load(open(tpath)) if os.path.exists(tpath) else {}
        old.update(traffic)
        json.dump(old, open(tpath, "w"), indent=1, sort_keys=True)
        print(tpath)


if __name__ == "__main__":
    main()
