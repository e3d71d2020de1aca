"""Summarise rocprofv3 databases into the text records kept under profiles/.

  python -m block_sparse_attention_amd.prof_summary --trace T.db --fetch F.db --write W.db \
      --cmd-trace "..." --cmd-pmc "..." --out profiles

* kernel table: calls, total / average / min / max duration per kernel (trace run);
* HBM traffic per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
  each scaled by what the same counter reads for the plain 1 GiB device copy
  the profiling workload runs (known bytes); written to traffic.json together
  with a digest of the kernel source, so a stale record is ignored.
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

# kernel-name fragment -> (source file, workload key, launches used).  The
# profiling workload runs its parts in a fixed order (GQA prefill, decode with
# the bf16 indexer cache, decode with the MXFP4 cache, early-stopped
# heavy-hitter prefill), so "first" takes the first `--steps` launches of a
# kernel that several parts use, "all" every launch.
TRACKED = {
    "prefill_mfma_kernel<128, 8, 1, false, false>": ("prefill.hip", "prefill_mfma_kernel@gqa-bf16-L8192", "all"),
    "prefill_mfma_kernel<128, 8, 1, true, true>": ("prefill.hip",
                                                   "prefill_mfma_kernel_early_stop@heavy-perm-bf16-L32768", "all"),
    "decode_split_kernel<128, 4>": ("decode.hip", "decode_split_kernel@decode-b16-T131072", "first"),
    "indexer_score_kernel<": ("score.hip", "indexer_score_kernel@decode-b16-T131072", "all"),
    "indexer_score_mxfp4_kernel": ("score.hip", "indexer_score_mxfp4_kernel@decode-b16-T131072", "all"),
    "pool_blocks_kernel<unsigned short>": ("score.hip", "pool_blocks_kernel@gqa-bf16-L8192", "first"),
}


def digest(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def kernel_durations(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall() if _has(con, "kernels") else []
    if not rows:
        rows = con.execute(
            "select s.string, (k.end - k.start) from rocpd_kernel_dispatch k join rocpd_info_kernel_symbol ks "
            "on k.kernel_id = ks.id join rocpd_string s on ks.kernel_name_id = s.id").fetchall()
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
    args = ap.parse_args()
    os.makedirs(args.out, exist_ok=True)

    durs = kernel_durations(args.trace)
    lines = [f"# rocprofv3 kernel trace: {args.name}", "", "Command:", "", "```", args.cmd_trace, "```", "",
             "| kernel | calls | total us | avg us | min us | max us |", "|---|---:|---:|---:|---:|---:|"]
    for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short(name)}` | {len(ds)} | {sum(ds) / 1e3:.1f} | {statistics.mean(ds) / 1e3:.2f} | "
                     f"{min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")

    traffic = {}
    if args.fetch and args.write:
        fv, wv = counter_values(args.fetch), counter_values(args.write)
        ff, wf = copy_factor(fv), copy_factor(wv)
        lines += ["", "HBM traffic per launch (rocprofv3 --pmc, one counter per run):", "", "```", args.cmd_pmc, "```",
                  "", f"Calibration on a 1 GiB device copy: FETCH_SIZE reads {ff:.4f} x the bytes moved, "
                  f"WRITE_SIZE {wf:.4f} x; measured values below are divided by these factors.", "",
                  "| kernel | launches | fetch MB | write MB | total MB |", "|---|---:|---:|---:|---:|"]
        for frag, (src, key, use) in TRACKED.items():
            fk = [k for k in fv if frag in k]
            wk = [k for k in wv if frag in k]
            if not fk or not wk:
                continue
            fl, wl = fv[fk[0]], wv[wk[0]]
            if use == "first":
                fl, wl = fl[:args.steps], wl[:args.steps]
            fetch = statistics.median(fl) * 1024 / ff
            write = statistics.median(wl) * 1024 / wf
            lines.append(f"| `{frag}` ({key.split('@')[1]}) | {len(fl)} | {fetch / 1e6:.2f} | {write / 1e6:.2f} | "
                         f"{(fetch + write) / 1e6:.2f} |")
            traffic[key] = {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
                            "write_bytes": round(write), "source_sha256_16": digest(os.path.join(KDIR, src)),
                            "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)}
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
