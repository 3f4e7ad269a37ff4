"""Summaries of rocprofv3 CSV output for the layer-shard kernels.

    python -m tensor_transformer_layer_tp_amd.profsum stats  <dir>            # per-kernel durations
    python -m tensor_transformer_layer_tp_amd.profsum counters <dir> [filter] # per-kernel counter means

<dir> is a rocprofv3 output directory written with --output-format csv. The
counter summary averages every counter over the dispatches of each kernel
whose name contains `filter`.
"""
from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict


def _rows(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def short(name: str) -> str:
    n = name.split("(")[0]
    return n.replace("tpk::", "").replace("(anonymous namespace)::", "").replace("void ", "")


def stats(d: str) -> str:
    out = ["| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in _rows(d, "kernel_stats.csv"):
        out.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def counters(d: str, filt: str = "") -> str:
    acc = defaultdict(lambda: defaultdict(list))
    for r in _rows(d, "counter_collection.csv"):
        if filt and filt not in r["Kernel_Name"]:
            continue
        acc[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in acc.values() for c in k})
    out = ["| kernel | dispatches | " + " | ".join(names) + " |", "|---" * (len(names) + 2) + "|"]
    for k, cs in sorted(acc.items()):
        n = max(len(v) for v in cs.values())
        vals = [f"{sum(cs[c]) / len(cs[c]):.6g}" if cs.get(c) else "" for c in names]
        out.append(f"| {k} | {n} | " + " | ".join(vals) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    mode, d = sys.argv[1], sys.argv[2]
    print(stats(d) if mode == "stats" else counters(d, sys.argv[3] if len(sys.argv) > 3 else ""))
