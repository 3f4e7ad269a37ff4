"""Summaries of rocprofv3 CSV output for the layer-shard kernels.

    python -m tensor_transformer_layer_tp_amd.profsum stats  <dir>            # per-kernel durations
    python -m tensor_transformer_layer_tp_amd.profsum counters <dir> [filter] # per-kernel counter means
    python -m tensor_transformer_layer_tp_amd.profsum util <sq_dir> <mem_dir>  # MFMA busy, LDS, TA, L2, DRAM
    python -m tensor_transformer_layer_tp_amd.profsum traffic <fetch_dir> <write_dir> \
        <copy_fetch_dir> <copy_write_dir> <copy_bytes> <kernel>                # HBM bytes per launch

<dir> is a rocprofv3 output directory written with --output-format csv. The
counter summary averages every counter over the dispatches of each kernel
whose name contains `filter`.
"""
from __future__ import annotations

import csv
import glob
import os
import re
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
    n = name.replace("void ", "").replace("(anonymous namespace)::", "").replace("tpk::", "")
    m = re.match(r"_ZN3tpk12_GLOBAL__N_1(\d+)", n)  # a mangled name the tracer left as is
    if m:
        k = int(m.group(1))
        base = n[m.end():m.end() + k]
        rest = n[m.end() + k:]
        if not rest.startswith("I"):
            return base
        args, rest = [], rest[1:]
        while rest and not rest.startswith("E"):
            t = re.match(r"DF16b|f|Li(\d+)E|Lb([01])E", rest)
            if not t:
                break
            tok = t.group(0)
            args.append("bf16" if tok == "DF16b" else "float" if tok == "f" else t.group(1) if t.group(1)
                        else ("true" if t.group(2) == "1" else "false"))
            rest = rest[t.end():]
        return base + ("<" + ", ".join(args) + ">" if args else "")
    return n.split("(")[0]


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


XCDS, CUS, SIMDS = 8, 256, 1024  # MI355X: GRBM_GUI_ACTIVE is summed over its 8 XCDs


def _per_kernel(d: str):
    acc = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    for r in _rows(d, "counter_collection.csv"):
        k = short(r["Kernel_Name"])
        acc[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}
    return mean, {k: sum(v) / len(v) for k, v in dur.items()}, {k: len(v) for k, v in dur.items()}


def util(sq_dir: str, mem_dir: str, top: int = 16) -> str:
    """Per kernel, from a pass of SQ counters and a pass of memory counters
    (each with GRBM_GUI_ACTIVE): the shader clock it ran at (busy cycles per
    XCD over the dispatch's duration), MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES over
    1024 SIMDs x those cycles, the MfmaUtil definition), LDS active and
    bank-conflict cycles per CU, TA busy and TCP pending-data stall per CU, the
    L2 hit rate and the L2's DRAM-side read and write requests (x 64 bytes)."""
    A, dA, nA = _per_kernel(sq_dir)
    B, _, _ = _per_kernel(mem_dir)
    out = ["| kernel | dispatches | avg us | clock GHz | MFMA busy % | LDS active % | LDS bank-conflict % | "
           "TA busy % | TCP pending stall % | L2 hit % | DRAM read GB | DRAM write GB |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(A, key=lambda k: -dA.get(k, 0))[:top]:
        a, b = A[k], B.get(k, {})
        cyc = a["GRBM_GUI_ACTIVE"] / XCDS
        bc = b.get("GRBM_GUI_ACTIVE", 0) / XCDS or 1.0
        hit, miss = b.get("TCC_HIT_sum", 0.0), b.get("TCC_MISS_sum", 0.0)
        out.append(
            f"| {k} | {nA[k]} | {dA[k] / 1e3:.1f} | {cyc / dA[k]:.2f} | "
            f"{100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc):.1f} | "
            f"{100 * a['SQ_LDS_IDX_ACTIVE'] / (CUS * cyc):.1f} | {100 * a['SQ_LDS_BANK_CONFLICT'] / (CUS * cyc):.1f} | "
            f"{100 * b.get('TA_TA_BUSY_sum', 0) / (CUS * bc):.1f} | "
            f"{100 * b.get('TCP_PENDING_STALL_CYCLES_sum', 0) / (CUS * bc):.1f} | "
            f"{100 * hit / max(hit + miss, 1):.1f} | {b.get('TCC_EA0_RDREQ_DRAM_sum', 0) * 64 / 1e9:.3f} | "
            f"{b.get('TCC_EA0_WRREQ_DRAM_sum', 0) * 64 / 1e9:.3f} |")
    return "\n".join(out)


def _mean(d: str, counter: str, kernel: str) -> float:
    v = [float(r["Counter_Value"]) for r in _rows(d, "counter_collection.csv")
         if r["Counter_Name"] == counter and short(r["Kernel_Name"]) == kernel]
    if not v:
        raise SystemExit(f"no {counter} rows for {kernel} under {d}")
    return sum(v) / len(v)


def traffic(fetch_dir: str, write_dir: str, copyf_dir: str, copyw_dir: str, copy_bytes: int, kernel: str) -> str:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of `kernel`, each scaled by
    the factor that makes a device copy of copy_bytes read and write exactly
    copy_bytes."""
    cf = copy_bytes / (_mean(copyf_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer") * 1024)
    cw = copy_bytes / (_mean(copyw_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer") * 1024)
    f = _mean(fetch_dir, "FETCH_SIZE", kernel) * 1024 * cf
    w = _mean(write_dir, "WRITE_SIZE", kernel) * 1024 * cw
    here = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, os.path.dirname(here))
    import bench  # noqa: E402  (source hash of the GEMM kernels)
    return "\n".join([
        f"calibration: copy of {copy_bytes} bytes -> FETCH_SIZE x {cf:.4f}, WRITE_SIZE x {cw:.4f}",
        f"fetch_bytes_per_launch = {f:.6e}",
        f"write_bytes_per_launch = {w:.6e}",
        f"traffic_bytes_per_launch = {f + w:.6e}",
        f"source_sha256_16 = {bench.gemm_source_hash()}",
    ])


def hbm(fetch_dir: str, write_dir: str, copyf_dir: str, copyw_dir: str, copy_bytes: int, *prefixes: str) -> str:
    """Bandwidth-bound kernels (short names starting with one of `prefixes`):
    per dispatch, FETCH_SIZE and WRITE_SIZE scaled as in `traffic`, the
    dispatch's duration (from the GRBM_GUI_ACTIVE rows of the FETCH_SIZE pass)
    and the rate those bytes give against the 8 TB/s of HBM3E."""
    cf = copy_bytes / (_mean(copyf_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer") * 1024)
    cw = copy_bytes / (_mean(copyw_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer") * 1024)
    F, dF, nF = _per_kernel(fetch_dir)
    W, _, _ = _per_kernel(write_dir)
    out = [f"calibration: copy of {copy_bytes} bytes -> FETCH_SIZE x {cf:.4f}, WRITE_SIZE x {cw:.4f}", "",
           "| kernel | dispatches | avg us | fetched MB | written MB | GB/s | % of 8 TB/s |",
           "|---|---|---|---|---|---|---|"]
    for k in sorted(F, key=lambda k: -dF.get(k, 0)):
        if not k.startswith(prefixes) or k not in dF:
            continue
        f = F[k].get("FETCH_SIZE", 0.0) * 1024 * cf
        w = W.get(k, {}).get("WRITE_SIZE", 0.0) * 1024 * cw
        gbs = (f + w) / dF[k]  # bytes per ns = GB/s
        out.append(f"| {k} | {nF[k]} | {dF[k] / 1e3:.1f} | {f / 1e6:.1f} | {w / 1e6:.1f} | {gbs:.0f} | "
                   f"{100 * gbs / 8000:.1f} |")
    return "\n".join(out)


if __name__ == "__main__":
    mode, d = sys.argv[1], sys.argv[2]
    if mode == "stats":
        print(stats(d))
    elif mode == "counters":
        print(counters(d, sys.argv[3] if len(sys.argv) > 3 else ""))
    elif mode == "util":
        print(util(d, sys.argv[3], int(sys.argv[4]) if len(sys.argv) > 4 else 16))
    elif mode == "hbm":
        print(hbm(d, sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), *sys.argv[7:]))
    elif mode == "traffic":
        print(traffic(d, sys.argv[3], sys.argv[4], sys.argv[5], int(sys.argv[6]), sys.argv[7]))
    else:
        raise SystemExit(f"unknown mode {mode}")
