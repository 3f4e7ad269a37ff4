"""Benchmark: one tensor-parallel rank's layer shard, forward + backward, on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is the whole path on one micro-batch: tp_attn_fwd, tp_mlp_fwd,
tp_mlp_bwd, tp_attn_bwd (the twelve products, the attention kernels and the
bias-gradient sums), inputs resident in HBM. Throughput is algorithmic flops
per second:
    F = 3 * [2 T h (4 h_l + 2 f_l) + 2 b n_l d s (s + 1)]
(causal attention counts the j <= i triangle; the backward pass is twice the
forward; recomputation and elementwise work are not credited).
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def layer_flops(w, n_l=None, f_l=None) -> float:
    n_l = w.heads_local if n_l is None else n_l
    f_l = w.ffn_local if f_l is None else f_l
    h_l = n_l * w.head_dim
    T, h, b, s, d = w.tokens, w.hidden, w.batch, w.seq, w.head_dim
    return 3.0 * (2.0 * T * h * (4 * h_l + 2 * f_l) + 2.0 * b * n_l * d * s * (s + 1))


def step_flops(w) -> dict:
    """Algorithmic flops of each timed step (per launch sequence)."""
    T, h, hl, fl = w.tokens, w.hidden, w.h_local, w.ffn_local
    att = 2.0 * w.batch * w.heads_local * w.head_dim * w.seq * (w.seq + 1)
    g = lambda m, n, k: 2.0 * m * n * k  # noqa: E731
    return {
        "qkv_proj": g(T, 3 * hl, h), "attn_fwd": att, "out_proj": g(T, h, hl), "fc1": g(T, fl, h),
        "fc2": g(T, h, fl), "fc2_dgrad": g(T, fl, h), "fc2_wgrad": g(fl, h, T), "fc1_wgrad": g(h, fl, T),
        "fc1_dgrad": g(T, h, fl), "out_dgrad": g(T, hl, h), "out_wgrad": g(hl, h, T), "attn_bwd": 2 * att,
        "qkv_wgrad": g(h, 3 * hl, T), "qkv_dgrad": g(T, h, 3 * hl), "bias_grads": 0.0, "transposes": 0.0,
    }


# The GEMM steps (products) of the layer; the library names the kernel each
# one launches for a shape (tp_step_kernel), for the roofline record.
GEMM_STEPS = ("qkv_proj", "out_proj", "fc1", "fc2", "fc2_dgrad", "fc2_wgrad", "fc1_wgrad", "fc1_dgrad", "out_dgrad",
              "out_wgrad", "qkv_wgrad", "qkv_dgrad")


def kernel_of(step, shape) -> str:
    """Name of the kernel the library launches for a step's product."""
    import tensor_transformer_layer_tp_amd as tp
    name = tp.tp_step_kernel(shape, step)
    if name is None:
        raise SystemExit(f"the library names no kernel for step {step}")
    return name


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm_mfma.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "tensor_transformer_layer_tp_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"traffic_bytes_per_launch\s*=\s*([0-9.eE+]+)", text)
    m_h = re.search(r"source_sha256_16\s*=\s*([0-9a-f]+)", text)
    if not (m_b and m_h) or m_h.group(1) != gemm_source_hash():
        return None
    return float(m_b.group(1))


PARITY_OUTS = ("qkv", "ctx", "lse", "O", "pre", "y", "Z", "dX_mlp", "dA", "db1", "dB", "db2", "dX_attn", "dWqkv",
               "dbqkv", "dWo", "dbo")


def saved_qkv_f64(buf, w):
    """q | k | v [T, 3h_l] from the saved projection tp_attn_fwd wrote: the
    bf16 planes 1, 3, 4 of the matrix-core layout, or the fp32 layout."""
    import numpy as np
    import torch
    T, hl = w.tokens, w.h_local
    b = buf.contiguous()
    if w.dtype == "bf16" and w.head_dim in (64, 96, 128, 160):
        n = T * hl
        h16 = b[: 10 * n].view(torch.int16)
        return np.concatenate([h16[k * n:(k + 1) * n].view(torch.bfloat16).double().reshape(T, hl).numpy()
                               for k in (1, 3, 4)], axis=1)
    return b[: 12 * T * hl].view(torch.float32).double().reshape(T, 3 * hl).numpy()


def cpu_baseline(w, inp, target_s: float, gpu_out=None) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    a sub-shard of this rank (its first n_sub heads and first f_sub FFN
    columns; a column block of a column-parallel shard is itself a shard), on
    the same tokens. Rate = algorithmic flops of the sample / wall time. When
    the sample is the whole shard and the GPU step's outputs are given (host
    copies, same inputs), also the relative Frobenius error of every output."""
    import numpy as np
    import oracle
    cores = blas_threads()
    f64 = lambda t: t.double().numpy()  # noqa: E731
    X_attn, X_mlp, dO, dZ = f64(inp["X_attn"]), f64(inp["X_mlp"]), f64(inp["dO"]), f64(inp["dZ"])
    n_l, f_l, d = w.heads_local, w.ffn_local, w.head_dim
    h_l = n_l * d

    def run(n_sub: int, f_sub: int) -> float:
        cols = np.concatenate([np.arange(k * h_l, k * h_l + n_sub * d) for k in range(3)])
        Wqkv = f64(inp["Wqkv"][:, cols])
        bqkv = f64(inp["bqkv"][cols])
        Wo = f64(inp["Wo"][:n_sub * d])
        A, b1, B = f64(inp["A"][:, :f_sub]), f64(inp["b1"][:f_sub]), f64(inp["B"][:f_sub])
        kw = dict(batch=w.batch, seq=w.seq, n_heads=w.n_heads, tp_size=w.n_heads // n_sub, tp_rank=0,
                  alibi=w.alibi)
        t0 = time.perf_counter()
        qkv, ctx, lse, O = oracle.attn_fwd(X_attn, Wqkv, bqkv, Wo, **kw)
        dXa, dWqkv, dbqkv, dWo, dbo = oracle.attn_bwd(X_attn, Wqkv, bqkv, Wo, dO, **kw)
        pre, y, Z = oracle.mlp_fwd(X_mlp, A, b1, B)
        dXm, dA, db1, dB, db2 = oracle.mlp_bwd(X_mlp, A, B, pre, y, dZ)
        t = time.perf_counter() - t0
        outs.clear()
        if n_sub == n_l and f_sub == f_l:
            outs.update(qkv=qkv, ctx=ctx, lse=lse, O=O, pre=pre, y=y, Z=Z, dX_mlp=dXm, dA=dA, db1=db1, dB=dB,
                        db2=db2, dX_attn=dXa, dWqkv=dWqkv, dbqkv=dbqkv, dWo=dWo, dbo=dbo)
        return t

    outs = {}

    k = n_l  # start at 1/n_l of the shard (one head, f_l/n_l FFN columns)
    while True:
        n_sub, f_sub = max(1, n_l // k), max(8, f_l // k)
        t = run(n_sub, f_sub)
        log(f"cpu baseline: {n_sub}/{n_l} heads, {f_sub}/{f_l} ffn columns: {t:.2f} s")
        if t >= target_s / 3 or k == 1 or t * 2 > target_s:
            break
        grow = max(2, 2 ** int(math.log2(max(1.0, target_s / max(t, 1e-3)))))
        k = max(1, k // grow)
        while n_l % k:
            k -= 1
    fl = layer_flops(w, n_l=n_sub, f_l=f_sub)
    res = {"value": fl / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
           "sample": f"fp64 NumPy oracle, fwd+bwd of a sub-shard of rank 0: {n_sub} of {n_l} heads and "
                     f"{f_sub} of {f_l} FFN columns on all {w.tokens} tokens ({fl:.3e} algorithmic flops "
                     f"in {t:.2f} s)"}
    if gpu_out is not None and outs:
        err = {}
        for k in PARITY_OUTS:
            if k in gpu_out and k in outs:
                if k == "qkv":  # the saved projection's bf16 planes (q, k, v), or fp32
                    g, r = saved_qkv_f64(gpu_out[k], w), outs[k]
                else:
                    g, r = f64(gpu_out[k]).reshape(outs[k].shape), outs[k]
                nr = float(np.linalg.norm(r))
                err[k] = float(np.linalg.norm(g - r)) / (nr if nr > 0 else 1.0)
        worst = max(err, key=err.get)
        log(f"parity of the timed step's outputs vs the oracle: worst {worst} rel_fro {err[worst]:.3e}")
        res["parity"] = {"rel_fro": {k: float(f"{v:.3e}") for k, v in err.items()}, "bar": 1e-2,
                         "pass": all(v <= 1e-2 for v in err.values())}
    return res


def ln_residual_measure(w, reps: int = 20) -> dict:
    """The residual add + LayerNorm after a block (outside the layer-shard step
    and its metric): one forward + backward per repetition at the workload's
    T x hidden, bf16, one block output (after g), replicated bias, residual
    gradient. The bias gradient is left to the block's own backward (its
    db2 / dbo column sum of the same gradient), so dbias is not requested.
    HBM-bound: achieved = algorithmic bytes / average launch-sequence time
    (HIP events on the library's stream)."""
    import torch
    import synth
    import tensor_transformer_layer_tp_amd as tp

    inp = synth.draw_ln(w, seed=0, n_parts=1, bias_std=0.02)
    dev = {k: (v.cuda() if torch.is_tensor(v) else [p.cuda() for p in v]) for k, v in inp.items()}
    s = tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                        head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))
    T, h = w.tokens, w.hidden
    bf = torch.bfloat16
    r, y, dr = (torch.empty((T, h), dtype=bf, device="cuda") for _ in range(3))
    mean, rstd = (torch.empty(T, dtype=torch.float32, device="cuda") for _ in range(2))
    dg, db = (torch.empty(h, dtype=bf, device="cuda") for _ in range(2))
    ws = torch.empty(tp.tp_ln_workspace_bytes(s), dtype=torch.uint8, device="cuda")

    def once():
        tp.tp_ln_residual_fwd(s, dev["resid_in"], dev["parts"], dev["bias"], dev["gamma"], dev["beta"], 1e-5, r, y,
                              mean, rstd)
        tp.tp_ln_residual_bwd(s, r, mean, rstd, dev["gamma"], dev["d_ln_out"], dev["d_resid_out"], dr, dg, db,
                              None, workspace=ws)

    for _ in range(3):
        once()
    torch.cuda.synchronize()
    tp.tp_profile_enable((1 << tp.STEPS["ln_fwd"]) | (1 << tp.STEPS["ln_bwd"]))
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    res = {}
    # algorithmic bytes: every tensor once (bf16), statistics fp32
    nbytes = {"fwd": 2 * (3 * T * h + 3 * h) + 2 * T * h + 8 * T,   # resid_in, part, bias, gamma, beta -> r, y, stats
              "bwd": 2 * (3 * T * h + h) + 2 * (T * h + 2 * h) + 8 * T}  # r, dy, dr_in, gamma, stats -> dr, 2 sums
    for name in ("fwd", "bwd"):
        n, ms = tp.tp_profile_collect(tp.STEPS["ln_" + name])
        avg = ms / max(n, 1)
        gbs = nbytes[name] / (avg / 1e3) / 1e9
        res[name] = {"avg_launch_ms": round(avg, 4), "launches": n, "algorithmic_bytes": nbytes[name],
                     "achieved": round(gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS,
                     "frac": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"  ln_residual {name}: {avg * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM)")
    tp.tp_profile_enable(0)
    # the variant with dropout (p = 0.1) on the block output: same tensors plus the
    # keep bytes (T h / 8) written / read and the block-output gradient written
    drop = tp.TpDropout(0.1, 7, 0)
    mask = torch.empty(tp.tp_ln_dropout_mask_bytes(s), dtype=torch.uint8, device="cuda")
    dblk = torch.empty((T, h), dtype=bf, device="cuda")

    def once_do():
        tp.tp_ln_residual_fwd_dropout(s, drop, dev["resid_in"], dev["parts"], dev["bias"], dev["gamma"], dev["beta"],
                                      1e-5, r, y, mean, rstd, mask)
        tp.tp_ln_residual_bwd_dropout(s, drop, r, mean, rstd, dev["gamma"], dev["d_ln_out"], dev["d_resid_out"], mask,
                                      dr, dblk, dg, db, None, workspace=ws)

    for _ in range(3):
        once_do()
    torch.cuda.synchronize()
    tp.tp_profile_enable((1 << tp.STEPS["ln_fwd"]) | (1 << tp.STEPS["ln_bwd"]))
    for _ in range(reps):
        once_do()
    torch.cuda.synchronize()
    extra = {"fwd": T * h // 8, "bwd": T * h // 8 + 2 * T * h}
    for name in ("fwd", "bwd"):
        n, ms = tp.tp_profile_collect(tp.STEPS["ln_" + name])
        avg = ms / max(n, 1)
        gbs = (nbytes[name] + extra[name]) / (avg / 1e3) / 1e9
        res[name + "_dropout_p0.1"] = {"avg_launch_ms": round(avg, 4), "achieved": round(gbs, 1), "unit": "GB/s",
                                       "frac": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"  ln_residual {name} (dropout 0.1): {avg * 1e3:.1f} us, {gbs:.0f} GB/s")
    tp.tp_profile_enable(0)
    return {"bound": "hbm", "workload": f"{w.name}: T={T}, hidden={h}, bf16, 1 block output, bias, residual grad",
            **res}


def vocab_ce_measure(reps: int = 10) -> dict:
    """The vocabulary-parallel output layer (outside the layer-shard step and
    its metric), at the 8.3B-like shard (16384 tokens, hidden 3072) with the
    padded GPT-2 vocabulary of 51,200 over 8 ranks, rank 0 (6,400 vocabulary
    rows): logits GEMM + slice aggregates, the emulated exchange over 8
    ranks' aggregates (rank 0's stand in for all: timing only), dlogits, and
    the input- and table-gradient GEMMs. GEMMs against the MFMA peak (2 T n h
    flops each), the row kernels against HBM (algorithmic bytes)."""
    import torch
    import synth
    import tensor_transformer_layer_tp_amd as tp

    w = synth.WORKLOADS["gpt_8p3b_tp8"]
    V = synth.VOCAB_PADDED
    T, h, n = w.tokens, w.hidden, V // w.tp_size
    inp = synth.draw_vocab(w, V, seed=0, ranks=(0,), dloss="mean")
    s = tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                        head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype)
    X, W0 = inp["X"].cuda(), inp["W"][0].cuda()
    labels, dloss = inp["labels"].cuda(), inp["dloss"].cuda()
    bf = torch.bfloat16
    logits = torch.empty((T, n), dtype=bf, device="cuda")
    stats = torch.empty(3 * T, dtype=torch.float32, device="cuda")
    loss, lse = (torch.empty(T, dtype=torch.float32, device="cuda") for _ in range(2))
    dX = torch.empty((T, h), dtype=bf, device="cuda")
    dW = torch.empty((n, h), dtype=bf, device="cuda")
    ws = torch.empty(tp.tp_vocab_workspace_bytes(s, V), dtype=torch.uint8, device="cuda")

    def once():
        tp.tp_vocab_ce_fwd(s, V, X, W0, labels, logits, stats, workspace=ws)
        tp.tp_vocab_ce_combine(s, [stats] * w.tp_size, loss, lse)
        tp.tp_vocab_ce_bwd(s, V, X, W0, labels, logits, lse, dloss, dX, dW, workspace=ws)

    for _ in range(2):
        once()
    torch.cuda.synchronize()
    names = ("logits", "ce_stats", "ce_combine", "ce_dlogits", "logits_dgrad", "logits_wgrad")
    tp.tp_profile_enable(sum(1 << tp.STEPS[k] for k in names))
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    gemm = 2.0 * T * n * h
    work = {"logits": ("mfma", gemm), "logits_dgrad": ("mfma", gemm), "logits_wgrad": ("mfma", gemm),
            "ce_stats": ("hbm", 2 * T * n + 4 * T + 12 * T),                 # logits, labels -> 3 aggregates
            "ce_combine": ("hbm", 12 * T * w.tp_size + 8 * T),             # every rank's aggregates -> loss, lse
            "ce_dlogits": ("hbm", 2 * T * n * 2 + 12 * T)}                 # logits -> dlogits (+ labels, lse, dloss)
    res, fwd_ms, bwd_ms = {}, 0.0, 0.0
    for k in names:
        cnt, ms = tp.tp_profile_collect(tp.STEPS[k])
        avg = ms / max(cnt, 1)
        bound, amount = work[k]
        if bound == "mfma":
            ach, unit, peak = amount / (avg / 1e3) / 1e12, "TFLOP/s", PEAK_BF16_TFLOPS
        else:
            ach, unit, peak = amount / (avg / 1e3) / 1e9, "GB/s", PEAK_HBM_GBS
        res[k] = {"avg_launch_ms": round(avg, 4), "bound": bound, "achieved": round(ach, 1), "unit": unit,
                  "frac": round(ach / peak, 4)}
        if k in ("logits", "ce_stats", "ce_combine"):
            fwd_ms += avg
        else:
            bwd_ms += avg
        log(f"  vocab {k:12s} {avg * 1e3:8.1f} us  {ach:8.1f} {unit} ({100 * ach / peak:.1f}% of peak)")
    tp.tp_profile_enable(0)
    return {"workload": f"gpt_8p3b_tp8 output layer: T={T}, hidden={h}, vocab {V} over {w.tp_size} ranks "
                        f"(rank 0: {n} rows), bf16", "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "steps": res}


def attn_dropout_measure(w, ls, reps: int = 10) -> dict:
    """Attention-probability dropout variant (outside the step and its metric):
    the attention block's forward and backward at the workload's shape with
    p = 0.1, next to the same calls without dropout, timed over the attention
    steps only (HIP events)."""
    import torch
    import tensor_transformer_layer_tp_amd as tp

    s, i, o = ls.shape, ls.inp, ls.out
    mask = torch.empty(tp.tp_attn_dropout_mask_bytes(s) // 2, dtype=torch.int16, device="cuda")
    drop = tp.TpDropout(0.1, 1234, 0)

    def once(dr):
        if dr is None:
            tp.tp_attn_fwd(s, i["X_attn"], i["Wqkv"], i["bqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"], o["O"],
                           ls.workspace)
            tp.tp_attn_bwd(s, i["X_attn"], i["Wqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"], i["dO"], o["dX_attn"],
                           o["dWqkv"], o["dbqkv"], o["dWo"], o.get("dbo"), ls.workspace)
        else:
            tp.tp_attn_fwd_dropout(s, dr, i["X_attn"], i["Wqkv"], i["bqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"],
                                   mask, o["O"], ls.workspace)
            tp.tp_attn_bwd_dropout(s, dr, i["X_attn"], i["Wqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"], mask,
                                   i["dO"], o["dX_attn"], o["dWqkv"], o["dbqkv"], o["dWo"], o.get("dbo"),
                                   ls.workspace)

    res = {}
    for name, dr in (("p0_plain", None), ("p0.1", drop)):
        for _ in range(2):
            once(dr)
        torch.cuda.synchronize()
        tp.tp_profile_enable((1 << tp.STEPS["attn_fwd"]) | (1 << tp.STEPS["attn_bwd"]))
        for _ in range(reps):
            once(dr)
        torch.cuda.synchronize()
        nf, msf = tp.tp_profile_collect(tp.STEPS["attn_fwd"])
        nb, msb = tp.tp_profile_collect(tp.STEPS["attn_bwd"])
        tp.tp_profile_enable(0)
        res[name] = {"attn_fwd_ms": round(msf / max(nf, 1), 4), "attn_bwd_ms": round(msb / max(nb, 1), 4)}
        log(f"  attention {name:8s}: fwd {res[name]['attn_fwd_ms']:.3f} ms, bwd {res[name]['attn_bwd_ms']:.3f} ms")
    return {"workload": f"{w.name} attention block, bf16, p = 0.1 (Philox4x64-10 keep bits)", **res}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_tiny(reps: int = 100) -> dict:
    """The fp64 oracle on the tiny fp32 workload (both emulated ranks' shards,
    fwd + bwd), averaged over `reps` runs."""
    import oracle
    import synth
    w = synth.WORKLOADS["tiny_fp32_tp2"]
    full = synth.draw_full(w, seed=0)
    a = {k: v.double().numpy() for k, v in full.items()}
    shards = []
    for r in range(w.tp_size):
        shards.append(dict(Wqkv=oracle.qkv_weight_shard(a["Wqkv"], r, w.tp_size),
                           bqkv=oracle.qkv_bias_shard(a["bqkv"], r, w.tp_size),
                           Wo=oracle.row_shard(a["Wo"], r, w.tp_size), A=oracle.column_shard(a["A"], r, w.tp_size),
                           b1=oracle.column_shard(a["b1"], r, w.tp_size), B=oracle.row_shard(a["B"], r, w.tp_size)))

    def once():
        for r, sh in enumerate(shards):
            kw = dict(batch=w.batch, seq=w.seq, n_heads=w.n_heads, tp_size=w.tp_size, tp_rank=r, alibi=w.alibi)
            oracle.attn_fwd(a["X_attn"], sh["Wqkv"], sh["bqkv"], sh["Wo"], **kw)
            oracle.attn_bwd(a["X_attn"], sh["Wqkv"], sh["bqkv"], sh["Wo"], a["dO"], **kw)
            pre, y, _ = oracle.mlp_fwd(a["X_mlp"], sh["A"], sh["b1"], sh["B"])
            oracle.mlp_bwd(a["X_mlp"], sh["A"], sh["B"], pre, y, a["dZ"])

    once()
    t0 = time.perf_counter()
    for _ in range(reps):
        once()
    t = (time.perf_counter() - t0) / reps
    fl = w.tp_size * layer_flops(w)
    return {"workload": w.name, "runs": reps, "avg_s": t, "flops_per_run": fl, "value": fl / t / 1e12,
            "unit": "TFLOP/s", "sample": f"fp64 NumPy oracle, fwd+bwd of both emulated ranks' shards, mean of {reps} runs"}


def time_steps(ls, steps: int, dom_step=None):
    """Run `steps` layer steps on the library's stream bracketed by events:
    -> (ms per step, per-step stats, host wall s, dominant-kernel record).
    With dom_step, every launch sequence of that step is also bracketed by
    events (a separate pass: those events are not in the headline timing)."""
    import torch
    import tensor_transformer_layer_tp_amd as tp
    if dom_step is not None:
        tp.tp_profile_enable(1 << tp.STEPS[dom_step])
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for k in range(steps):
        ls.step()
        (ev[k] if k < steps - 1 else e1).record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / steps
    marks = [e0, *ev, e1]
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(steps))
    stats = {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4),
             "p90": round(per_step[min(len(per_step) - 1, int(math.ceil(0.9 * len(per_step))) - 1)], 4)}
    dom = None
    if dom_step is not None:
        n, ms = tp.tp_profile_collect(tp.STEPS[dom_step])
        tp.tp_profile_enable(0)
        dom = (n, ms / max(n, 1))
    return ms_step, stats, wall, dom


def breakdown_pass(ls, reps: int = 3) -> dict:
    """Per-step GPU time (ms per step) from a pass with events around every step."""
    import torch
    import tensor_transformer_layer_tp_amd as tp
    tp.tp_profile_enable(sum(1 << v for v in tp.STEPS.values()))
    for _ in range(reps):
        ls.step()
    torch.cuda.synchronize()
    out = {}
    for name, sid in tp.STEPS.items():
        n, ms = tp.tp_profile_collect(sid)
        if n:
            out[name] = ms / reps
    tp.tp_profile_enable(0)
    return out


def other_workload(name: str, steps: int, warmup: int) -> dict:
    """One more configuration, timed like the headline one (reported under
    `configs`, not in `value`)."""
    import torch
    import synth
    import tensor_transformer_layer_tp_amd as tp
    from tensor_transformer_layer_tp_amd.shard import INPUTS, LayerShard
    w = synth.WORKLOADS[name]
    log(f"workload {name}: drawing seeded inputs")
    inp = synth.draw_shard(w, seed=0)
    shape = tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                            head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))
    ls = LayerShard(shape, {k: inp[k].cuda() for k in INPUTS})
    del inp
    for _ in range(warmup):
        ls.step()
    torch.cuda.synchronize()
    bd = breakdown_pass(ls)
    ms, stats, _, _ = time_steps(ls, steps)
    F = layer_flops(w)
    tf = F / (ms / 1e3) / 1e12
    sf = step_flops(w)
    tot = sum(bd.values())
    attn = bd.get("attn_fwd", 0.0) + bd.get("attn_bwd", 0.0)
    log(f"  {name}: {ms:.3f} ms/step, {tf:.1f} TFLOP/s ({100 * tf / PEAK_BF16_TFLOPS:.1f}% of peak), "
        f"attention {100 * attn / tot:.1f}% of the step")
    del ls
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "step_ms": stats, "tflops": round(tf, 2),
            "pct_of_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "flops_per_step": F,
            "attention_share_of_step": round(attn / tot, 4),
            "breakdown_ms": {k: round(v, 4) for k, v in bd.items()},
            "breakdown_tflops": {k: round(sf[k] / (v / 1e3) / 1e12, 1) for k, v in bd.items() if sf.get(k)},
            "config": {"batch": w.batch, "seq_len": w.seq, "hidden": w.hidden,
                       "heads": f"{w.heads_local} of {w.n_heads}", "head_dim": w.head_dim,
                       "ffn_shard": f"{w.ffn_local} of {w.ffn}", "tp_rank": 0, "tp_size": w.tp_size,
                       "alibi": w.alibi}}


OTHER_WORKLOADS = ("gpt2_1p2b_tp1", "gpt_8p3b_tp8", "bloom_176b_tp8")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mtnlg_530b_tp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ln", action="store_true", help="skip the residual + LayerNorm measurement")
    ap.add_argument("--no-vocab", action="store_true", help="skip the vocabulary-parallel output-layer measurement")
    ap.add_argument("--no-dropout", action="store_true", help="skip the attention-dropout measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip timing the other bf16 workloads")
    ap.add_argument("--cpu-target-s", type=float, default=15.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run device-to-device copies of this many MiB (calibrates byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {a.gpus} requested): it runs one tensor-parallel "
              "rank's shard on one device; runs on several GPUs are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    if a.copy_probe_mib:
        n = a.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x5")
        return

    import synth
    import tensor_transformer_layer_tp_amd as tp
    from tensor_transformer_layer_tp_amd.shard import INPUTS, LayerShard

    w = synth.WORKLOADS[a.workload]
    if w.dtype != "bf16":
        raise SystemExit("the benchmark runs the bf16 workloads")
    tp.load_library()
    log(f"workload {w.name}: drawing seeded inputs")
    inp = synth.draw_shard(w, seed=0)
    shape = tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                            head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))
    dev = {k: inp[k].cuda() for k in INPUTS}
    ls = LayerShard(shape, dev)
    torch.cuda.synchronize()
    log(f"warmup {a.warmup} steps")
    for _ in range(a.warmup):
        ls.step()
    torch.cuda.synchronize()

    # per-step breakdown (separate pass, every step bracketed by events)
    sf = step_flops(w)
    breakdown = breakdown_pass(ls)
    tot = sum(breakdown.values())
    for name, ms in sorted(breakdown.items(), key=lambda kv: -kv[1]):
        tf = sf[name] / (ms / 1e3) / 1e12 if ms > 0 else 0.0
        log(f"  {name:11s} {ms:8.3f} ms  {100 * ms / tot:5.1f}%  {tf:7.1f} TFLOP/s  {100 * tf / PEAK_BF16_TFLOPS:5.1f}% peak")
    gemm_steps = {k: v for k, v in breakdown.items() if k in GEMM_STEPS}
    dom = max(gemm_steps, key=gemm_steps.get)
    kernel = kernel_of(dom, shape)

    # the timed region: K steps, events only between steps
    log(f"timing {a.steps} steps")
    ms_step, step_stats, wall, _ = time_steps(ls, a.steps)
    # host copies of the timed step's outputs (later measurements reuse the buffers)
    gpu_out = None if a.no_cpu_baseline else {k: v.cpu() for k, v in ls.out.items()}
    F = layer_flops(w)
    value = F / (ms_step / 1e3) / 1e12
    log(f"{ms_step:.3f} ms/step, {value:.1f} TFLOP/s ({100 * value / PEAK_BF16_TFLOPS:.1f}% of peak); "
        f"host wall {wall:.3f} s for {a.steps} steps")
    # the same K steps again with the dominant kernel's launches bracketed by
    # events on the library's stream (its average launch time for the roofline)
    log(f"timing {a.steps} steps again with events around the dominant kernel ({kernel})")
    ms_step2, _, _, (n_dom, avg_dom_ms) = time_steps(ls, a.steps, dom_step=dom)
    achieved = sf[dom] / (avg_dom_ms / 1e3) / 1e12
    traffic = stored_traffic(kernel, w.name)
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": kernel,
            "flops_per_launch": sf[dom], "avg_launch_ms": round(avg_dom_ms, 4), "launches": n_dom,
            "ms_per_step_of_that_pass": round(ms_step2, 4)}

    configs = {}
    if not a.no_configs:
        del ls, dev
        torch.cuda.empty_cache()
        log("the other bf16 configurations (timed like the headline one)")
        configs[w.name] = {"ms_per_step": round(ms_step, 4), "tflops": round(value, 2),
                           "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                           "attention_share_of_step": round((breakdown.get("attn_fwd", 0) + breakdown.get("attn_bwd", 0)) / tot, 4)}
        for name in OTHER_WORKLOADS:
            if name != w.name:
                configs[name] = other_workload(name, a.steps, a.warmup)
        dev = {k: inp[k].cuda() for k in INPUTS}
        ls = LayerShard(shape, dev)
        ls.step()
        torch.cuda.synchronize()

    ln = None
    if not a.no_ln:
        log("residual add + LayerNorm (measured apart from the step)")
        ln = ln_residual_measure(w)

    adrop = None
    if not a.no_dropout:
        log("attention-probability dropout (measured apart from the step)")
        adrop = attn_dropout_measure(w, ls)

    vocab = None
    if not a.no_vocab:
        log("vocabulary-parallel logits + cross-entropy (measured apart from the step)")
        vocab = vocab_ce_measure()

    cpu = None
    if not a.no_cpu_baseline:
        log("cpu baseline (fp64 oracle on a bounded sample)")
        cpu = cpu_baseline(w, inp, a.cpu_target_s, gpu_out)
        gpu_out = None
        cpu["cpu_model"] = cpu_model()
        log("cpu baseline on the tiny fp32 workload (mean of 100 runs)")
        cpu["tiny_fp32_tp2"] = cpu_baseline_tiny()

    out = {
        "metric": "layer-shard fwd+bwd TFLOP/s (bf16) on 1 MI355X; % of MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4), "step_ms": step_stats, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) activations and gradients, N(0,0.02) weights)",
        "pct_of_mfma_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seq, "hidden": w.hidden,
                   "heads": f"{w.heads_local} of {w.n_heads}", "head_dim": w.head_dim,
                   "ffn_shard": f"{w.ffn_local} of {w.ffn}", "tp_rank": 0, "tp_size": w.tp_size,
                   "alibi": w.alibi, "flops_per_step": F},
        "breakdown_ms": {k: round(v, 4) for k, v in breakdown.items()},
        "breakdown_tflops": {k: round(sf[k] / (v / 1e3) / 1e12, 1) for k, v in breakdown.items() if sf[k] > 0},
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": configs or None,
        "ln_residual": ln,
        "vocab_ce": vocab,
        "attn_dropout": adrop,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
