"""Comparison helpers shared by the GPU parity tests (HIP path vs fp64 oracle)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Relative Frobenius bound per storage type (the stated bar); the element-wise
# bound |gpu - ref| <= a * scale + b * |ref| catches a localized error (a wrong
# tile errs by ~rms) that a norm over millions of elements hides. One band for
# every output (qkv is kept in fp32 and the scores are formed from fp16 q and
# k, so the outputs downstream of the softmax need no wider band). `scale` is the larger of the output's rms and the rms of the
# element's own row: the rounding of a bf16 intermediate errs in proportion to
# the magnitudes of its row, and some rows are far above the average (the first
# token's key and value gradients collect every query's contribution; in a
# d = 160 shard its input-gradient row is 13x the global rms, and the bf16
# rounding of dqkv alone puts one of its elements at 1.1x a band scaled by the
# global rms, 0.10x one scaled by the row's).
FRO_TOL = {"fp32": 1e-5, "bf16": 1e-2}
ELEM_TOL = {"fp32": (2e-5, 1e-5), "bf16": (0.08, 0.02)}  # (x scale, x |ref|)


def band_scale(r: np.ndarray):
    """max(rms of r, rms of each row of r) for matrices; rms of r otherwise."""
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    if r.ndim == 2 and r.shape[1] > 1 and r.size:
        return np.maximum(rms, np.sqrt(np.mean(r * r, axis=1, keepdims=True)))
    return rms


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def compare(name: str, gpu, ref, dtype: str, report: dict | None = None, verbose: bool = True):
    g, r = f64(gpu), f64(ref)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values in the HIP output"
    nr = np.linalg.norm(r)
    err = np.linalg.norm(g - r) / (nr if nr > 0 else 1.0)
    a, b = ELEM_TOL[dtype]
    scale = band_scale(r)
    worst = float(np.max(np.abs(g - r) / (a * scale + b * np.abs(r) + 1e-300))) if r.size else 0.0
    if report is not None:
        report[name] = {"rel_fro": float(err), "worst_over_band": worst}
    if verbose:
        print(f"    {name:14s} rel_fro {err:.3e} (bar {FRO_TOL[dtype]:.0e})  worst element / band {worst:.3f}",
              flush=True)
    assert err <= FRO_TOL[dtype], f"{name}: relative Frobenius error {err:.3e} > {FRO_TOL[dtype]:.0e}"
    if r.size:
        bad = np.abs(g - r) > a * scale + b * np.abs(r)
        if np.any(bad):
            idx = np.argwhere(bad)[0]
            sc = float(np.broadcast_to(scale, r.shape)[tuple(idx)])
            raise AssertionError(f"{name}: {int(bad.sum())} elements out of bound, first at {tuple(idx)}: "
                                 f"gpu {g[tuple(idx)]:.6g} ref {r[tuple(idx)]:.6g} scale {sc:.3g}")
    return err


MFMA_HEAD_DIMS = (64, 96, 128, 160)


def saved_qkv(buf, T: int, hl: int, head_dim: int, dtype: str):
    """The saved projection qkv_i as written by tp_attn_fwd, decoded for
    comparison: -> (qkv [T, 3hl] float64 from the bf16 planes (or the fp32
    buffer), q16 and k16 [T, hl] float64 from the fp16 planes with q16's
    log2(e)/sqrt(d) factor divided out (None on the fp32 layout))."""
    b = buf.detach().to("cpu").contiguous()
    if dtype == "bf16" and head_dim in MFMA_HEAD_DIMS:
        n = T * hl
        h16 = b[: 10 * n].view(torch.int16)
        plane = lambda k, dt: h16[k * n:(k + 1) * n].view(dt).to(torch.float64).reshape(T, hl).numpy()  # noqa: E731
        qkv = np.concatenate([plane(1, torch.bfloat16), plane(3, torch.bfloat16), plane(4, torch.bfloat16)], axis=1)
        qscale = 1.4426950408889634 / np.sqrt(head_dim)
        return qkv, plane(0, torch.float16) / qscale, plane(2, torch.float16)
    return b[: 12 * T * hl].view(torch.float32).to(torch.float64).reshape(T, 3 * hl).numpy(), None, None


def compare_saved_qkv(buf, ref_qkv, T, hl, head_dim, dtype, report=None):
    """The bf16 (or fp32) copy of the projection against the oracle's, and the
    fp16 score copies of q and k against its q and k."""
    qkv, q16, k16 = saved_qkv(buf, T, hl, head_dim, dtype)
    compare("qkv", qkv, ref_qkv, dtype, report)
    if q16 is not None:
        compare("qkv(q fp16)", q16, ref_qkv[:, :hl], "bf16", report)
        compare("qkv(k fp16)", k16, ref_qkv[:, hl:2 * hl], "bf16", report)


def oracle_rank(w, inp: dict, rank: int, alibi=None) -> dict:
    """Full oracle for one rank's shard (small shapes)."""
    a = {k: f64(v) for k, v in inp.items()}
    alibi = w.alibi if alibi is None else alibi
    kw = dict(batch=w.batch, seq=w.seq, n_heads=w.n_heads, tp_size=w.tp_size, tp_rank=rank, alibi=alibi)
    qkv, ctx, lse, O = oracle.attn_fwd(a["X_attn"], a["Wqkv"], a["bqkv"], a["Wo"], **kw)
    dXa, dWqkv, dbqkv, dWo, dbo = oracle.attn_bwd(a["X_attn"], a["Wqkv"], a["bqkv"], a["Wo"], a["dO"], **kw)
    pre, y, Z = oracle.mlp_fwd(a["X_mlp"], a["A"], a["b1"], a["B"])
    dXm, dA, db1, dB, db2 = oracle.mlp_bwd(a["X_mlp"], a["A"], a["B"], pre, y, a["dZ"])
    return dict(qkv=qkv, ctx=ctx, lse=lse, O=O, pre=pre, y=y, Z=Z, dX_mlp=dXm, dA=dA, db1=db1, dB=dB, db2=db2,
                dX_attn=dXa, dWqkv=dWqkv, dbqkv=dbqkv, dWo=dWo, dbo=dbo)


def shape_of(w, rank: int, **kw):
    import tensor_transformer_layer_tp_amd as tp
    return tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                           head_dim=w.head_dim, tp_rank=rank, tp_size=w.tp_size, dtype=w.dtype,
                           alibi=int(kw.get("alibi", w.alibi)))


def shard_of_full(full: dict, rank: int, tp: int) -> dict:
    """One rank's inputs sliced from the unsharded draw (column / row / head split)."""
    out = {}
    for k, v in full.items():
        n = v.numpy() if v.dtype != torch.bfloat16 else v.view(torch.int16).numpy()
        if k == "Wqkv" or k == "bqkv":
            s = oracle.qkv_weight_shard(n, rank, tp)
        elif k in ("A", "b1"):
            s = oracle.column_shard(n, rank, tp)
        elif k in ("Wo", "B"):
            s = oracle.row_shard(n, rank, tp)
        else:
            s = n
        t = torch.from_numpy(np.ascontiguousarray(s))
        out[k] = t.view(torch.bfloat16) if v.dtype == torch.bfloat16 else t
    return out
