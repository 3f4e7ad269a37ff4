"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Small shapes compare every element of every output; the
full-size workloads compare sampled outputs the oracle computes exactly
(column sub-shards, rows, heads) plus the complete attention outputs."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import compare, compare_saved_qkv, f64, oracle_rank, shape_of, shard_of_full

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")
from tensor_transformer_layer_tp_amd.shard import INPUTS, LayerShard  # noqa: E402

OUTS = ("qkv", "ctx", "lse", "O", "pre", "y", "Z", "dX_mlp", "dA", "db1", "dB", "db2", "dX_attn", "dWqkv", "dbqkv",
        "dWo", "dbo")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def run_shard(w, inp, rank, fill=float("nan"), alibi=None):
    kw = {} if alibi is None else {"alibi": alibi}
    s = shape_of(w, rank, **kw)
    dev = {k: inp[k].cuda().contiguous() for k in INPUTS}
    ls = LayerShard(s, dev, fill=fill)
    ls.step()
    torch.cuda.synchronize()
    return ls


def _recording(rep: dict):
    """compare() that also keeps each output's errors in rep."""
    def cmp(name, gpu, ref, dtype):
        return compare(name, gpu, ref, dtype, rep)
    return cmp


def _write_report(case: str, rep: dict):
    """Per-output errors of a full-size case, as JSON under the directory named
    by TP_PARITY_REPORT_DIR (nothing is written when it is unset)."""
    import json
    import os
    out = os.environ.get("TP_PARITY_REPORT_DIR")
    if not out:
        return
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, f"{case}.json"), "w") as fh:
        json.dump(rep, fh, indent=1)


def check_all(ls, ref, dtype, names=OUTS):
    rep = {}
    s = ls.shape
    T, hl = s.batch * s.seq, s.n_heads // s.tp_size * s.head_dim
    for k in names:
        if k == "qkv":
            compare_saved_qkv(ls.out[k], ref[k], T, hl, s.head_dim, dtype, rep)
        else:
            compare(k, ls.out[k], ref[k], dtype, rep)
    return rep


# ---------------------------------------------------------------------------
# Tiny fp32 layer, TP = 2 emulated: both ranks, then the f / g sums.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["as_specified", "biases_alibi"])
def test_tiny_fp32_tp2_both_ranks_and_sums(variant):
    w = synth.WORKLOADS["tiny_fp32_tp2"]
    if variant == "biases_alibi":
        w = w.with_(bias_std=0.5, alibi=True)
    full = synth.draw_full(w, seed=0)
    parts = {"Z": [], "O": [], "dX_mlp": [], "dX_attn": []}
    shards = []
    for r in range(w.tp_size):
        inp = shard_of_full(full, r, w.tp_size)
        ls = run_shard(w, inp, r)
        ref = oracle_rank(w, inp, r)
        check_all(ls, ref, "fp32")
        for k in parts:
            parts[k].append(ls.out[k])
        shards.append(ls)
    # emulated g (forward) and f (backward): sum of the ranks' partials
    s = shape_of(w, 0)
    fu = {k: f64(v) for k, v in full.items()}
    w1 = w.with_(tp_size=1)
    ref1 = oracle_rank(w1, full, 0)
    for k, bias in (("Z", "b2"), ("O", "bo"), ("dX_mlp", None), ("dX_attn", None)):
        out = torch.empty_like(parts[k][0])
        b = full[bias].cuda() if bias else None
        tp.tp_sum_partials(s, parts[k], b, out)
        torch.cuda.synchronize()
        want = ref1[k] + (fu[bias] if bias else 0.0)
        compare(f"sum({k})", out, want, "fp32")


# ---------------------------------------------------------------------------
# Small bf16 shards: several tiles, ragged tails, every head width.
# ---------------------------------------------------------------------------

SMALL = [
    # name, batch, seq, n_heads, head_dim, tp_size, rank, alibi
    ("d64_tp2_r1", 2, 200, 4, 64, 2, 1, False),
    ("d96_tp2_r0_alibi", 1, 300, 6, 96, 2, 0, True),
    ("d128_tp1_alibi", 2, 130, 4, 128, 1, 0, True),
    ("d160_tp2_r1", 1, 257, 4, 160, 2, 1, False),
    ("d16_tp2_r1_vector_path", 2, 40, 8, 16, 2, 1, True),
    ("d128_tp4_r3_seq1", 3, 1, 8, 128, 4, 3, True),
    # longer, ragged sequences: many key tiles per query tile, partial last tiles
    ("d64_tp1_alibi_long_ragged", 1, 777, 2, 64, 1, 0, True),
    ("d160_tp2_r0_long_ragged", 2, 1100, 4, 160, 2, 0, False),
    ("d96_tp1_long_ragged", 1, 1025, 2, 96, 1, 0, False),
    ("d128_tp2_r1_alibi_long_ragged", 2, 1300, 4, 128, 2, 1, True),
]


# Wide layers (hidden >= 8192) give the weight gradients transposed copies of
# one operand (y^T, dPre^T, ctx^T, dqkv^T, with the bias gradients' column
# partials); these token counts make the copies mostly padding (T < 8, a
# ragged 8-row group, a partial 32-row run) and K = T a single partial k-step.
@pytest.mark.parametrize("batch,seq", [(3, 1), (1, 77)], ids=["T3", "T77"])
def test_wide_layer_weight_gradient_copies_few_tokens(batch, seq):
    w = synth.Workload(f"wide_copies_T{batch * seq}", batch=batch, seq=seq, hidden=8192, n_heads=64, head_dim=128,
                       ffn=8192, tp_size=8, dtype="bf16", alibi=False, bias_std=0.5)
    inp = synth.draw_shard(w, seed=5)
    ls = run_shard(w, inp, 5)
    check_all(ls, oracle_rank(w, inp, 5), "bf16")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_bf16_shard_matches_oracle(case):
    name, batch, seq, nh, d, tps, rank, alibi = case
    h = nh * d
    w = synth.Workload(name, batch=batch, seq=seq, hidden=h, n_heads=nh, head_dim=d, ffn=4 * h, tp_size=tps,
                       dtype="bf16", alibi=alibi, bias_std=0.5)
    inp = synth.draw_shard(w, seed=1)
    ls = run_shard(w, inp, rank)
    check_all(ls, oracle_rank(w, inp, rank), "bf16")


def test_small_fp32_shard_every_rank_alibi():
    w = synth.Workload("fp32_tp4", batch=2, seq=45, hidden=128, n_heads=8, head_dim=16, ffn=512, tp_size=4,
                       dtype="fp32", alibi=True, bias_std=0.5)
    for r in range(4):
        inp = synth.draw_shard(w, seed=2 + r)
        check_all(run_shard(w, inp, r), oracle_rank(w, inp, r), "fp32")


# ---------------------------------------------------------------------------
# Emulated tensor parallelism in bf16: the sum over p ranks equals the
# unsharded layer, and the ranks' weight gradients tile the unsharded ones.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tps", [2, 4])
def test_emulated_tp_bf16_equals_unsharded(tps):
    w = synth.Workload("emu", batch=2, seq=96, hidden=512, n_heads=4, head_dim=128, ffn=2048, tp_size=tps,
                       dtype="bf16", alibi=True, bias_std=0.5)
    full = synth.draw_full(w, seed=3)
    w1 = w.with_(tp_size=1)
    ref = oracle_rank(w1, full, 0)
    fu = {k: f64(v) for k, v in full.items()}
    outs = [run_shard(w, shard_of_full(full, r, tps), r) for r in range(tps)]
    s = shape_of(w, 0)
    for k, bias in (("Z", "b2"), ("O", "bo"), ("dX_mlp", None), ("dX_attn", None)):
        out = torch.empty_like(outs[0].out[k])
        tp.tp_sum_partials(s, [o.out[k] for o in outs], full[bias].cuda() if bias else None, out)
        torch.cuda.synchronize()
        compare(f"sum({k})", out, ref[k] + (fu[bias] if bias else 0.0), "bf16")
    cat = lambda k, ax: np.concatenate([f64(o.out[k]) for o in outs], axis=ax)  # noqa: E731
    compare("cat(dA)", cat("dA", 1), ref["dA"], "bf16")
    compare("cat(db1)", cat("db1", 0), ref["db1"], "bf16")
    compare("cat(dB)", cat("dB", 0), ref["dB"], "bf16")
    compare("cat(dWo)", cat("dWo", 0), ref["dWo"], "bf16")
    dW = [oracle.qkv_weight_shard(ref["dWqkv"], r, tps) for r in range(tps)]
    for r, o in enumerate(outs):
        compare(f"dWqkv[{r}]", o.out["dWqkv"], dW[r], "bf16")
        compare(f"lse[{r}]", o.out["lse"], ref["lse"][:, r * (w.n_heads // tps):(r + 1) * (w.n_heads // tps)], "bf16")


# ---------------------------------------------------------------------------
# Edge cases: empty batch, every output written, determinism.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,hidden", [("fp32", 256), ("bf16", 256), ("bf16", 8192)],
                         ids=["fp32", "bf16", "bf16_wide_copies"])
def test_empty_batch_gives_zero_weight_grads(dtype, hidden):
    # hidden 8192: the weight gradients' copy path (no copies are made; the
    # bias-gradient final passes see zero partial rows)
    w = synth.Workload("empty", batch=0, seq=64, hidden=hidden, n_heads=hidden // 128, head_dim=128, ffn=1024,
                       tp_size=2, dtype=dtype)
    inp = synth.draw_shard(w, seed=4)
    ls = run_shard(w, inp, 1)
    for k in ("dA", "db1", "dB", "db2", "dWqkv", "dbqkv", "dWo", "dbo"):
        assert torch.all(ls.out[k] == 0), k


def test_deterministic_repeat():
    w = synth.Workload("det", batch=2, seq=200, hidden=640, n_heads=4, head_dim=160, ffn=2560, tp_size=1,
                       dtype="bf16", bias_std=0.5)
    inp = synth.draw_shard(w, seed=5)
    a = run_shard(w, inp, 0)
    first = {k: v.clone() for k, v in a.out.items()}
    a.step()
    torch.cuda.synchronize()
    for k, v in a.out.items():
        assert torch.equal(v, first[k]), k


# ---------------------------------------------------------------------------
# The four named workloads at full size, in the launch configuration the
# benchmark times (rank 0 of the shard; every output sampled or complete).
# ---------------------------------------------------------------------------

# (workload, rank): rank 0 of each, and the last rank of the ALiBi workload,
# whose heads (global 99..112 of 112) carry the smallest slopes, down to 2^-8.
FULL = [("gpt2_1p2b_tp1", 0), ("gpt_8p3b_tp8", 0), ("mtnlg_530b_tp8", 0), ("bloom_176b_tp8", 0),
        ("bloom_176b_tp8", 7)]


@pytest.mark.parametrize("name,rank", FULL, ids=[f"{n}_r{r}" for n, r in FULL])
def test_full_size_workload(name, rank):
    w = synth.WORKLOADS[name]
    print(f"[full-size] {name} rank {rank}: drawing inputs", flush=True)
    inp = synth.draw_shard(w, seed=0)
    print(f"[full-size] {name} rank {rank}: running the HIP path", flush=True)
    ls = run_shard(w, inp, rank)
    out = ls.out
    rep = {}
    compare = _recording(rep)
    rng = np.random.default_rng(7)
    T, h, fl = w.tokens, w.hidden, w.ffn_local
    hl, nl, d = w.h_local, w.heads_local, w.head_dim
    a = {k: f64(inp[k]) for k in INPUTS}
    print(f"[full-size] {name} rank {rank}: oracle on sampled outputs", flush=True)
    # MLP: a column sub-shard C of the rank's FFN columns is itself a valid shard
    C = np.unique(np.concatenate([[0, 1, fl // 2, fl - 1], rng.choice(fl, 60, replace=False)]))
    pre_C, y_C, _ = oracle.mlp_fwd(a["X_mlp"], a["A"][:, C], a["b1"][C], a["B"][C, :])
    compare("pre[:,C]", out["pre"][:, C], pre_C, "bf16")
    compare("y[:,C]", out["y"][:, C], y_C, "bf16")
    _, dA_C, db1_C, dB_C, db2 = oracle.mlp_bwd(a["X_mlp"], a["A"][:, C], a["B"][C, :], pre_C, y_C, a["dZ"])
    compare("dA[:,C]", out["dA"][:, C], dA_C, "bf16")
    compare("db1[C]", out["db1"][C], db1_C, "bf16")
    compare("dB[C,:]", out["dB"][C, :], dB_C, "bf16")
    compare("db2", out["db2"], db2, "bf16")
    # MLP rows R (the block is row-wise independent)
    R = np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.choice(T, 12, replace=False)]))
    pre_R, y_R, Z_R = oracle.mlp_fwd(a["X_mlp"][R], a["A"], a["b1"], a["B"])
    compare("Z[R]", out["Z"][R], Z_R, "bf16")
    dX_R = oracle.mlp_bwd(a["X_mlp"][R], a["A"], a["B"], pre_R, y_R, a["dZ"][R])[0]
    compare("dX_mlp[R]", out["dX_mlp"][R], dX_R, "bf16")
    # attention: the complete per-head core, projections sampled
    kw = dict(batch=w.batch, seq=w.seq, n_local=nl, head_dim=d, head0=rank * nl, n_heads=w.n_heads, alibi=w.alibi)
    qkv = a["X_attn"] @ a["Wqkv"] + a["bqkv"]
    compare_saved_qkv(out["qkv"], qkv, T, hl, d, "bf16", rep)
    ctx, lse = oracle.attn_core_fwd(qkv, **kw)
    compare("ctx", out["ctx"], ctx, "bf16")
    compare("lse", out["lse"], lse, "bf16")
    compare("O[R]", out["O"][R], ctx[R] @ a["Wo"], "bf16")
    dC = a["dO"] @ a["Wo"].T
    dqkv = oracle.attn_core_bwd(qkv, dC, **kw)
    Ch = np.unique(np.concatenate([[0, h - 1], rng.choice(h, 30, replace=False)]))
    compare("dWo[:,Ch]", out["dWo"][:, Ch], ctx.T @ a["dO"][:, Ch], "bf16")
    C3 = np.unique(np.concatenate([[0, 3 * hl - 1], rng.choice(3 * hl, 60, replace=False)]))
    compare("dWqkv[:,C3]", out["dWqkv"][:, C3], a["X_attn"].T @ dqkv[:, C3], "bf16")
    compare("dbqkv", out["dbqkv"], dqkv.sum(axis=0), "bf16")
    compare("dbo", out["dbo"], a["dO"].sum(axis=0), "bf16")
    compare("dX_attn[R]", out["dX_attn"][R], dqkv[R] @ a["Wqkv"].T, "bf16")
    _write_report(f"{name}_r{rank}", rep)
    print(f"[full-size] {name} rank {rank}: done", flush=True)
