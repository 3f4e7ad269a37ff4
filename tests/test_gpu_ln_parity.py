"""GPU parity of the residual add + LayerNorm (tp_ln_residual_fwd / _bwd)
against the fp64 oracle on the same seeded inputs: every element of every
output, at the hidden sizes of the configured layers (ragged row counts, 0 to
8 partial block outputs, with and without bias and residual gradient), at the
530B-like shard's full size, and the empty batch."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import compare, f64

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")

EPS = 1e-5
OUTS = ("resid_out", "ln_out", "mean", "rstd", "d_resid", "dgamma", "dbeta", "dbias")
_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def tp_shape(w):
    return tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                           head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))


def run_gpu(w, inp, with_dr_in=True, with_dbias=True):
    s = tp_shape(w)
    T, h, dt = w.tokens, w.hidden, _DT[w.dtype]
    dev = lambda t: None if t is None else t.cuda().contiguous()  # noqa: E731
    nan = float("nan")
    o = {"resid_out": torch.full((T, h), nan, dtype=dt, device="cuda"),
         "ln_out": torch.full((T, h), nan, dtype=dt, device="cuda"),
         "mean": torch.full((T,), nan, dtype=torch.float32, device="cuda"),
         "rstd": torch.full((T,), nan, dtype=torch.float32, device="cuda"),
         "d_resid": torch.full((T, h), nan, dtype=dt, device="cuda"),
         "dgamma": torch.full((h,), nan, dtype=dt, device="cuda"),
         "dbeta": torch.full((h,), nan, dtype=dt, device="cuda"),
         "dbias": torch.full((h,), nan, dtype=dt, device="cuda") if with_dbias else None}
    parts = [dev(p) for p in inp["parts"]]
    gamma = dev(inp["gamma"])
    tp.tp_ln_residual_fwd(s, dev(inp["resid_in"]), parts, dev(inp["bias"]), gamma, dev(inp["beta"]), EPS,
                          o["resid_out"], o["ln_out"], o["mean"], o["rstd"])
    ws = torch.empty(max(tp.tp_ln_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    tp.tp_ln_residual_bwd(s, o["resid_out"], o["mean"], o["rstd"], gamma, dev(inp["d_ln_out"]),
                          dev(inp["d_resid_out"]) if with_dr_in else None, o["d_resid"], o["dgamma"], o["dbeta"],
                          o["dbias"], workspace=ws)
    torch.cuda.synchronize()
    return o


def run_oracle(inp, with_dr_in=True):
    a = {k: (None if v is None else (f64(v) if not isinstance(v, list) else [f64(p) for p in v]))
         for k, v in inp.items()}
    r, y, mu, rstd = oracle.ln_residual_fwd(a["resid_in"], a["parts"], a["bias"], a["gamma"], a["beta"], EPS)
    dr, dg, db, dbias = oracle.ln_residual_bwd(r, a["gamma"], EPS, a["d_ln_out"],
                                               a["d_resid_out"] if with_dr_in else None)
    return dict(resid_out=r, ln_out=y, mean=mu, rstd=rstd, d_resid=dr, dgamma=dg, dbeta=db, dbias=dbias)


# name, workload, rows (batch 1 x seq), partial outputs, bias std, residual gradient
CASES = [
    ("c1_fp32_h64_two_ranks", "tiny_fp32_tp2", 64, 2, 0.5, True),
    ("c2_h1536_ragged_rows", "gpt2_1p2b_tp1", 300, 1, 0.5, True),
    ("c3_h3072_no_parts_no_bias", "gpt_8p3b_tp8", 77, 0, 0.0, False),
    ("c4_h20480_37_rows", "mtnlg_530b_tp8", 37, 1, 0.02, True),
    ("c5_h14336_eight_parts", "bloom_176b_tp8", 96, 8, 0.02, False),
    ("c4_h20480_one_row", "mtnlg_530b_tp8", 1, 2, 0.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ln_residual_matches_oracle(case):
    name, wname, rows, n_parts, bias_std, with_dr_in = case
    w = synth.WORKLOADS[wname].with_(batch=1, seq=rows)
    print(f"\n  [ln case {name}] T={w.tokens} h={w.hidden} parts={n_parts} dtype={w.dtype}", flush=True)
    inp = synth.draw_ln(w, seed=3, n_parts=n_parts, bias_std=bias_std)
    got = run_gpu(w, inp, with_dr_in=with_dr_in)
    ref = run_oracle(inp, with_dr_in=with_dr_in)
    for k in OUTS:
        compare(k, got[k], ref[k], w.dtype)


def test_ln_residual_full_size_530b_shard():
    # the configuration the benchmark times: 2048 tokens x hidden 20480, bf16, one
    # block output (after g), replicated bias, residual gradient
    w = synth.WORKLOADS["mtnlg_530b_tp8"]
    print(f"\n  [ln full] T={w.tokens} h={w.hidden}", flush=True)
    inp = synth.draw_ln(w, seed=0, n_parts=1, bias_std=0.02)
    got = run_gpu(w, inp)
    ref = run_oracle(inp)
    for k in OUTS:
        compare(k, got[k], ref[k], w.dtype)


def test_ln_residual_empty_batch_and_no_dbias():
    w = synth.WORKLOADS["gpt2_1p2b_tp1"].with_(batch=0, seq=16)
    inp = synth.draw_ln(w, seed=1, n_parts=1)
    got = run_gpu(w, inp)
    for k in ("dgamma", "dbeta", "dbias"):
        assert torch.all(got[k] == 0), k
    # dbias NULL: the other outputs are unchanged
    w = synth.WORKLOADS["gpt2_1p2b_tp1"].with_(batch=1, seq=40)
    inp = synth.draw_ln(w, seed=2, n_parts=1, bias_std=0.5)
    a = run_gpu(w, inp, with_dbias=True)
    b = run_gpu(w, inp, with_dbias=False)
    for k in OUTS:
        if k != "dbias":
            assert torch.equal(a[k], b[k]), k


def test_ln_residual_deterministic():
    w = synth.WORKLOADS["bloom_176b_tp8"].with_(batch=1, seq=600)
    inp = synth.draw_ln(w, seed=4, n_parts=1, bias_std=0.02)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for k in OUTS:
        assert torch.equal(a[k], b[k]), k


# ---------------------------------------------------------------------------
# dropout on the block output before the residual add (identical on every rank)
# ---------------------------------------------------------------------------

def run_gpu_dropout(w, inp, drop):
    s = tp_shape(w)
    T, h, dt = w.tokens, w.hidden, _DT[w.dtype]
    dev = lambda t: None if t is None else t.cuda().contiguous()  # noqa: E731
    nan = float("nan")
    o = {k: torch.full((T, h), nan, dtype=dt, device="cuda") for k in ("resid_out", "ln_out", "d_resid", "d_block")}
    o.update({k: torch.full((T,), nan, dtype=torch.float32, device="cuda") for k in ("mean", "rstd")})
    o.update({k: torch.full((h,), nan, dtype=dt, device="cuda") for k in ("dgamma", "dbeta", "dbias")})
    mask = torch.zeros(max(tp.tp_ln_dropout_mask_bytes(s), 1), dtype=torch.uint8, device="cuda")
    gamma = dev(inp["gamma"])
    tp.tp_ln_residual_fwd_dropout(s, drop, dev(inp["resid_in"]), [dev(p) for p in inp["parts"]], dev(inp["bias"]),
                                  gamma, dev(inp["beta"]), EPS, o["resid_out"], o["ln_out"], o["mean"], o["rstd"],
                                  mask)
    ws = torch.empty(max(tp.tp_ln_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    tp.tp_ln_residual_bwd_dropout(s, drop, o["resid_out"], o["mean"], o["rstd"], gamma, dev(inp["d_ln_out"]),
                                  dev(inp["d_resid_out"]), mask, o["d_resid"], o["d_block"], o["dgamma"], o["dbeta"],
                                  o["dbias"], workspace=ws)
    torch.cuda.synchronize()
    o["mask"] = mask
    return o


DROP_CASES = [
    ("c1_fp32_h64_two_ranks_p03", "tiny_fp32_tp2", 64, 2, 0.5, 0.3),
    ("c4_h20480_37_rows_p01", "mtnlg_530b_tp8", 37, 1, 0.02, 0.1),
    ("c2_h1536_ragged_p05", "gpt2_1p2b_tp1", 300, 1, 0.5, 0.5),
    # the forward draws one Philox block per two neighbouring threads' chunks
    # and swaps halves: two chunks per thread (h 3072), eight of which the
    # last is past the row (h 14336), and an odd chunk count (h 4104: 513
    # chunks, the last one's neighbour past the row)
    ("c3_h3072_p02", "gpt_8p3b_tp8", 33, 1, 0.5, 0.2),
    ("c5_h14336_p01", "bloom_176b_tp8", 21, 2, 0.02, 0.1),
    ("h4104_odd_chunks_p03", "h4104", 19, 1, 0.5, 0.3),
]


@pytest.mark.parametrize("case", DROP_CASES, ids=[c[0] for c in DROP_CASES])
def test_ln_residual_dropout_matches_oracle(case):
    name, wname, rows, n_parts, bias_std, p = case
    if wname == "h4104":
        w = synth.WORKLOADS["gpt2_1p2b_tp1"].with_(batch=1, seq=rows, hidden=4104, n_heads=27, head_dim=152,
                                                   ffn=4 * 4104)
    else:
        w = synth.WORKLOADS[wname].with_(batch=1, seq=rows)
    print(f"\n  [ln dropout case {name}]", flush=True)
    inp = synth.draw_ln(w, seed=9, n_parts=n_parts, bias_std=bias_std)
    got = run_gpu_dropout(w, inp, tp.TpDropout(p, 99, 5))
    R = oracle.residual_multipliers(tokens=w.tokens, hidden=w.hidden, p=p, seed=99, offset=5)
    # keep bits, bit-exact
    bits = got["mask"].cpu().numpy()[:w.tokens * w.hidden // 8].reshape(w.tokens, w.hidden // 8)
    keep = np.unpackbits(bits[:, :, None], axis=2, bitorder="little").reshape(w.tokens, w.hidden).astype(bool)
    assert np.array_equal(keep, R > 0)
    a = {k: (None if v is None else (f64(v) if not isinstance(v, list) else [f64(q) for q in v]))
         for k, v in inp.items()}
    r, y, mu, rstd = oracle.ln_residual_fwd(a["resid_in"], a["parts"], a["bias"], a["gamma"], a["beta"], EPS,
                                            dropout=R)
    dr, dblk, dg, db, dbias = oracle.ln_residual_bwd_dropout(r, a["gamma"], EPS, a["d_ln_out"], a["d_resid_out"], R)
    for k, ref in (("resid_out", r), ("ln_out", y), ("mean", mu), ("rstd", rstd), ("d_resid", dr),
                   ("d_block", dblk), ("dgamma", dg), ("dbeta", db), ("dbias", dbias)):
        compare(k, got[k], ref, w.dtype)


def test_ln_residual_dropout_p0_equals_plain():
    w = synth.WORKLOADS["bloom_176b_tp8"].with_(batch=1, seq=50)
    inp = synth.draw_ln(w, seed=4, n_parts=2, bias_std=0.02)
    a = run_gpu_dropout(w, inp, tp.TpDropout(0.0, 1, 1))
    b = run_gpu(w, inp)
    for k in ("resid_out", "ln_out", "mean", "rstd", "d_resid", "dgamma", "dbeta"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["d_block"], b["d_resid"])
