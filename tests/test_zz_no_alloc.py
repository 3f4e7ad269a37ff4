"""The allocation-free residual + LayerNorm backward (tp_ln_residual_bwd_noalloc,
scratch held by the library) against the entry point that takes a caller
workspace (tp_ln_residual_bwd), through the C ABI: two calls in a row, the
second on a smaller input (the scratch then holds the first call's partials),
each output bit-identical to the workspace version's and within the bf16 /
fp32 bar of the fp64 oracle."""
import pytest
import torch

import oracle
import synth
from parity_util import compare, f64

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")

EPS = 1e-5
_DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def _shape(w):
    return tp.TpShape.make(batch=w.batch, seq=w.seq, hidden=w.hidden, ffn=w.ffn, n_heads=w.n_heads,
                           head_dim=w.head_dim, tp_rank=0, tp_size=w.tp_size, dtype=w.dtype, alibi=int(w.alibi))


def _both(w, seed):
    """Forward once, then the backward through both entry points on the same
    saved statistics; every output pre-filled with NaN."""
    s = _shape(w)
    inp = synth.draw_ln(w, seed=seed, n_parts=2, bias_std=0.5)
    T, h, dt = w.tokens, w.hidden, _DT[w.dtype]
    dev = lambda t: None if t is None else t.cuda().contiguous()  # noqa: E731
    nan = float("nan")
    r = torch.full((T, h), nan, dtype=dt, device="cuda")
    y = torch.full((T, h), nan, dtype=dt, device="cuda")
    mean = torch.full((T,), nan, dtype=torch.float32, device="cuda")
    rstd = torch.full((T,), nan, dtype=torch.float32, device="cuda")
    gamma = dev(inp["gamma"])
    tp.tp_ln_residual_fwd(s, dev(inp["resid_in"]), [dev(p) for p in inp["parts"]], dev(inp["bias"]), gamma,
                          dev(inp["beta"]), EPS, r, y, mean, rstd)
    dy, dr_in = dev(inp["d_ln_out"]), dev(inp["d_resid_out"])

    def outs():
        return {"d_resid": torch.full((T, h), nan, dtype=dt, device="cuda"),
                "dgamma": torch.full((h,), nan, dtype=dt, device="cuda"),
                "dbeta": torch.full((h,), nan, dtype=dt, device="cuda"),
                "dbias": torch.full((h,), nan, dtype=dt, device="cuda")}

    a, b = outs(), outs()
    ws = torch.empty(max(tp.tp_ln_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    tp.tp_ln_residual_bwd(s, r, mean, rstd, gamma, dy, dr_in, a["d_resid"], a["dgamma"], a["dbeta"], a["dbias"],
                          workspace=ws)
    tp.tp_ln_residual_bwd_noalloc(s, r, mean, rstd, gamma, dy, dr_in, b["d_resid"], b["dgamma"], b["dbeta"],
                                  b["dbias"])
    torch.cuda.synchronize()
    return inp, r, a, b


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point_twice(order):
    assert tp.tp_ln_residual_bwd_noalloc_max_scratch_bytes() == 48 << 20
    big = synth.WORKLOADS["mtnlg_530b_tp8"]  # T 2048, hidden 20480: 40 MiB of run partials
    small = synth.WORKLOADS["gpt2_1p2b_tp1"].with_(batch=1, seq=77)  # T 77, hidden 1536
    for w, seed in ((big, 11), (small, 12)):
        s = _shape(w)
        need = tp.tp_ln_workspace_bytes(s)
        print(f"\n  [noalloc] T={w.tokens} h={w.hidden} {w.dtype}: scratch needed {need} bytes", flush=True)
        assert 0 < need <= tp.tp_ln_residual_bwd_noalloc_max_scratch_bytes()
        inp, r, a, b = _both(w, seed)
        for k in a:
            assert torch.equal(a[k], b[k]), f"{k}: allocation-free entry point differs from the workspace one"
        # and within the bar of the fp64 oracle (on the stored resid_out)
        dr, dg, dbt, dbi = oracle.ln_residual_bwd(f64(r), f64(inp["gamma"]), EPS, f64(inp["d_ln_out"]),
                                                  f64(inp["d_resid_out"]))
        for k, ref in (("d_resid", dr), ("dgamma", dg), ("dbeta", dbt), ("dbias", dbi)):
            compare(k, b[k], ref, w.dtype)
