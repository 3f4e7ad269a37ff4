"""GPU parity of attention-probability dropout (tp_attn_fwd_dropout /
tp_attn_bwd_dropout) against the fp64 oracle with the same counter-based
multipliers: every output of the attention block forward and backward, and
the keep bits the forward stores (bit-exact against the oracle's generator),
for head widths 64 / 96 / 128 / 160, ALiBi on and off, ranks 0..7, ragged
sequence lengths and p in {0.1, 0.5}; p = 0 against the entry points without
dropout (bit-exact); and at the 530B-like shard's full size on sampled heads."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import compare, compare_saved_qkv, f64, shape_of

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")

ATTN_IN = ("X_attn", "Wqkv", "bqkv", "Wo", "dO")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def run_gpu(w, inp, rank, drop):
    s = shape_of(w, rank)
    T, h, hl, nl = w.tokens, w.hidden, w.h_local, w.heads_local
    dev = {k: inp[k].cuda().contiguous() for k in ATTN_IN}
    bf, nan = torch.bfloat16, float("nan")
    o = {"qkv": torch.full((max(tp.tp_attn_qkv_bytes(s), 1),), 255, dtype=torch.uint8, device="cuda"),
         "ctx": torch.full((T, hl), nan, dtype=bf, device="cuda"),
         "lse": torch.full((w.batch, nl, w.seq), nan, dtype=torch.float32, device="cuda"),
         "O": torch.full((T, h), nan, dtype=bf, device="cuda"),
         "dX_attn": torch.full((T, h), nan, dtype=bf, device="cuda"),
         "dWqkv": torch.full((h, 3 * hl), nan, dtype=bf, device="cuda"),
         "dbqkv": torch.full((3 * hl,), nan, dtype=bf, device="cuda"),
         "dWo": torch.full((hl, h), nan, dtype=bf, device="cuda"),
         "dbo": torch.full((h,), nan, dtype=bf, device="cuda")}
    ws = torch.empty(max(tp.tp_attn_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    if drop is None:
        tp.tp_attn_fwd(s, dev["X_attn"], dev["Wqkv"], dev["bqkv"], dev["Wo"], o["qkv"], o["ctx"], o["lse"], o["O"], ws)
        tp.tp_attn_bwd(s, dev["X_attn"], dev["Wqkv"], dev["Wo"], o["qkv"], o["ctx"], o["lse"], dev["dO"],
                       o["dX_attn"], o["dWqkv"], o["dbqkv"], o["dWo"], o["dbo"], ws)
    else:
        mask = torch.zeros(tp.tp_attn_dropout_mask_bytes(s) // 2, dtype=torch.int16, device="cuda")
        tp.tp_attn_fwd_dropout(s, drop, dev["X_attn"], dev["Wqkv"], dev["bqkv"], dev["Wo"], o["qkv"], o["ctx"],
                               o["lse"], mask, o["O"], ws)
        tp.tp_attn_bwd_dropout(s, drop, dev["X_attn"], dev["Wqkv"], dev["Wo"], o["qkv"], o["ctx"], o["lse"], mask,
                               dev["dO"], o["dX_attn"], o["dWqkv"], o["dbqkv"], o["dWo"], o["dbo"], ws)
        o["mask"] = mask
    torch.cuda.synchronize()
    return o


def gpu_keep(w, mask, heads=None):
    """Decode the stored keep bits to keep[b, l, i, j] for the causal pairs j <= i."""
    s, nl = w.seq, w.heads_local
    nkb, ms = (s + 31) // 32, (s + 7) // 8 * 8
    M = mask.cpu().numpy().view(np.uint16).reshape(w.batch, nl, nkb, 2, ms)
    j = np.arange(s)
    kb, o = j // 32, j % 32
    g, q = (o >> 2) & 1, 4 * (o >> 3) + (o & 3)
    i = np.arange(s)
    heads = range(nl) if heads is None else heads
    out = {}
    for b in range(w.batch):
        for l in heads:
            words = M[b, l][kb[None, :], g[None, :], i[:, None]]  # [i, j]
            out[(b, l)] = ((words >> q[None, :]) & 1).astype(bool)
    return out


def check_keep(w, mask, D, heads=None):
    """D: multipliers indexable by (b, l) (an array [b, l, i, j] or a dict)."""
    causal = np.tril(np.ones((w.seq, w.seq), dtype=bool))
    for (b, l), keep in gpu_keep(w, mask, heads).items():
        want = D[b, l] > 0
        bad = (keep != want) & causal
        assert not bad.any(), f"keep bits differ at head {l}, batch {b}: {int(bad.sum())} elements, first {np.argwhere(bad)[0]}"


CASES = [
    # name, workload, rank, p
    ("d64_tp2_r1_alibi_ragged_p01", synth.Workload("d64", batch=2, seq=130, hidden=256, n_heads=4, head_dim=64,
                                                   ffn=1024, tp_size=2, dtype="bf16", alibi=True, bias_std=0.5), 1, 0.1),
    ("d160_tp1_seq300_p05", synth.Workload("d160", batch=1, seq=300, hidden=320, n_heads=2, head_dim=160, ffn=1280,
                                           tp_size=1, dtype="bf16"), 0, 0.5),
    ("d128_tp8_r7_alibi_seq257_p01", synth.Workload("d128", batch=1, seq=257, hidden=2048, n_heads=16,
                                                    head_dim=128, ffn=8192, tp_size=8, dtype="bf16", alibi=True), 7, 0.1),
    ("d96_tp1_seq33_p03", synth.Workload("d96", batch=3, seq=33, hidden=192, n_heads=2, head_dim=96, ffn=768,
                                         tp_size=1, dtype="bf16", bias_std=0.5), 0, 0.3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dropout_attention_matches_oracle(case):
    name, w, rank, p = case
    print(f"\n  [dropout case {name}]", flush=True)
    inp = synth.draw_shard(w, seed=11)
    drop = tp.TpDropout(p, 0x1234ABCD, 17 + rank)
    got = run_gpu(w, inp, rank, drop)
    nl = w.heads_local
    D = oracle.attention_multipliers(batch=w.batch, seq=w.seq, n_local=nl, head0=rank * nl, p=p,
                                     seed=0x1234ABCD, offset=17 + rank)
    check_keep(w, got["mask"], D)
    a = {k: f64(inp[k]) for k in ATTN_IN}
    kw = dict(batch=w.batch, seq=w.seq, n_heads=w.n_heads, tp_size=w.tp_size, tp_rank=rank, alibi=w.alibi,
              dropout=D)
    qkv, ctx, lse, O = oracle.attn_fwd(a["X_attn"], a["Wqkv"], a["bqkv"], a["Wo"], **kw)
    dX, dWqkv, dbqkv, dWo, dbo = oracle.attn_bwd(a["X_attn"], a["Wqkv"], a["bqkv"], a["Wo"], a["dO"], **kw)
    compare_saved_qkv(got["qkv"], qkv, w.tokens, w.h_local, w.head_dim, "bf16")
    for k, ref in (("ctx", ctx), ("lse", lse), ("O", O), ("dX_attn", dX), ("dWqkv", dWqkv),
                   ("dbqkv", dbqkv), ("dWo", dWo), ("dbo", dbo)):
        compare(k, got[k], ref, "bf16")


@pytest.mark.parametrize("case", [0, 1], ids=["d64_four_wave_backward", "d160_split_role_backward"])
def test_dropout_p0_equals_no_dropout(case):
    # D <= 96 runs the 4-wave backward, wider heads the 8-wave split-role one;
    # with p = 0 each dropout variant repeats its plain kernel bit for bit
    _, w, rank, _ = CASES[case]
    inp = synth.draw_shard(w, seed=12)
    a = run_gpu(w, inp, rank, tp.TpDropout(0.0, 5, 6))
    b = run_gpu(w, inp, rank, None)
    for k in b:
        assert torch.equal(a[k], b[k]), k
    causal = np.tril(np.ones((w.seq, w.seq), dtype=bool))
    for keep in gpu_keep(w, a["mask"]).values():  # p = 0 keeps every key
        assert keep[causal].all()


def test_dropout_full_size_530b_sampled_heads():
    w = synth.WORKLOADS["mtnlg_530b_tp8"]
    inp = synth.draw_shard(w, seed=0, skip=("X_mlp", "A", "b1", "B", "dZ"))
    print("\n  [dropout full] mtnlg_530b_tp8 p=0.1", flush=True)
    got = run_gpu(w, inp, 0, tp.TpDropout(0.1, 2024, 1))
    heads = (0, w.heads_local - 1)
    d, hl = w.head_dim, w.h_local
    D = {(0, l): oracle.attention_multipliers(batch=1, seq=w.seq, n_local=1, head0=l, p=0.1, seed=2024,
                                              offset=1)[0, 0] for l in heads}
    check_keep(w, got["mask"], D, heads)
    X, W, bq = f64(inp["X_attn"]), f64(inp["Wqkv"]), f64(inp["bqkv"])
    for l in heads:
        cols = np.concatenate([np.arange(k * hl + l * d, k * hl + (l + 1) * d) for k in range(3)])
        qkv_l = X @ W[:, cols] + bq[cols]
        ctx_l, lse_l = oracle.attn_core_fwd(qkv_l, batch=1, seq=w.seq, n_local=1, head_dim=d, head0=l,
                                            n_heads=w.n_heads, dropout=D[(0, l)][None, None])
        compare(f"ctx[head {l}]", got["ctx"][:, l * d:(l + 1) * d], ctx_l, "bf16")
        compare(f"lse[head {l}]", got["lse"][:, l], lse_l[:, 0], "bf16")
