"""GPU parity of the 256x320-tile products against the fp64 oracle. The library
takes that tile for products with a k-inner B (the input gradients) when N is
a multiple of 320 and the tiles fill the CUs at least once, which the small
parity shapes never reach; these MLP shapes do, with a ragged token count (a
partial last row of tiles) and a stream-K tail:
  * h = 3200, f = 9600: the GEMM2 input gradient (+ GeLU' epilogue) runs 320
    wide (N = f);
  * h = 9600, f = 3200: the GEMM1 input gradient runs 320 wide (N = h).
The GEMM1 weight gradient (X^T times a transposed dPre copy) runs 320 wide in
both shapes, with K = 2100 tokens (a partial last k-step).
  * h = f = 8960: GEMM2 and its weight gradient run 256-wide tiles with a
    stream-K tail (9 x 35 and 35 x 35 tiles; K = 2100 for the weight
    gradient: a partial last k-step).
The output projection takes a 256x320 tile on 16x16x32 MFMAs when its tiles
run in whole data-parallel rounds; at h = 8960 over 8 ranks (7 heads of 160
per rank, K = 1120) and T = 2100 that is 9 x 28 = 252 tiles, one round, the
last row of tiles 52 rows.
With fewer 320-wide tiles than CUs the input gradients take that tile when
its k-split covers every CU exactly; at T = 1900 (8 row tiles, the last one
108 rows) on a 256-CU device:
  * h = 2720, f = 2560: the GEMM2 input gradient (+ GeLU' epilogue), 8 x 8 =
    64 tiles in 4 k-parts, K = 2720 (the last part ends in a partial k-step);
  * h = 2560, f = 2720: the GEMM1 input gradient, the same split over K = 2720.
Narrow layers take 256x192 tiles for the input gradients where their plan is
shorter; at h = 384, f = 3000, T = 2100 (9 row tiles, the last one 52 rows):
  * the GEMM2 input gradient (N = f = 3000, K = 384) runs 9 x 16 data-parallel
    tiles, the last column of tiles 120 wide;
  * the GEMM1 input gradient (N = h = 384, K = 3000: a partial last k-step)
    runs 18 tiles dealt out stream-K over the CUs, with the fix-up.
The oracle recomputes column sub-shards and sampled token rows exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import compare, f64, shape_of

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("tensor_transformer_layer_tp_amd")

MLP_IN = ("X_mlp", "A", "b1", "B", "dZ")
ATTN_IN = ("X_attn", "Wqkv", "bqkv", "Wo", "dO")
TOKENS = 2100  # 9 row tiles of 256, the last one 52 rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tp.load_library()
    yield
    torch.cuda.synchronize()


def workload(h, ffn, tokens=TOKENS):
    d = 160 if h % 160 == 0 else 128
    return synth.Workload(f"wide_h{h}_f{ffn}", batch=1, seq=tokens, hidden=h, n_heads=h // d, head_dim=d,
                          ffn=ffn, tp_size=1, dtype="bf16", bias_std=0.5)


def samples(n, k, rng):
    return np.unique(np.concatenate([[0, 1, n // 2, n - 1], rng.choice(n, k, replace=False)]))


@pytest.mark.parametrize("h,ffn,tokens,exact_split", [
    (3200, 9600, TOKENS, False), (9600, 3200, TOKENS, False), (8960, 8960, TOKENS, False),
    (2720, 2560, 1900, True), (2560, 2720, 1900, True), (384, 3000, TOKENS, False)],
    ids=["fc2_dgrad_wide", "fc1_dgrad_wide", "fwd_wide", "fc2_dgrad_exact_ksplit", "fc1_dgrad_exact_ksplit",
         "dgrads_192_wide"])
def test_mlp_wide_tiles_ragged_tokens(h, ffn, tokens, exact_split):
    if exact_split and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the exact k-split of 64 tiles in 4 parts is planned for a 256-CU device only")
    w = workload(h, ffn, tokens)
    s = shape_of(w, 0)
    print(f"\n  [wide MLP] T={tokens} h={h} f={ffn}: {tp.tp_step_kernel(s, 'fc2_dgrad')}, "
          f"{tp.tp_step_kernel(s, 'fc1_dgrad')}", flush=True)
    if h == 384 and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert tp.tp_step_kernel(s, "fc2_dgrad").endswith("_n192")
        assert tp.tp_step_kernel(s, "fc1_dgrad").endswith("_n192")
    inp = synth.draw_shard(w, seed=21, skip=ATTN_IN)
    T, bf, nan = w.tokens, torch.bfloat16, float("nan")
    d = {k: inp[k].cuda().contiguous() for k in MLP_IN}
    o = {"pre": torch.full((T, ffn), nan, dtype=bf, device="cuda"),
         "y": torch.full((T, ffn), nan, dtype=bf, device="cuda"),
         "Z": torch.full((T, h), nan, dtype=bf, device="cuda"),
         "dX": torch.full((T, h), nan, dtype=bf, device="cuda"),
         "dA": torch.full((h, ffn), nan, dtype=bf, device="cuda"),
         "db1": torch.full((ffn,), nan, dtype=bf, device="cuda"),
         "dB": torch.full((ffn, h), nan, dtype=bf, device="cuda"),
         "db2": torch.full((h,), nan, dtype=bf, device="cuda")}
    ws = torch.empty(max(tp.tp_mlp_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    tp.tp_mlp_fwd(s, d["X_mlp"], d["A"], d["b1"], d["B"], o["pre"], o["y"], o["Z"], workspace=ws)
    tp.tp_mlp_bwd(s, d["X_mlp"], d["A"], d["B"], o["pre"], o["y"], d["dZ"], o["dX"], o["dA"], o["db1"], o["dB"],
                  o["db2"], workspace=ws)
    torch.cuda.synchronize()
    a = {k: f64(inp[k]) for k in MLP_IN}
    rng = np.random.default_rng(3)
    # a column sub-shard C of the FFN columns is itself a valid shard
    C = samples(ffn, 60, rng)
    pre_C, y_C, _ = oracle.mlp_fwd(a["X_mlp"], a["A"][:, C], a["b1"][C], a["B"][C, :])
    compare("pre[:,C]", o["pre"][:, C], pre_C, "bf16")
    compare("y[:,C]", o["y"][:, C], y_C, "bf16")
    _, dA_C, db1_C, dB_C, db2 = oracle.mlp_bwd(a["X_mlp"], a["A"][:, C], a["B"][C, :], pre_C, y_C, a["dZ"])
    compare("dA[:,C]", o["dA"][:, C], dA_C, "bf16")
    compare("db1[C]", o["db1"][C], db1_C, "bf16")
    compare("dB[C,:]", o["dB"][C, :], dB_C, "bf16")
    compare("db2", o["db2"], db2, "bf16")
    # token rows R, including the ragged last row tile
    R = np.unique(np.concatenate([samples(T, 12, rng), np.arange(T - 8, T)]))
    pre_R, y_R, Z_R = oracle.mlp_fwd(a["X_mlp"][R], a["A"], a["b1"], a["B"])
    compare("pre[R]", o["pre"][R], pre_R, "bf16")
    compare("Z[R]", o["Z"][R], Z_R, "bf16")
    dX_R = oracle.mlp_bwd(a["X_mlp"][R], a["A"], a["B"], pre_R, y_R, a["dZ"][R])[0]
    compare("dX_mlp[R]", o["dX"][R], dX_R, "bf16")


def test_out_projection_wide_tile_ragged_tokens():
    w = synth.Workload("wide_attn_h8960", batch=1, seq=TOKENS, hidden=8960, n_heads=56, head_dim=160,
                       ffn=4 * 8960, tp_size=8, dtype="bf16", bias_std=0.5)
    rank = 3
    s = shape_of(w, rank)
    print(f"\n  [wide out-projection] T={TOKENS} h={w.hidden} rank {rank}: {tp.tp_step_kernel(s, 'out_proj')}",
          flush=True)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert tp.tp_step_kernel(s, "out_proj") == "gemm_out_proj_n320"
    inp = synth.draw_shard(w, seed=23, skip=MLP_IN)
    T, h, hl, nl, bf, nan = w.tokens, w.hidden, w.h_local, w.heads_local, torch.bfloat16, float("nan")
    d = {k: inp[k].cuda().contiguous() for k in ("X_attn", "Wqkv", "bqkv", "Wo")}
    qkv = torch.full((max(tp.tp_attn_qkv_bytes(s), 1),), 255, dtype=torch.uint8, device="cuda")
    ctx = torch.full((T, hl), nan, dtype=bf, device="cuda")
    lse = torch.full((w.batch, nl, w.seq), nan, dtype=torch.float32, device="cuda")
    O = torch.full((T, h), nan, dtype=bf, device="cuda")
    ws = torch.empty(max(tp.tp_attn_workspace_bytes(s), 1), dtype=torch.uint8, device="cuda")
    tp.tp_attn_fwd(s, d["X_attn"], d["Wqkv"], d["bqkv"], d["Wo"], qkv, ctx, lse, O, ws)
    torch.cuda.synchronize()
    a = {k: f64(inp[k]) for k in ("X_attn", "Wqkv", "bqkv", "Wo")}
    ctx_ref, _ = oracle.attn_core_fwd(a["X_attn"] @ a["Wqkv"] + a["bqkv"], batch=w.batch, seq=w.seq, n_local=nl,
                                      head_dim=w.head_dim, head0=rank * nl, n_heads=w.n_heads, alibi=w.alibi)
    compare("ctx", ctx, ctx_ref, "bf16")
    rng = np.random.default_rng(5)
    R = np.unique(np.concatenate([samples(T, 12, rng), np.arange(T - 8, T)]))
    compare("O[R]", O[R], ctx_ref[R] @ a["Wo"], "bf16")
