"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
function the header declares, sizes workspaces, and rejects invalid arguments
before touching the device (every call here returns before any HIP call)."""
import ctypes
import subprocess

import os

import pytest

import tensor_transformer_layer_tp_amd as tp

FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced by these calls


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


# These calls pass fake device addresses and rely on validation refusing them
# before any launch; where a GPU is visible a regression in that validation
# would dereference them, so the module runs only where none is.
pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only checks (fake device addresses); no GPU may be visible")


def shape(**kw):
    base = dict(batch=2, seq=32, hidden=64, ffn=256, n_heads=4, head_dim=16, tp_rank=0, tp_size=2, dtype=tp.TP_FP32)
    base.update(kw)
    return tp.TpShape.make(**base)


def test_library_loads_and_exports_every_declared_symbol():
    lib = tp.load_library()
    names = tp.exported_symbols()
    assert set(names) == {"tp_mlp_workspace_bytes", "tp_attn_workspace_bytes", "tp_mlp_fwd", "tp_mlp_bwd",
                          "tp_attn_fwd", "tp_attn_bwd", "tp_sum_partials", "tp_last_error", "tp_profile_enable",
                          "tp_profile_collect", "tp_ln_workspace_bytes", "tp_ln_residual_fwd", "tp_ln_residual_bwd",
                          "tp_vocab_workspace_bytes", "tp_vocab_ce_fwd", "tp_vocab_ce_combine", "tp_vocab_ce_bwd",
                          "tp_attn_dropout_mask_bytes", "tp_attn_fwd_dropout", "tp_attn_bwd_dropout",
                          "tp_ln_dropout_mask_bytes", "tp_ln_residual_fwd_dropout", "tp_ln_residual_bwd_dropout",
                          "tp_ln_residual_bwd_noalloc", "tp_ln_residual_bwd_noalloc_max_scratch_bytes", "tp_step_kernel",
                          "tp_attn_qkv_bytes"}
    for n in names:
        assert isinstance(getattr(lib, n), ctypes._CFuncPtr), n
    out = subprocess.run(["nm", "-D", "--defined-only", tp.library_path()], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_workspace_sizes():
    assert tp.tp_mlp_workspace_bytes(shape()) > 0
    assert tp.tp_attn_workspace_bytes(shape()) > 0
    big = shape(batch=1, seq=2048, hidden=20480, ffn=81920, n_heads=128, head_dim=160, tp_size=8, dtype=tp.TP_BF16)
    # dPre [T, f_l] bf16 alone is 2048*10240*2 bytes
    assert tp.tp_mlp_workspace_bytes(big) >= 2048 * 10240 * 2
    # dctx + dqkv + delta
    assert tp.tp_attn_workspace_bytes(big) >= 2048 * 2560 * 2 * 4 + 2048 * 16 * 4
    assert tp.tp_mlp_workspace_bytes(shape(tp_rank=2)) == 0  # invalid shape -> 0


def test_saved_projection_bytes():
    # matrix-core path (bf16, head_dim 64/96/128/160): five 16-bit planes [T, h_l];
    # otherwise fp32 [T, 3 h_l]
    big = shape(batch=1, seq=2048, hidden=20480, ffn=81920, n_heads=128, head_dim=160, tp_size=8, dtype=tp.TP_BF16)
    assert tp.tp_attn_qkv_bytes(big) == 5 * 2 * 2048 * 2560
    assert tp.tp_attn_qkv_bytes(shape()) == 12 * 64 * 32  # fp32 tiny shard: T = 64, h_l = 32
    d16 = shape(batch=2, seq=40, hidden=128, ffn=512, n_heads=8, head_dim=16, tp_size=2, dtype=tp.TP_BF16)
    assert tp.tp_attn_qkv_bytes(d16) == 12 * 80 * 64  # bf16 with head_dim 16: vector-ALU path, fp32
    assert tp.tp_attn_qkv_bytes(shape(tp_rank=2)) == 0


def _mlp_fwd(s, ws=(FAKE, 1 << 40), **override):
    args = dict(X=FAKE, A_i=FAKE, b1_i=FAKE, B_i=FAKE, pre_i=FAKE, y_i=FAKE, Z_i=FAKE)
    args.update(override)
    tp.tp_mlp_fwd(s, workspace=ws, stream=0, **args)


@pytest.mark.parametrize("kw,status", [
    (dict(tp_rank=2), "TP_ERR_RANK"),
    (dict(tp_rank=-1), "TP_ERR_RANK"),
    (dict(tp_size=0, tp_rank=0), "TP_ERR_RANK"),
    (dict(n_heads=4, tp_size=3), "TP_ERR_DIVISIBILITY"),
    (dict(ffn=255), "TP_ERR_DIVISIBILITY"),
    (dict(head_dim=8), "TP_ERR_DIVISIBILITY"),
    (dict(hidden=60, n_heads=6, head_dim=10, ffn=240), "TP_ERR_HEADDIM"),
    (dict(dtype=7), "TP_ERR_DTYPE"),
    (dict(causal=0), "TP_ERR_SHAPE"),
    (dict(batch=-1), "TP_ERR_SHAPE"),
    (dict(hidden=72, n_heads=4, head_dim=18, ffn=256, dtype=tp.TP_BF16), "TP_ERR_HEADDIM"),
    (dict(hidden=96, n_heads=4, head_dim=24, ffn=264, tp_size=2, dtype=tp.TP_BF16), "TP_ERR_ALIGN"),
])
def test_shape_validation(kw, status):
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(shape(**kw))
    assert ei.value.name == status, str(ei.value)
    assert tp.tp_last_error() != ""


def test_pointer_validation():
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(shape(), X=None)
    assert ei.value.name == "TP_ERR_NULL"
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(shape(), A_i=FAKE + 2)
    assert ei.value.name == "TP_ERR_ALIGN"
    s = shape(dtype=tp.TP_BF16, hidden=512, ffn=2048, n_heads=4, head_dim=128)
    need = tp.tp_mlp_workspace_bytes(s)
    assert need > 0
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(s, ws=(FAKE, 16))
    assert ei.value.name == "TP_ERR_WORKSPACE"
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(s, ws=(None, 0))
    assert ei.value.name == "TP_ERR_WORKSPACE"
    with pytest.raises(tp.TPError) as ei:
        _mlp_fwd(s, ws=(FAKE + 16, need))
    assert ei.value.name == "TP_ERR_ALIGN"


def test_every_entry_point_validates():
    s = shape(tp_rank=5)
    with pytest.raises(tp.TPError):
        tp.tp_mlp_bwd(s, *([FAKE] * 10), workspace=(FAKE, 1 << 40), stream=0)
    with pytest.raises(tp.TPError):
        tp.tp_attn_fwd(s, *([FAKE] * 8), workspace=(FAKE, 1 << 40), stream=0)
    with pytest.raises(tp.TPError):
        tp.tp_attn_bwd(s, *([FAKE] * 11), workspace=(FAKE, 1 << 40), stream=0)
    with pytest.raises(tp.TPError):
        tp.tp_sum_partials(s, [FAKE, FAKE], None, FAKE, stream=0)
    with pytest.raises(tp.TPError) as ei:
        tp.tp_sum_partials(shape(), [], None, FAKE, stream=0)
    assert ei.value.name == "TP_ERR_SHAPE"
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_bwd(shape(), *([FAKE] * 7), None, FAKE, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_NULL"


def test_profile_mask_without_gpu():
    # enabling / disabling records nothing by itself; collecting an empty step is a no-op
    tp.tp_profile_enable(1 << tp.STEPS["fc1"])
    tp.tp_profile_enable(0)
    assert tp.tp_profile_collect(tp.STEPS["fc1"]) == (0, 0.0)
    # the binding's step ids are exactly the header's TP_STEP_* values
    import re
    with open(os.path.join(os.path.dirname(__file__), "..", "include", "tp_layer.h")) as fh:
        ids = {int(v) for v in re.findall(r"TP_STEP_\w+ = (\d+)", fh.read())}
    assert set(tp.STEPS.values()) == ids == set(range(1, 25))


def test_empty_batch_needs_no_token_pointers():
    # batch 0: token-shaped pointers may be NULL; the forward enqueues nothing
    s = shape(batch=0)
    tp.tp_mlp_fwd(s, None, FAKE, FAKE, FAKE, None, None, None, workspace=(FAKE, 1 << 40), stream=0)
    tp.tp_attn_fwd(s, None, FAKE, FAKE, FAKE, None, None, None, None, workspace=(FAKE, 1 << 40), stream=0)


# ---------------------------------------------------------------------------
# residual add + LayerNorm
# ---------------------------------------------------------------------------

def _ln_fwd(s, parts=(FAKE,), eps=1e-5, **override):
    args = dict(resid_in=FAKE, bias_or_null=None, gamma=FAKE, beta=FAKE, resid_out=FAKE, ln_out=FAKE, mean=FAKE,
                rstd=FAKE)
    args.update(override)
    tp.tp_ln_residual_fwd(s, args["resid_in"], list(parts), args["bias_or_null"], args["gamma"], args["beta"], eps,
                          args["resid_out"], args["ln_out"], args["mean"], args["rstd"], stream=0)


def _ln_bwd(s, ws=(FAKE, 1 << 40), **override):
    args = dict(resid_out=FAKE, mean=FAKE, rstd=FAKE, gamma=FAKE, d_ln_out=FAKE, d_resid_out_or_null=None,
                d_resid=FAKE, dgamma=FAKE, dbeta=FAKE, dbias_or_null=None)
    args.update(override)
    tp.tp_ln_residual_bwd(s, workspace=ws, stream=0, **args)


def test_ln_workspace_bytes():
    # fp32 partial rows of dgamma and dbeta per run of rows (at most 256 runs), then
    # the column-sum scratch of dbias
    big = shape(batch=1, seq=2048, hidden=20480, ffn=81920, n_heads=128, head_dim=160, tp_size=8, dtype=tp.TP_BF16)
    assert 256 * 2 * 20480 * 4 < tp.tp_ln_workspace_bytes(big) <= 256 * 3 * 20480 * 4
    assert 64 * 2 * 64 * 4 < tp.tp_ln_workspace_bytes(shape()) <= 64 * 3 * 64 * 4  # 64 rows -> 64 runs
    assert tp.tp_ln_workspace_bytes(shape(batch=0)) == 0
    wide = shape(hidden=32768, n_heads=256, head_dim=128, ffn=256)
    assert tp.tp_ln_workspace_bytes(wide) == 0  # hidden above the supported width


@pytest.mark.parametrize("kw,override,status", [
    (dict(hidden=32768, n_heads=256, head_dim=128), {}, "TP_ERR_SHAPE"),
    (dict(hidden=60, n_heads=6, head_dim=10, ffn=240), {}, "TP_ERR_HEADDIM"),
    (dict(hidden=72, n_heads=4, head_dim=18, ffn=256), {}, "TP_ERR_HEADDIM"),
    (dict(hidden=40, n_heads=5, head_dim=8, ffn=240, tp_size=2), {}, "TP_ERR_DIVISIBILITY"),
    ({}, dict(eps=0.0), "TP_ERR_SHAPE"),
    ({}, dict(eps=float("inf")), "TP_ERR_SHAPE"),
    ({}, dict(eps=float("nan")), "TP_ERR_SHAPE"),
    ({}, dict(gamma=None), "TP_ERR_NULL"),
    ({}, dict(beta=FAKE + 8), "TP_ERR_ALIGN"),
    ({}, dict(parts=[FAKE] * 65), "TP_ERR_SHAPE"),
    ({}, dict(parts=[FAKE, None]), "TP_ERR_NULL"),
    (dict(tp_rank=3), {}, "TP_ERR_RANK"),
])
def test_ln_fwd_validation(kw, override, status):
    with pytest.raises(tp.TPError) as ei:
        _ln_fwd(shape(**kw), **override)
    assert ei.value.name == status, str(ei.value)


def test_ln_hidden_multiple_of_8():
    # hidden = n_heads * head_dim with 8 | head_dim, so a hidden of 100 is already refused by the shape checks
    s = shape(hidden=100, n_heads=4, head_dim=25, ffn=256)
    with pytest.raises(tp.TPError) as ei:
        _ln_fwd(s)
    assert ei.value.name in ("TP_ERR_ALIGN", "TP_ERR_HEADDIM"), str(ei.value)


def test_ln_bwd_validation():
    with pytest.raises(tp.TPError) as ei:
        _ln_bwd(shape(), dgamma=None)
    assert ei.value.name == "TP_ERR_NULL"
    with pytest.raises(tp.TPError) as ei:
        _ln_bwd(shape(), ws=(FAKE, 16))
    assert ei.value.name == "TP_ERR_WORKSPACE"
    with pytest.raises(tp.TPError) as ei:
        _ln_bwd(shape(), d_resid_out_or_null=FAKE + 4)
    assert ei.value.name == "TP_ERR_ALIGN"


def test_ln_empty_batch_needs_no_token_pointers():
    _ln_fwd(shape(batch=0), parts=(None,), resid_in=None, resid_out=None, ln_out=None, mean=None, rstd=None)


# ---------------------------------------------------------------------------
# vocabulary-parallel logits + cross-entropy
# ---------------------------------------------------------------------------

def test_vocab_workspace_bytes():
    c3 = shape(batch=16, seq=1024, hidden=3072, ffn=12288, n_heads=24, head_dim=128, tp_size=8, dtype=tp.TP_BF16)
    # dlogits [T, V/p] bf16 at least
    assert tp.tp_vocab_workspace_bytes(c3, 51200) >= 16384 * 6400 * 2
    assert tp.tp_vocab_workspace_bytes(c3, 51201) == 0  # not divisible by tp_size
    assert tp.tp_vocab_workspace_bytes(c3, 8 * 12) == 0  # slice of 12: not a multiple of 8
    assert tp.tp_vocab_workspace_bytes(c3, 8 * 32776) == 0  # slice above 32768


@pytest.mark.parametrize("vocab,kw,status", [
    (513, {}, "TP_ERR_DIVISIBILITY"),
    (2 * 12, {}, "TP_ERR_ALIGN"),
    (0, {}, "TP_ERR_SHAPE"),
    (2 * 32776, {}, "TP_ERR_SHAPE"),
    (512, dict(tp_rank=2), "TP_ERR_RANK"),
])
def test_vocab_validation(vocab, kw, status):
    s = shape(**kw)
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_fwd(s, vocab, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == status, str(ei.value)
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_bwd(s, vocab, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=(FAKE, 1 << 40),
                           stream=0)
    assert ei.value.name == status, str(ei.value)


def test_vocab_pointer_validation():
    s = shape()
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_fwd(s, 512, FAKE, FAKE, None, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_NULL"
    sb = shape(dtype=tp.TP_BF16, hidden=512, ffn=2048, n_heads=4, head_dim=128)  # its logits GEMM needs a workspace
    assert tp.tp_vocab_workspace_bytes(sb, 512) > 16
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_fwd(sb, 512, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=(FAKE, 16), stream=0)
    assert ei.value.name == "TP_ERR_WORKSPACE"
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_bwd(s, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, workspace=(FAKE, 1 << 40),
                           stream=0)
    assert ei.value.name == "TP_ERR_ALIGN"
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_combine(s, [], FAKE, FAKE, stream=0)
    assert ei.value.name == "TP_ERR_SHAPE"
    with pytest.raises(tp.TPError) as ei:
        tp.tp_vocab_ce_combine(s, [FAKE, None], FAKE, FAKE, stream=0)
    assert ei.value.name == "TP_ERR_NULL"


def test_vocab_empty_batch_forward_needs_no_token_pointers():
    s = shape(batch=0)
    tp.tp_vocab_ce_fwd(s, 512, None, FAKE, None, None, None, workspace=(FAKE, 1 << 40), stream=0)
    tp.tp_vocab_ce_combine(s, [None, None], None, None, stream=0)


# ---------------------------------------------------------------------------
# attention dropout
# ---------------------------------------------------------------------------

def _bf16_attn(**kw):
    base = dict(dtype=tp.TP_BF16, hidden=512, ffn=2048, n_heads=4, head_dim=128)
    base.update(kw)
    return shape(**base)


def test_dropout_mask_bytes():
    # [batch][n_l][ceil(seq/32)][2][seq rounded up to 8] 16-bit words
    s = _bf16_attn(batch=2, seq=130)
    assert tp.tp_attn_dropout_mask_bytes(s) == 2 * 2 * 5 * 2 * 136 * 2
    c4 = shape(batch=1, seq=2048, hidden=20480, ffn=81920, n_heads=128, head_dim=160, tp_size=8, dtype=tp.TP_BF16)
    assert tp.tp_attn_dropout_mask_bytes(c4) == 16 * 64 * 2 * 2048 * 2


@pytest.mark.parametrize("kw,p,status", [
    ({}, 1.0, "TP_ERR_SHAPE"),
    ({}, -0.1, "TP_ERR_SHAPE"),
    ({}, float("nan"), "TP_ERR_SHAPE"),
    (dict(dtype=tp.TP_FP32), 0.1, "TP_ERR_DTYPE"),
    (dict(hidden=128, n_heads=4, head_dim=32), 0.1, "TP_ERR_HEADDIM"),
    (dict(tp_rank=3), 0.1, "TP_ERR_RANK"),
])
def test_dropout_validation(kw, p, status):
    s = _bf16_attn(**kw)
    d = tp.TpDropout(p, 1, 2)
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_fwd_dropout(s, d, *([FAKE] * 9), workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == status, str(ei.value)
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_bwd_dropout(s, d, *([FAKE] * 13), workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == status, str(ei.value)


def test_dropout_null_arguments():
    s = _bf16_attn()
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_fwd_dropout(s, None, *([FAKE] * 9), workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_NULL"
    args = [FAKE] * 9
    args[7] = None  # mask_i
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_fwd_dropout(s, tp.TpDropout(0.1, 1, 2), *args, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_NULL"
    args = [FAKE] * 13
    args[6] = FAKE + 2  # mask_i misaligned
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_bwd_dropout(s, tp.TpDropout(0.1, 1, 2), *args, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_ALIGN"



def test_ln_dropout_validation():
    s = shape()
    assert tp.tp_ln_dropout_mask_bytes(s) == 64 * 64 // 8
    for p, status in ((1.0, "TP_ERR_SHAPE"), (-1.0, "TP_ERR_SHAPE")):
        with pytest.raises(tp.TPError) as ei:
            tp.tp_ln_residual_fwd_dropout(s, tp.TpDropout(p, 1, 2), FAKE, [FAKE], None, FAKE, FAKE, 1e-5, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, stream=0)
        assert ei.value.name == status
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_fwd_dropout(s, tp.TpDropout(0.1, 1, 2), FAKE, [FAKE], None, FAKE, FAKE, 1e-5, FAKE, FAKE,
                                      FAKE, FAKE, None, stream=0)
    assert ei.value.name == "TP_ERR_NULL"  # mask
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_fwd_dropout(s, None, FAKE, [FAKE], None, FAKE, FAKE, 1e-5, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      stream=0)
    assert ei.value.name == "TP_ERR_NULL"  # dropout
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_bwd_dropout(s, tp.TpDropout(0.1, 1, 2), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                      None, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_NULL"  # d_block


def test_binding_refuses_host_and_strided_tensors():
    # The header wants contiguous device memory; the binding refuses a host
    # tensor or a strided view before the library sees its address.
    import torch
    s = shape()
    host = torch.zeros(64, 64)
    with pytest.raises(ValueError, match="device memory"):
        tp.tp_mlp_fwd(s, host, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)
    with pytest.raises(ValueError, match="device memory"):
        tp.tp_mlp_fwd(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=torch.zeros(16, dtype=torch.uint8),
                      stream=0)
    strided = torch.zeros(64, 128)[:, :64]

    class _View:  # a strided "device" tensor: is_cuda true, not contiguous
        is_cuda = True
        def is_contiguous(self):
            return strided.is_contiguous()
        def data_ptr(self):
            return FAKE
    with pytest.raises(ValueError, match="contiguous"):
        tp.tp_mlp_fwd(s, _View(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, workspace=(FAKE, 1 << 40), stream=0)


@pytest.mark.parametrize("p", [1.0 - 2.0 ** -17, 1.0 - 2.0 ** -20, 1.0 - 2.0 ** -24])
def test_dropout_p_with_nothing_kept_is_refused(p):
    # round(65536 p) = 65536 would keep nothing and make the scale infinite
    import numpy as np
    assert np.floor(np.float32(p) * np.float32(65536.0) + np.float32(0.5)) >= 65536
    s = _bf16_attn()
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_fwd_dropout(s, tp.TpDropout(p, 1, 2), *([FAKE] * 9), workspace=(FAKE, 1 << 40), stream=0)
    assert ei.value.name == "TP_ERR_SHAPE"
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_fwd_dropout(shape(), tp.TpDropout(p, 1, 2), FAKE, [FAKE], None, FAKE, FAKE, 1e-5, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.name == "TP_ERR_SHAPE"


def test_dropout_largest_realizable_p_passes_validation():
    # p = 65535/65536 (thr 65535) is valid: the call then fails only on the
    # workspace check that follows, proving p itself was accepted
    s = _bf16_attn()
    with pytest.raises(tp.TPError) as ei:
        tp.tp_attn_fwd_dropout(s, tp.TpDropout(65535.0 / 65536.0, 1, 2), *([FAKE] * 9), workspace=(FAKE, 0),
                               stream=0)
    assert ei.value.name == "TP_ERR_WORKSPACE", str(ei.value)


def test_noalloc_ln_backward_refuses_shapes_beyond_its_scratch():
    assert tp.tp_ln_residual_bwd_noalloc_max_scratch_bytes() == 48 << 20
    # hidden 24576 with 256 rows needs 256 runs x 2 x 24576 fp32 partials (48 MiB) plus the
    # bias column sums: more than the scratch; refused before any device call
    s = shape(batch=1, seq=256, hidden=24576, ffn=4 * 24576, n_heads=192, head_dim=128, tp_size=8, dtype=tp.TP_BF16)
    assert tp.tp_ln_workspace_bytes(s) > 48 << 20
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_bwd_noalloc(s, *([FAKE] * 10), stream=0)
    assert ei.value.name == "TP_ERR_SHAPE" and "scratch" in str(ei.value)
    # its other argument checks are those of tp_ln_residual_bwd
    with pytest.raises(tp.TPError) as ei:
        tp.tp_ln_residual_bwd_noalloc(shape(), None, *([FAKE] * 9), stream=0)
    assert ei.value.name == "TP_ERR_NULL"
    # the 530B-like shard's hidden size fits
    c4 = shape(batch=1, seq=2048, hidden=20480, ffn=81920, n_heads=128, head_dim=160, tp_size=8, dtype=tp.TP_BF16)
    assert 0 < tp.tp_ln_workspace_bytes(c4) <= 48 << 20
