"""One tensor-parallel rank's share of a Megatron-style Transformer layer on
AMD Instinct MI355X (gfx950): Python binding of the C ABI in include/tp_layer.h.

This module only marshals arguments: every step of the computation runs in the
HIP library lib/libtp_layer.so (build it with
`python -m tensor_transformer_layer_tp_amd.build`). Importing this module does
not need a GPU; calling a compute entry point does. If the library is missing,
every call raises -- there is no fallback.

Tensors are passed as torch tensors (their data_ptr is used), plain integer
device addresses, or None for the optional outputs. `stream` defaults to
torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "TpShape", "TPError", "TP_FP32", "TP_BF16", "STATUS", "library_path", "load_library",
    "exported_symbols", "tp_mlp_workspace_bytes", "tp_attn_workspace_bytes", "tp_mlp_fwd",
    "tp_mlp_bwd", "tp_attn_fwd", "tp_attn_bwd", "tp_sum_partials", "tp_last_error", "tp_profile_enable",
    "tp_profile_collect", "STEPS", "tp_ln_workspace_bytes", "tp_ln_residual_fwd", "tp_ln_residual_bwd",
    "tp_vocab_workspace_bytes", "tp_vocab_ce_fwd", "tp_vocab_ce_combine", "tp_vocab_ce_bwd", "TpDropout",
    "tp_attn_dropout_mask_bytes", "tp_attn_fwd_dropout", "tp_attn_bwd_dropout", "tp_ln_dropout_mask_bytes",
    "tp_ln_residual_fwd_dropout", "tp_ln_residual_bwd_dropout", "tp_ln_residual_bwd_noalloc", "tp_attn_qkv_bytes",
    "tp_ln_residual_bwd_noalloc_max_scratch_bytes", "tp_step_kernel",
]

TP_FP32, TP_BF16 = 0, 1
STATUS = {
    0: "TP_OK", -1: "TP_ERR_NULL", -2: "TP_ERR_SHAPE", -3: "TP_ERR_DIVISIBILITY", -4: "TP_ERR_RANK",
    -5: "TP_ERR_DTYPE", -6: "TP_ERR_HEADDIM", -7: "TP_ERR_WORKSPACE", -8: "TP_ERR_ALIGN", -9: "TP_ERR_HIP",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "tp_layer.h")


def library_path() -> str:
    return os.environ.get("TP_LAYER_LIB", os.path.join(_HERE, "lib", "libtp_layer.so"))


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class TpShape(ctypes.Structure):
    """Mirror of tp_shape: full (unsharded) sizes plus (tp_rank, tp_size)."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "seq", "hidden", "ffn", "n_heads", "head_dim", "tp_rank", "tp_size", "dtype", "causal", "alibi")]

    @classmethod
    def make(cls, *, batch, seq, hidden, ffn, n_heads, head_dim, tp_rank=0, tp_size=1, dtype=TP_BF16,
             causal=1, alibi=0) -> "TpShape":
        if isinstance(dtype, str):
            dtype = {"fp32": TP_FP32, "bf16": TP_BF16}[dtype]
        return cls(batch, seq, hidden, ffn, n_heads, head_dim, tp_rank, tp_size, dtype, int(causal), int(alibi))


class TpDropout(ctypes.Structure):
    """Mirror of tp_dropout: drop probability and the Philox key (seed, offset)."""
    _fields_ = [("p", ctypes.c_float), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


_lib = None
_vp, _sz, _st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "tp_mlp_workspace_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_attn_workspace_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_attn_qkv_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_mlp_fwd": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 7 + [_vp, _sz, _vp]),
    "tp_mlp_bwd": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 11 + [_vp, _sz, _vp]),
    "tp_attn_fwd": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 8 + [_vp, _sz, _vp]),
    "tp_attn_bwd": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 12 + [_vp, _sz, _vp]),
    "tp_sum_partials": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp, _vp]),
    "tp_ln_workspace_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_ln_residual_fwd": (_st, [ctypes.POINTER(TpShape), _vp, ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp, _vp,
                                 ctypes.c_float, _vp, _vp, _vp, _vp, _vp]),
    "tp_ln_residual_bwd": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 10 + [_vp, _sz, _vp]),
    "tp_vocab_workspace_bytes": (_sz, [ctypes.POINTER(TpShape), ctypes.c_int32]),
    "tp_vocab_ce_fwd": (_st, [ctypes.POINTER(TpShape), ctypes.c_int32] + [_vp] * 5 + [_vp, _sz, _vp]),
    "tp_vocab_ce_combine": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(_vp), ctypes.c_int32, _vp, _vp, _vp]),
    "tp_vocab_ce_bwd": (_st, [ctypes.POINTER(TpShape), ctypes.c_int32] + [_vp] * 8 + [_vp, _sz, _vp]),
    "tp_attn_dropout_mask_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_attn_fwd_dropout": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(TpDropout)] + [_vp] * 9 + [_vp, _sz, _vp]),
    "tp_attn_bwd_dropout": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(TpDropout)] + [_vp] * 13 + [_vp, _sz, _vp]),
    "tp_ln_dropout_mask_bytes": (_sz, [ctypes.POINTER(TpShape)]),
    "tp_ln_residual_fwd_dropout": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(TpDropout), _vp, ctypes.POINTER(_vp),
                                         ctypes.c_int32, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tp_ln_residual_bwd_dropout": (_st, [ctypes.POINTER(TpShape), ctypes.POINTER(TpDropout)] + [_vp] * 12
                                   + [_vp, _sz, _vp]),
    "tp_ln_residual_bwd_noalloc": (_st, [ctypes.POINTER(TpShape)] + [_vp] * 10 + [_vp]),
    "tp_ln_residual_bwd_noalloc_max_scratch_bytes": (_sz, []),
    "tp_profile_enable": (_st, [ctypes.c_uint32]),
    "tp_profile_collect": (_st, [ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_step_kernel": (ctypes.c_char_p, [ctypes.POINTER(TpShape), ctypes.c_int32]),
}

# Step ids of tp_profile_enable / tp_profile_collect (TP_STEP_* in the header).
STEPS = {
    "qkv_proj": 1, "attn_fwd": 2, "out_proj": 3, "fc1": 4, "fc2": 5, "fc2_dgrad": 6, "fc2_wgrad": 7,
    "fc1_wgrad": 8, "fc1_dgrad": 9, "out_dgrad": 10, "out_wgrad": 11, "attn_bwd": 12, "qkv_wgrad": 13,
    "qkv_dgrad": 14, "bias_grads": 15, "ln_fwd": 16, "ln_bwd": 17, "logits": 18, "ce_stats": 19,
    "ce_combine": 20, "ce_dlogits": 21, "logits_dgrad": 22, "logits_wgrad": 23, "transposes": 24,
}


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is missing: build it with "
                               "`python -m tensor_transformer_layer_tp_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols() -> list[str]:
    """Names of the functions include/tp_layer.h declares."""
    with open(_HEADER) as fh:
        text = fh.read()
    return re.findall(r"^\s*(?:size_t|tp_status|const char\*)\s+(tp_\w+)\s*\(", text, flags=re.M)


def _device_tensor(t, what: str = "tensor"):
    """Refuse a tensor the library cannot read as the header requires: host
    memory (a kernel would fault on its address) or a non-contiguous view
    (the library reads dense row-major storage)."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be in device memory (got a tensor on {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (row-major); call .contiguous() first")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t or None
    _device_tensor(t)
    return t.data_ptr() or None


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    _device_tensor(ws, "workspace")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _check(status: int):
    if status != 0:
        raise TPError(status, tp_last_error())


def tp_last_error() -> str:
    return load_library().tp_last_error().decode()


def tp_step_kernel(shape: TpShape, step) -> str | None:
    """Name of the main kernel a GEMM step (a STEPS name or id) launches for
    this shape, or None (invalid shape, not a product, or no launch)."""
    r = load_library().tp_step_kernel(ctypes.byref(shape), STEPS[step] if isinstance(step, str) else int(step))
    return r.decode() if r is not None else None


def tp_mlp_workspace_bytes(shape: TpShape) -> int:
    return load_library().tp_mlp_workspace_bytes(ctypes.byref(shape))


def tp_attn_workspace_bytes(shape: TpShape) -> int:
    return load_library().tp_attn_workspace_bytes(ctypes.byref(shape))


def tp_attn_qkv_bytes(shape: TpShape) -> int:
    """Bytes of the saved projection qkv_i (five 16-bit planes on the matrix-core path, else fp32)."""
    return load_library().tp_attn_qkv_bytes(ctypes.byref(shape))


def tp_mlp_fwd(shape, X, A_i, b1_i, B_i, pre_i, y_i, Z_i, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_mlp_fwd(ctypes.byref(shape), _ptr(X), _ptr(A_i), _ptr(b1_i), _ptr(B_i), _ptr(pre_i),
                                     _ptr(y_i), _ptr(Z_i), w, wn, _stream(stream)))


def tp_mlp_bwd(shape, X, A_i, B_i, pre_i, y_i, dZ, dX_i, dA_i, db1_i, dB_i, db2_or_null=None, workspace=None,
               stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_mlp_bwd(ctypes.byref(shape), _ptr(X), _ptr(A_i), _ptr(B_i), _ptr(pre_i), _ptr(y_i),
                                     _ptr(dZ), _ptr(dX_i), _ptr(dA_i), _ptr(db1_i), _ptr(dB_i), _ptr(db2_or_null),
                                     w, wn, _stream(stream)))


def tp_attn_fwd(shape, X, Wqkv_i, bqkv_i, Wo_i, qkv_i, ctx_i, lse_i, O_i, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_attn_fwd(ctypes.byref(shape), _ptr(X), _ptr(Wqkv_i), _ptr(bqkv_i), _ptr(Wo_i),
                                      _ptr(qkv_i), _ptr(ctx_i), _ptr(lse_i), _ptr(O_i), w, wn, _stream(stream)))


def tp_attn_bwd(shape, X, Wqkv_i, Wo_i, qkv_i, ctx_i, lse_i, dO, dX_i, dWqkv_i, dbqkv_i, dWo_i, dbo_or_null=None,
                workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_attn_bwd(ctypes.byref(shape), _ptr(X), _ptr(Wqkv_i), _ptr(Wo_i), _ptr(qkv_i),
                                      _ptr(ctx_i), _ptr(lse_i), _ptr(dO), _ptr(dX_i), _ptr(dWqkv_i), _ptr(dbqkv_i),
                                      _ptr(dWo_i), _ptr(dbo_or_null), w, wn, _stream(stream)))


def tp_profile_enable(step_mask: int):
    _check(load_library().tp_profile_enable(step_mask))


def tp_profile_collect(step: int):
    """-> (launch sequences recorded, total GPU ms) for one step id."""
    n, ms = ctypes.c_int32(), ctypes.c_double()
    _check(load_library().tp_profile_collect(step, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def tp_sum_partials(shape, parts, bias_or_null, out, stream=None):
    arr = (_vp * len(parts))(*[_ptr(p) for p in parts])
    _check(load_library().tp_sum_partials(ctypes.byref(shape), arr, len(parts), _ptr(bias_or_null), _ptr(out),
                                          _stream(stream)))


def tp_ln_workspace_bytes(shape: TpShape) -> int:
    return load_library().tp_ln_workspace_bytes(ctypes.byref(shape))


def tp_ln_residual_fwd(shape, resid_in, parts, bias_or_null, gamma, beta, eps, resid_out, ln_out, mean, rstd,
                       stream=None):
    """resid_out = resid_in + sum(parts) + bias; ln_out = LayerNorm(resid_out) (see the header)."""
    arr = (_vp * max(len(parts), 1))(*[_ptr(p) for p in parts])
    _check(load_library().tp_ln_residual_fwd(ctypes.byref(shape), _ptr(resid_in), arr, len(parts),
                                             _ptr(bias_or_null), _ptr(gamma), _ptr(beta), float(eps),
                                             _ptr(resid_out), _ptr(ln_out), _ptr(mean), _ptr(rstd), _stream(stream)))


def tp_ln_residual_bwd(shape, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null, d_resid, dgamma, dbeta,
                       dbias_or_null=None, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_ln_residual_bwd(ctypes.byref(shape), _ptr(resid_out), _ptr(mean), _ptr(rstd),
                                             _ptr(gamma), _ptr(d_ln_out), _ptr(d_resid_out_or_null), _ptr(d_resid),
                                             _ptr(dgamma), _ptr(dbeta), _ptr(dbias_or_null), w, wn,
                                             _stream(stream)))


def tp_ln_residual_bwd_noalloc_max_scratch_bytes() -> int:
    return load_library().tp_ln_residual_bwd_noalloc_max_scratch_bytes()


def tp_ln_residual_bwd_noalloc(shape, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null, d_resid, dgamma,
                               dbeta, dbias_or_null=None, stream=None):
    """tp_ln_residual_bwd with the library's own scratch instead of a workspace."""
    _check(load_library().tp_ln_residual_bwd_noalloc(ctypes.byref(shape), _ptr(resid_out), _ptr(mean), _ptr(rstd),
                                                     _ptr(gamma), _ptr(d_ln_out), _ptr(d_resid_out_or_null),
                                                     _ptr(d_resid), _ptr(dgamma), _ptr(dbeta), _ptr(dbias_or_null),
                                                     _stream(stream)))


def tp_vocab_workspace_bytes(shape: TpShape, vocab: int) -> int:
    return load_library().tp_vocab_workspace_bytes(ctypes.byref(shape), int(vocab))


def tp_vocab_ce_fwd(shape, vocab, X, W_i, labels, logits_i, stats_i, workspace=None, stream=None):
    """logits_i = X W_i^T and the slice's per-token aggregates (see the header)."""
    w, wn = _ws(workspace)
    _check(load_library().tp_vocab_ce_fwd(ctypes.byref(shape), int(vocab), _ptr(X), _ptr(W_i), _ptr(labels),
                                          _ptr(logits_i), _ptr(stats_i), w, wn, _stream(stream)))


def tp_vocab_ce_combine(shape, stats, loss, lse, stream=None):
    arr = (_vp * len(stats))(*[_ptr(p) for p in stats])
    _check(load_library().tp_vocab_ce_combine(ctypes.byref(shape), arr, len(stats), _ptr(loss), _ptr(lse),
                                              _stream(stream)))


def tp_vocab_ce_bwd(shape, vocab, X, W_i, labels, logits_i, lse, dloss, dX_i, dW_i, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_vocab_ce_bwd(ctypes.byref(shape), int(vocab), _ptr(X), _ptr(W_i), _ptr(labels),
                                          _ptr(logits_i), _ptr(lse), _ptr(dloss), _ptr(dX_i), _ptr(dW_i), w, wn,
                                          _stream(stream)))


def tp_attn_dropout_mask_bytes(shape: TpShape) -> int:
    return load_library().tp_attn_dropout_mask_bytes(ctypes.byref(shape))


def _drop(dropout):
    return None if dropout is None else ctypes.byref(dropout)


def tp_attn_fwd_dropout(shape, dropout, X, Wqkv_i, bqkv_i, Wo_i, qkv_i, ctx_i, lse_i, mask_i, O_i, workspace=None,
                        stream=None):
    """tp_attn_fwd with attention-probability dropout; mask_i receives the keep bits."""
    w, wn = _ws(workspace)
    _check(load_library().tp_attn_fwd_dropout(ctypes.byref(shape), _drop(dropout), _ptr(X), _ptr(Wqkv_i),
                                              _ptr(bqkv_i), _ptr(Wo_i), _ptr(qkv_i), _ptr(ctx_i), _ptr(lse_i),
                                              _ptr(mask_i), _ptr(O_i), w, wn, _stream(stream)))


def tp_attn_bwd_dropout(shape, dropout, X, Wqkv_i, Wo_i, qkv_i, ctx_i, lse_i, mask_i, dO, dX_i, dWqkv_i, dbqkv_i,
                        dWo_i, dbo_or_null=None, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_attn_bwd_dropout(ctypes.byref(shape), _drop(dropout), _ptr(X), _ptr(Wqkv_i),
                                              _ptr(Wo_i), _ptr(qkv_i), _ptr(ctx_i), _ptr(lse_i), _ptr(mask_i),
                                              _ptr(dO), _ptr(dX_i), _ptr(dWqkv_i), _ptr(dbqkv_i), _ptr(dWo_i),
                                              _ptr(dbo_or_null), w, wn, _stream(stream)))


def tp_ln_dropout_mask_bytes(shape: TpShape) -> int:
    return load_library().tp_ln_dropout_mask_bytes(ctypes.byref(shape))


def tp_ln_residual_fwd_dropout(shape, dropout, resid_in, parts, bias_or_null, gamma, beta, eps, resid_out, ln_out,
                               mean, rstd, mask, stream=None):
    """tp_ln_residual_fwd with dropout on the block output; mask receives the keep bits."""
    arr = (_vp * max(len(parts), 1))(*[_ptr(p) for p in parts])
    _check(load_library().tp_ln_residual_fwd_dropout(ctypes.byref(shape), _drop(dropout), _ptr(resid_in), arr,
                                                     len(parts), _ptr(bias_or_null), _ptr(gamma), _ptr(beta),
                                                     float(eps), _ptr(resid_out), _ptr(ln_out), _ptr(mean), _ptr(rstd),
                                                     _ptr(mask), _stream(stream)))


def tp_ln_residual_bwd_dropout(shape, dropout, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null, mask,
                               d_resid, d_block, dgamma, dbeta, dbias_or_null=None, workspace=None, stream=None):
    w, wn = _ws(workspace)
    _check(load_library().tp_ln_residual_bwd_dropout(ctypes.byref(shape), _drop(dropout), _ptr(resid_out),
                                                     _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(d_ln_out),
                                                     _ptr(d_resid_out_or_null), _ptr(mask), _ptr(d_resid),
                                                     _ptr(d_block), _ptr(dgamma), _ptr(dbeta), _ptr(dbias_or_null),
                                                     w, wn, _stream(stream)))
