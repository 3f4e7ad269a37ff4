"""Device buffers for one rank's layer shard and the four calls of one step.

`LayerShard` owns (through torch's allocator) every output buffer and one
workspace shared by the four calls, which run back to back on one stream:
    forward:  tp_attn_fwd, tp_mlp_fwd
    backward: tp_mlp_bwd, tp_attn_bwd
It performs no arithmetic of its own.
"""
from __future__ import annotations

import torch

from . import TP_BF16, TP_FP32, TpShape, tp_attn_bwd, tp_attn_fwd, tp_attn_qkv_bytes, tp_attn_workspace_bytes, \
    tp_mlp_bwd, tp_mlp_fwd, tp_mlp_workspace_bytes

_DT = {TP_FP32: torch.float32, TP_BF16: torch.bfloat16}
INPUTS = ("X_attn", "Wqkv", "bqkv", "Wo", "dO", "X_mlp", "A", "b1", "B", "dZ")


class LayerShard:
    def __init__(self, shape: TpShape, inputs: dict, device="cuda", replicated_bias_grads=True, fill=None):
        """inputs: the rank's tensors named as in INPUTS, already on `device` in
        the shape's dtype. `fill` (e.g. float('nan')) pre-fills every output."""
        self.shape = shape
        self.dev = torch.device(device)
        dt = _DT[shape.dtype]
        self.inp = {k: inputs[k] for k in INPUTS}
        for k, t in self.inp.items():
            if t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"input {k} must be contiguous {dt}")
        T = shape.batch * shape.seq
        h = shape.hidden
        nl = shape.n_heads // shape.tp_size
        hl = nl * shape.head_dim
        fl = shape.ffn // shape.tp_size

        def buf(*s, dtype=dt):
            t = torch.empty(*s, dtype=dtype, device=self.dev)
            if fill is not None:
                # a byte buffer takes all-ones bytes: NaN in every float format it holds
                t.fill_(255 if dtype == torch.uint8 else fill)
            return t

        self.out = {
            # the saved projection, in the form tp_attn_qkv_bytes describes
            "qkv": buf(max(tp_attn_qkv_bytes(shape), 1), dtype=torch.uint8), "ctx": buf(T, hl), "lse": buf(shape.batch, nl, shape.seq, dtype=torch.float32),
            "O": buf(T, h), "pre": buf(T, fl), "y": buf(T, fl), "Z": buf(T, h),
            "dX_mlp": buf(T, h), "dA": buf(h, fl), "db1": buf(fl), "dB": buf(fl, h),
            "dX_attn": buf(T, h), "dWqkv": buf(h, 3 * hl), "dbqkv": buf(3 * hl), "dWo": buf(hl, h),
        }
        if replicated_bias_grads:
            self.out["db2"] = buf(h)
            self.out["dbo"] = buf(h)
        nbytes = max(tp_mlp_workspace_bytes(shape), tp_attn_workspace_bytes(shape), 1)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.dev)

    def forward(self, stream=None):
        i, o, s = self.inp, self.out, self.shape
        tp_attn_fwd(s, i["X_attn"], i["Wqkv"], i["bqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"], o["O"],
                    self.workspace, stream)
        tp_mlp_fwd(s, i["X_mlp"], i["A"], i["b1"], i["B"], o["pre"], o["y"], o["Z"], self.workspace, stream)

    def backward(self, stream=None):
        i, o, s = self.inp, self.out, self.shape
        tp_mlp_bwd(s, i["X_mlp"], i["A"], i["B"], o["pre"], o["y"], i["dZ"], o["dX_mlp"], o["dA"], o["db1"],
                   o["dB"], o.get("db2"), self.workspace, stream)
        tp_attn_bwd(s, i["X_attn"], i["Wqkv"], i["Wo"], o["qkv"], o["ctx"], o["lse"], i["dO"], o["dX_attn"],
                    o["dWqkv"], o["dbqkv"], o["dWo"], o.get("dbo"), self.workspace, stream)

    def step(self, stream=None):
        self.forward(stream)
        self.backward(stream)
