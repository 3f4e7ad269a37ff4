"""Seeded synthetic inputs for one tensor-parallel rank's layer shard.

This module is shared by the tests, the benchmark and the smoke check. It
only draws numbers and holds the workload table: it contains none of the
layer's arithmetic, so neither the fp64 oracle nor the HIP path depends on
the other through it.

Workloads follow the shapes the pages print:
  * GPT-2-like 1.2B row of the scaling study (hidden 1536, 16 heads) --
    Megatron-LM deep dive, "Scaling Study", Table 1.
  * 8.3B GPT-2 model (hidden 3072, 24 heads of 128) -- same page, Table 2.
  * MT-NLG 530B (105 layers, hidden 20480, 128 heads, seq 2048, 8-way
    tensor parallel) -- MT-NLG 530B deep dive, section 4.1.
  * BLOOM 176B under 8-way tensor parallelism with ALiBi -- Megatron-DeepSpeed
    blog, sections 2.3 and 4.3.
The FFN width is 4x hidden. Weights are drawn N(0, 0.02); the weights that
feed a residual add (the attention output projection and the second MLP
matrix) are scaled by 1/sqrt(2N) for the 530B-like shard, N = 105 layers
(Megatron-LM deep dive, "training recipe" table, initialization row).
X and the incoming gradients are N(0, 1): X stands for a LayerNorm output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "draw_shard", "draw_full", "DRAW_ORDER", "draw_ln", "LN_DRAW_ORDER", "draw_vocab", "GPT2_VOCAB", "VOCAB_PADDED"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    tp_size: int
    dtype: str            # "fp32" or "bf16": storage type; accumulation is fp32
    alibi: bool = False
    causal: bool = True
    w_std: float = 0.02   # Wqkv and A
    wout_std: float = 0.02  # Wo and B (weights before a residual add)
    bias_std: float = 0.0
    x_std: float = 1.0
    g_std: float = 1.0

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def h_local(self) -> int:
        return self.hidden // self.tp_size

    @property
    def heads_local(self) -> int:
        return self.n_heads // self.tp_size

    @property
    def ffn_local(self) -> int:
        return self.ffn // self.tp_size

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_fp32_tp2": Workload("tiny_fp32_tp2", batch=2, seq=32, hidden=64, n_heads=4,
                              head_dim=16, ffn=256, tp_size=2, dtype="fp32"),
    "gpt2_1p2b_tp1": Workload("gpt2_1p2b_tp1", batch=8, seq=1024, hidden=1536, n_heads=16,
                              head_dim=96, ffn=6144, tp_size=1, dtype="bf16"),
    "gpt_8p3b_tp8": Workload("gpt_8p3b_tp8", batch=16, seq=1024, hidden=3072, n_heads=24,
                             head_dim=128, ffn=12288, tp_size=8, dtype="bf16"),
    "mtnlg_530b_tp8": Workload("mtnlg_530b_tp8", batch=1, seq=2048, hidden=20480, n_heads=128,
                               head_dim=160, ffn=81920, tp_size=8, dtype="bf16",
                               wout_std=0.02 / math.sqrt(2 * 105)),
    "bloom_176b_tp8": Workload("bloom_176b_tp8", batch=2, seq=2048, hidden=14336, n_heads=112,
                               head_dim=128, ffn=57344, tp_size=8, dtype="bf16", alibi=True),
}

# Fixed order of the draws from one generator.
DRAW_ORDER = ("X_attn", "Wqkv", "bqkv", "Wo", "bo", "dO", "X_mlp", "A", "b1", "B", "b2", "dZ")

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def _normal(gen: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    if std == 0.0:
        return torch.zeros(shape, dtype=dtype)
    t = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)  # round-to-nearest-even for bf16


def _shapes(w: Workload, tp: int) -> dict:
    h, T = w.hidden, w.tokens
    hl, fl = h // tp, w.ffn // tp
    return {
        "X_attn": ((T, h), w.x_std), "Wqkv": ((h, 3 * hl), w.w_std), "bqkv": ((3 * hl,), w.bias_std),
        "Wo": ((hl, h), w.wout_std), "bo": ((h,), w.bias_std), "dO": ((T, h), w.g_std),
        "X_mlp": ((T, h), w.x_std), "A": ((h, fl), w.w_std), "b1": ((fl,), w.bias_std),
        "B": ((fl, h), w.wout_std), "b2": ((h,), w.bias_std), "dZ": ((T, h), w.g_std),
    }


def draw_shard(w: Workload, seed: int = 0, skip=()) -> dict:
    """Draw one rank's inputs directly at shard shape (a shard of iid N(0, s)
    entries is itself iid N(0, s)). Returns CPU tensors in the storage dtype.
    Names in `skip` are drawn (to keep the stream aligned) but not returned."""
    gen = torch.Generator().manual_seed(seed)
    dt = _TORCH_DTYPE[w.dtype]
    out = {}
    for name, (shape, std) in _shapes(w, w.tp_size).items():
        t = _normal(gen, shape, std, dt)
        if name not in skip:
            out[name] = t
    return out


def draw_full(w: Workload, seed: int = 0) -> dict:
    """Draw the unsharded layer (tp = 1 shapes) for emulation across ranks."""
    gen = torch.Generator().manual_seed(seed)
    dt = _TORCH_DTYPE[w.dtype]
    return {name: _normal(gen, shape, std, dt) for name, (shape, std) in _shapes(w, 1).items()}


# Residual add + LayerNorm after a block: fixed order of the draws.
LN_DRAW_ORDER = ("resid_in", "parts", "bias", "gamma", "beta", "d_ln_out", "d_resid_out")


def draw_ln(w: Workload, seed: int = 0, n_parts: int = 1, bias_std: float = 0.0) -> dict:
    """Inputs of the residual add + LayerNorm that follows a block, at w's
    token count and hidden size, from their own generator: the residual
    stream and each partial block output N(0, 1); gamma N(1, 0.1^2) and beta
    N(0, 0.1^2) (LayerNorm weights start at 1 and 0; the spread makes every
    term of the backward matter); the replicated bias N(0, bias_std^2) (None
    when bias_std is 0); the gradients arriving at the LayerNorm output and
    along the residual stream N(0, 1). CPU tensors in the storage dtype."""
    gen = torch.Generator().manual_seed(seed)
    dt = _TORCH_DTYPE[w.dtype]
    T, h = w.tokens, w.hidden
    out = {"resid_in": _normal(gen, (T, h), 1.0, dt),
           "parts": [_normal(gen, (T, h), 1.0, dt) for _ in range(n_parts)]}
    out["bias"] = _normal(gen, (h,), bias_std, dt) if bias_std > 0 else None
    out["gamma"] = (1.0 + _normal(gen, (h,), 0.1, torch.float32)).to(dt)
    out["beta"] = _normal(gen, (h,), 0.1, dt)
    out["d_ln_out"] = _normal(gen, (T, h), 1.0, dt)
    out["d_resid_out"] = _normal(gen, (T, h), 1.0, dt)
    return out


# Output layer: GPT-2's vocabulary padded so that it splits evenly over up to
# 8 ranks (Megatron-LM deep dive, training-recipe table).
GPT2_VOCAB = 50257
VOCAB_PADDED = 51200


def draw_vocab(w: Workload, vocab: int = VOCAB_PADDED, seed: int = 0, ranks=None, label_max: int | None = None,
               dloss: str = "mean") -> dict:
    """Inputs of the vocabulary-parallel output layer at w's tokens and hidden
    size, from their own generator: the final hidden states X N(0, 1) (a
    LayerNorm output), the embedding table N(0, w.w_std^2) -- only the slices
    of `ranks` (default: all) are returned, as {rank: [V/p, h]} (the whole
    table is drawn slice by slice in rank order, so any subset is the same
    numbers) -- labels uniform over [0, label_max) (default: the real GPT-2
    vocabulary when it fits, so padded ids are never targets), and the loss
    gradient: 1/T per token for a mean ("mean") or N(0, 1) ("normal")."""
    gen = torch.Generator().manual_seed(seed)
    dt = _TORCH_DTYPE[w.dtype]
    T, h, p = w.tokens, w.hidden, w.tp_size
    n = vocab // p
    out = {"X": _normal(gen, (T, h), 1.0, dt), "W": {}}
    want = set(range(p)) if ranks is None else set(ranks)
    for r in range(p):
        t = _normal(gen, (n, h), w.w_std, dt)
        if r in want:
            out["W"][r] = t
    if label_max is None:
        label_max = GPT2_VOCAB if vocab >= GPT2_VOCAB else vocab
    out["labels"] = torch.randint(0, label_max, (T,), generator=gen, dtype=torch.int64).to(torch.int32)
    if dloss == "mean":
        out["dloss"] = torch.full((T,), 1.0 / max(T, 1), dtype=torch.float32)
    else:
        out["dloss"] = torch.randn((T,), generator=gen, dtype=torch.float32)
    return out
