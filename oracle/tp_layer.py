"""The oracle's definitions (float64, NumPy). Test infrastructure only.

Notation (per rank r of p): T = batch*seq tokens, h hidden, h_l = h/p,
n_l = n_heads/p local heads of width d, f_l = ffn/p. All matrices are
row-major; token t = batch_index*seq + position.
"""
from __future__ import annotations

import math

import numpy as np

# tanh form of GeLU: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
# The pages name GeLU without a formula (Megatron-LM deep dive, "MLP: column
# parallel then row parallel", Fig. 3a); the tanh form is the reading taken.
GELU_C = 0.044715
_K0 = math.sqrt(2.0 / math.pi)


def gelu(x: np.ndarray) -> np.ndarray:
    u = _K0 * (x + GELU_C * x ** 3)
    return 0.5 * x * (1.0 + np.tanh(u))


def gelu_grad(x: np.ndarray) -> np.ndarray:
    """d gelu / dx: 0.5(1+t) + 0.5 x (1-t^2) u'(x), t = tanh(u)."""
    u = _K0 * (x + GELU_C * x ** 3)
    t = np.tanh(u)
    du = _K0 * (1.0 + 3.0 * GELU_C * x ** 2)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


# ---------------------------------------------------------------------------
# Sharding rules (Megatron-LM deep dive, Fig. 3a / 3b; MT-NLG deep dive 2.4):
# column-parallel weights are split by output columns, row-parallel weights by
# input rows. The QKV weight [h, 3h] = [Wq | Wk | Wv] is split by heads: rank r
# owns global heads r*n_l .. r*n_l+n_l-1 and keeps [Wq_r | Wk_r | Wv_r].
# ---------------------------------------------------------------------------

def column_shard(W: np.ndarray, rank: int, tp: int) -> np.ndarray:
    n = W.shape[-1]
    assert n % tp == 0
    w = n // tp
    return W[..., rank * w:(rank + 1) * w]


def row_shard(W: np.ndarray, rank: int, tp: int) -> np.ndarray:
    n = W.shape[0]
    assert n % tp == 0
    w = n // tp
    return W[rank * w:(rank + 1) * w]


def qkv_weight_shard(Wqkv: np.ndarray, rank: int, tp: int) -> np.ndarray:
    h3 = Wqkv.shape[-1]
    assert h3 % 3 == 0
    h = h3 // 3
    parts = [column_shard(Wqkv[..., i * h:(i + 1) * h], rank, tp) for i in range(3)]
    return np.concatenate(parts, axis=-1)


def qkv_bias_shard(bqkv: np.ndarray, rank: int, tp: int) -> np.ndarray:
    return qkv_weight_shard(bqkv, rank, tp)


def layer_weight_shapes(hidden: int, ffn: int, tp: int) -> dict:
    """Per-rank parameter shapes of the layer's two tensor-parallel blocks.
    b2 and bo are replicated (added once after the sum over ranks)."""
    hl, fl = hidden // tp, ffn // tp
    return {
        "Wqkv": (hidden, 3 * hl), "bqkv": (3 * hl,), "Wo": (hl, hidden), "bo": (hidden,),
        "A": (hidden, fl), "b1": (fl,), "B": (fl, hidden), "b2": (hidden,),
    }


# ---------------------------------------------------------------------------
# MLP block (Megatron-LM deep dive, Fig. 3a; Megatron-DeepSpeed blog 2.1):
#   pre_r = X A_r + b1_r ; y_r = GeLU(pre_r) ; Z_r = y_r B_r   (partial sum)
#   Z = sum_r Z_r + b2   (the g all-reduce, then the replicated bias)
# ---------------------------------------------------------------------------

def mlp_fwd(X, A_r, b1_r, B_r):
    pre = X @ A_r + b1_r
    y = gelu(pre)
    Z_r = y @ B_r
    return pre, y, Z_r


def mlp_bwd(X, A_r, B_r, pre, y, dZ):
    """Gradients of <Z_r + b2, dZ> (dZ replicated: g's backward is identity).
    Returns dX_r (partial; f's backward sums it over ranks), dA_r, db1_r, dB_r,
    db2 (replicated bias, counted once)."""
    dY = dZ @ B_r.T
    dPre = dY * gelu_grad(pre)
    dB_r = y.T @ dZ
    dA_r = X.T @ dPre
    db1_r = dPre.sum(axis=0)
    dX_r = dPre @ A_r.T
    db2 = dZ.sum(axis=0)
    return dX_r, dA_r, db1_r, dB_r, db2


# ---------------------------------------------------------------------------
# Attention block (Megatron-LM deep dive, Fig. 3b): QKV column-parallel by
# heads, per-head scores / softmax / value aggregation local to the rank,
# output projection row-parallel -> partial sum.
# Readings: score scale 1/sqrt(d); causal mask keeps key j <= query i
# (masked weights exactly zero); ALiBi adds -m_k (i - j) after the scaling,
# m_k = 2^(-8k/n_heads) for 1-based global head k (Megatron-DeepSpeed blog 4.3).
# ---------------------------------------------------------------------------

def alibi_slope(k: int, n_heads: int) -> float:
    return 2.0 ** (-8.0 * k / n_heads)


def _head_cols(l: int, d: int, h_l: int):
    q = slice(l * d, (l + 1) * d)
    k = slice(h_l + l * d, h_l + (l + 1) * d)
    v = slice(2 * h_l + l * d, 2 * h_l + (l + 1) * d)
    return q, k, v


def _scores(q, k, d, causal, slope):
    s = q.shape[0]
    S = (q @ k.T) / math.sqrt(d)
    i = np.arange(s)[:, None]
    j = np.arange(s)[None, :]
    if slope is not None:
        S = S - slope * (i - j)
    if causal:
        S = np.where(j <= i, S, -np.inf)
    return S


def _softmax_rows(S):
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    den = E.sum(axis=1, keepdims=True)
    return E / den, (mx + np.log(den))[:, 0]


def attn_core_fwd(qkv, *, batch, seq, n_local, head_dim, head0, n_heads, causal=True, alibi=False, dropout=None):
    """Per batch element and local head l (global head k = head0 + l + 1):
    ctx = softmax(q k^T / sqrt(d) + bias) v, lse = log-sum-exp of each score row.
    With dropout multipliers D [batch, n_local, seq, seq] (keep * scale, see
    oracle.dropout), the probabilities are multiplied by D before the value
    aggregation (the softmax and lse are those of the undropped scores).
    qkv [T, 3h_l] -> ctx [T, h_l], lse [batch, n_local, seq]."""
    h_l = n_local * head_dim
    ctx = np.zeros((batch * seq, h_l))
    lse = np.zeros((batch, n_local, seq))
    for bi in range(batch):
        rows = slice(bi * seq, (bi + 1) * seq)
        for l in range(n_local):
            cq, ck, cv = _head_cols(l, head_dim, h_l)
            slope = alibi_slope(head0 + l + 1, n_heads) if alibi else None
            S = _scores(qkv[rows, cq], qkv[rows, ck], head_dim, causal, slope)
            P, lse_h = _softmax_rows(S)
            if dropout is not None:
                P = P * dropout[bi, l]
            ctx[rows, cq] = P @ qkv[rows, cv]
            lse[bi, l] = lse_h
    return ctx, lse


def attn_core_bwd(qkv, dctx, *, batch, seq, n_local, head_dim, head0, n_heads, causal=True, alibi=False,
                  dropout=None):
    """Gradient of <ctx, dctx> with respect to qkv, per head:
    dv = P^T dc, dP = dc v^T, dS = P * (dP - rowsum(P * dP)),
    dq = dS k / sqrt(d), dk = dS^T q / sqrt(d).
    With dropout multipliers D: dv = (P D)^T dc and dP = D * (dc v^T)."""
    h_l = n_local * head_dim
    dqkv = np.zeros_like(qkv)
    for bi in range(batch):
        rows = slice(bi * seq, (bi + 1) * seq)
        for l in range(n_local):
            cq, ck, cv = _head_cols(l, head_dim, h_l)
            slope = alibi_slope(head0 + l + 1, n_heads) if alibi else None
            q, k, v = qkv[rows, cq], qkv[rows, ck], qkv[rows, cv]
            P, _ = _softmax_rows(_scores(q, k, head_dim, causal, slope))
            Dm = 1.0 if dropout is None else dropout[bi, l]
            dc = dctx[rows, cq]
            dP = (dc @ v.T) * Dm
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dqkv[rows, cq] = (dS @ k) / math.sqrt(head_dim)
            dqkv[rows, ck] = (dS.T @ q) / math.sqrt(head_dim)
            dqkv[rows, cv] = (P * Dm).T @ dc
    return dqkv


def _core_kw(Wqkv_r, batch, seq, n_heads, tp_size, tp_rank, causal, alibi, dropout=None):
    h_l = Wqkv_r.shape[1] // 3
    n_l = n_heads // tp_size
    return dict(batch=batch, seq=seq, n_local=n_l, head_dim=h_l // n_l, head0=tp_rank * n_l,
                n_heads=n_heads, causal=causal, alibi=alibi, dropout=dropout)


def attn_fwd(X, Wqkv_r, bqkv_r, Wo_r, *, batch, seq, n_heads, tp_size, tp_rank,
             causal=True, alibi=False, dropout=None):
    """Returns qkv_r [T, 3h_l], ctx_r [T, h_l], lse_r [batch, n_l, seq], O_r [T, h] (partial).
    dropout: optional multipliers [batch, n_l, seq, seq] on the attention probabilities."""
    kw = _core_kw(Wqkv_r, batch, seq, n_heads, tp_size, tp_rank, causal, alibi, dropout)
    qkv = X @ Wqkv_r + bqkv_r
    ctx, lse = attn_core_fwd(qkv, **kw)
    O_r = ctx @ Wo_r
    return qkv, ctx, lse, O_r


def attn_bwd(X, Wqkv_r, bqkv_r, Wo_r, dO, *, batch, seq, n_heads, tp_size, tp_rank,
             causal=True, alibi=False, dropout=None):
    """Gradients of <O_r + bo, dO>. Recomputes the forward from X.
    Returns dX_r (partial), dWqkv_r, dbqkv_r, dWo_r, dbo (replicated, once)."""
    kw = _core_kw(Wqkv_r, batch, seq, n_heads, tp_size, tp_rank, causal, alibi, dropout)
    qkv = X @ Wqkv_r + bqkv_r
    ctx, _ = attn_core_fwd(qkv, **kw)
    dC = dO @ Wo_r.T
    dqkv = attn_core_bwd(qkv, dC, **kw)
    dWo_r = ctx.T @ dO
    dbo = dO.sum(axis=0)
    dWqkv_r = X.T @ dqkv
    dbqkv_r = dqkv.sum(axis=0)
    dX_r = dqkv @ Wqkv_r.T
    return dX_r, dWqkv_r, dbqkv_r, dWo_r, dbo


# ---------------------------------------------------------------------------
# f / g (Megatron-LM deep dive, Fig. 4): g sums the ranks' partial outputs in
# the forward pass, f sums the ranks' partial input gradients in the backward
# pass. On one device both become a sum of the emulated ranks' partials; the
# replicated bias (b2 or bo) is added once after the sum.
# ---------------------------------------------------------------------------

def sum_partials(parts, bias=None):
    out = np.zeros_like(parts[0], dtype=np.float64)
    for p in parts:
        out = out + p
    if bias is not None:
        out = out + bias
    return out
