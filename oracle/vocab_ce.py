"""The oracle's vocabulary-parallel logits + cross-entropy (float64, NumPy).
Test infrastructure only.

The output layer multiplies the final hidden states by the (input-tied)
embedding table `W [V, h]`; with tensor parallelism the table is split along
the vocabulary, each rank computes the logits of its vocabulary slice only,
and the cross-entropy is fused with those parallel logits so that only
per-token aggregates (max, sum of exponentials, the target's logit) are
exchanged instead of the `[T, V]` logits (Megatron-LM deep dive, "vocabulary
parallelism and loss fusion" section; the training-recipe table pads the GPT-2
vocabulary of 50,257 to 51,200 so that it splits evenly over up to 8 ranks).

Per rank r of p, vocabulary slice [v0, v0 + V/p) with v0 = r V/p:
    logits_r = X W_r^T                               [T, V/p]
    m_r = max_j logits_r ; s_r = sum_j exp(logits_r - m_r)
    z_r = logits_r[t, label_t - v0] if label_t is in the slice, else 0
The exchange (emulated here by `ce_combine` over the ranks' aggregates):
    m = max_r m_r ; S = sum_r s_r exp(m_r - m) ; z = sum_r z_r
    lse = m + log S ; loss_t = lse - z   (= -log softmax(logits)[label_t])
Backward for the loss sum_t dloss_t * loss_t:
    dlogits_r = (exp(logits_r - lse) - onehot_r(label)) * dloss
    dX_r = dlogits_r W_r  [T, h]  (partial; f's all-reduce sums it)
    dW_r = dlogits_r^T X  [V/p, h]
Readings: the output projection is tied to the input embedding table and has
no bias; labels outside [0, V) are owned by no rank (their z is 0).
"""
from __future__ import annotations

import numpy as np


def vocab_shard(W, rank: int, tp: int):
    """Rows [rank V/p, (rank+1) V/p) of the [V, h] table."""
    V = W.shape[0]
    assert V % tp == 0
    n = V // tp
    return W[rank * n:(rank + 1) * n]


def logits_fwd(X, W_r):
    return X @ W_r.T


def ce_partial_stats(logits_r, labels, v0: int):
    """-> (m_r, s_r, z_r), each [T]."""
    m = logits_r.max(axis=1)
    s = np.exp(logits_r - m[:, None]).sum(axis=1)
    n = logits_r.shape[1]
    z = np.zeros(logits_r.shape[0])
    for t, lab in enumerate(labels):
        if v0 <= lab < v0 + n:
            z[t] = logits_r[t, lab - v0]
    return m, s, z


def ce_combine(stats):
    """stats: list over ranks of (m_r, s_r, z_r) -> (loss [T], lse [T])."""
    m = np.max(np.stack([st[0] for st in stats]), axis=0)
    S = np.zeros_like(m)
    z = np.zeros_like(m)
    for m_r, s_r, z_r in stats:
        S = S + s_r * np.exp(m_r - m)
        z = z + z_r
    lse = m + np.log(S)
    return lse - z, lse


def ce_bwd(X, W_r, labels, v0: int, lse, dloss):
    """-> dlogits_r [T, V/p], dX_r [T, h], dW_r [V/p, h]."""
    logits = X @ W_r.T
    d = np.exp(logits - lse[:, None])
    n = W_r.shape[0]
    for t, lab in enumerate(labels):
        if v0 <= lab < v0 + n:
            d[t, lab - v0] -= 1.0
    d = d * dloss[:, None]
    return d, d @ W_r, d.T @ X
