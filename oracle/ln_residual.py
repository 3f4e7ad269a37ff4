"""The oracle's residual add + LayerNorm (float64, NumPy). Test infrastructure only.

Where it sits in the layer: each tensor-parallel block (attention, MLP) ends in
a partial output per rank; g sums them before dropout and the residual add
(Megatron-LM deep dive, Fig. 4), and the layer's residual connections and
layer normalizations wrap the two blocks (same page, Fig. 2; the rearranged
order of Fig. 7 normalizes the input of each block). The Megatron-DeepSpeed
blog (section 4.3) fuses LayerNorm with the residual add into one kernel and
prints only its signature, so the arithmetic below is written from the
definition of layer normalization:

    r     = resid_in + sum_k parts[k] + bias        (the new residual stream)
    mu    = mean_j r[t, j]
    var   = mean_j (r[t, j] - mu)^2                 (biased: divide by h)
    rstd  = 1 / sqrt(var + eps)
    y     = (r - mu) * rstd * gamma + beta          (the next block's input)

Readings where the pages are silent: eps is the caller's argument (the pages
give no value; 1e-5 in the tests); the variance is the biased one. Dropout
on the block output (before the residual add; identical on every rank) is
optional: with multipliers R = keep * scale (oracle.dropout),
    r = resid_in + R * (sum_k parts[k] + bias),
and the block output, every part and the bias then receive dr * R.

Backward, for the loss <y, dy> + <r, dr_in> (dr_in: the gradient reaching r
along the residual stream from later in the network):

    xhat  = (r - mu) * rstd
    g     = dy * gamma
    dr    = dr_in + rstd * (g - mean_j g - xhat * mean_j (g * xhat))
    dgamma = sum_t dy * xhat ;  dbeta = sum_t dy ;  dbias = sum_t dr

dr is the gradient of resid_in, of every part and of the block output.
"""
from __future__ import annotations

import numpy as np


def ln_residual_fwd(resid_in, parts, bias, gamma, beta, eps, dropout=None):
    """-> r [T,h], y [T,h], mu [T], rstd [T]. `parts` is a list of [T,h]
    arrays (one per emulated rank); bias may be None; dropout: optional
    multipliers [T,h] on the block output (sum of parts + bias)."""
    blk = np.zeros_like(np.asarray(resid_in, dtype=np.float64))
    for p in parts:
        blk = blk + p
    if bias is not None:
        blk = blk + bias
    if dropout is not None:
        blk = blk * dropout
    r = np.array(resid_in, dtype=np.float64) + blk
    mu = r.mean(axis=1)
    cen = r - mu[:, None]
    var = (cen * cen).mean(axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    y = cen * rstd[:, None] * gamma + beta
    return r, y, mu, rstd


def ln_residual_bwd(r, gamma, eps, dy, dr_in=None):
    """Gradients of <y, dy> + <r, dr_in> with y = LayerNorm(r). The statistics
    are recomputed from r. -> dr [T,h], dgamma [h], dbeta [h], dbias [h]."""
    r = np.asarray(r, dtype=np.float64)
    mu = r.mean(axis=1)
    cen = r - mu[:, None]
    rstd = 1.0 / np.sqrt((cen * cen).mean(axis=1) + eps)
    xhat = cen * rstd[:, None]
    g = dy * gamma
    a = g.mean(axis=1)
    b = (g * xhat).mean(axis=1)
    dr = rstd[:, None] * (g - a[:, None] - xhat * b[:, None])
    if dr_in is not None:
        dr = dr + dr_in
    dgamma = (dy * xhat).sum(axis=0)
    dbeta = dy.sum(axis=0)
    dbias = dr.sum(axis=0)
    return dr, dgamma, dbeta, dbias


def ln_residual_bwd_dropout(r, gamma, eps, dy, dr_in, dropout):
    """With residual dropout multipliers R: -> dr (gradient of resid_in),
    d_block = dr * R (gradient of the block output, every part and the bias),
    dgamma, dbeta, dbias = sum_t d_block."""
    dr, dgamma, dbeta, _ = ln_residual_bwd(r, gamma, eps, dy, dr_in)
    d_block = dr * dropout
    return dr, d_block, dgamma, dbeta, d_block.sum(axis=0)
