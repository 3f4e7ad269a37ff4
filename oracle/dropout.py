"""The oracle's counter-based random numbers and attention-probability
dropout masks (NumPy). Test infrastructure only.

Dropout in the layer (Megatron-LM deep dive: the training-setup table uses
dropout 0.1; its note on random numbers says that dropout inside the
model-parallel region draws independent random numbers on each rank, while
dropout outside it, before the residual add, must be identical on the ranks
of one model replica). Attention-probability dropout is inside the region;
its random numbers come from a counter-based generator, so a kernel can draw
any element's number on its own, and the forward and backward passes agree.

Generator: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC 2011): a 256-bit counter (four 64-bit words)
and a 128-bit key; ten rounds, each multiplying words 0 and 2 by fixed
constants into 128-bit products, then
    (x0, x1, x2, x3) <- (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)),
with the key advanced by two Weyl constants between rounds.

Residual mask (dropout on a block's output before the residual add, outside
the model-parallel region, so identical on every rank): for token t and
column j the counter is (t, j // 16, 0, 2) -- no rank or head in it, and the
last word 2 keeps it apart from every attention counter -- with the same key;
the uniform is 16-bit lane j % 16, kept and scaled as below.

Attention mask (readings, the pages fix none of this): for batch b, global
head k (0-based), query i and key j, the counter is
    (i, j // 32, (b << 32) | k, g)   with g = ((j % 32) >> 2) & 1,
the key is (seed, offset), and the element's uniform is 16-bit lane
q = 4 ((j % 32) >> 3) + (j % 4) of the 256-bit output (word q >> 2, bits
16 (q & 3) ..). The element is kept iff that uniform >= thr = round(65536 p);
kept probabilities are scaled by 65536 / (65536 - thr), so each element's
expected multiplier is exactly 1. The global head index in the counter gives
every rank (which owns different heads) independent numbers from one seed.
"""
from __future__ import annotations

import numpy as np

M0, M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
W0, W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.uint64, b):
    """128-bit product of a (scalar) and b (array) as (hi, lo) 64-bit words."""
    a_lo, a_hi = a & _LO, a >> _S32
    b_lo, b_hi = b & _LO, b >> _S32
    ll = a_lo * b_lo
    c1 = a_hi * b_lo
    c2 = a_lo * b_hi
    mid = (ll >> _S32) + (c1 & _LO) + (c2 & _LO)
    hi = a_hi * b_hi + (c1 >> _S32) + (c2 >> _S32) + (mid >> _S32)
    return hi, a * b


def philox4x64_10(c0, c1, c2, c3, k0, k1):
    """Philox4x64-10 on arrays of counters (broadcast together) -> 4 arrays."""
    with np.errstate(over="ignore"):
        x = [np.asarray(c, dtype=np.uint64) for c in np.broadcast_arrays(c0, c1, c2, c3)]
        k0, k1 = np.uint64(k0), np.uint64(k1)
        for r in range(10):
            if r:
                k0 = k0 + W0
                k1 = k1 + W1
            hi0, lo0 = _mulhilo(M0, x[0])
            hi1, lo1 = _mulhilo(M1, x[2])
            x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
    return x


def keep_threshold(p: float) -> int:
    thr = int(np.floor(p * 65536.0 + 0.5))
    if not 0 <= thr < 65536:
        # every 16-bit uniform would be dropped and the scale 65536 / (65536 - thr)
        # would not exist: such p cannot be realized in steps of 2^-16
        raise ValueError(f"drop probability {p} rounds to a keep threshold of {thr} (needs 0 <= thr < 65536)")
    return thr


def keep_scale(p: float) -> float:
    thr = keep_threshold(p)
    return 65536.0 / (65536.0 - thr)


def attention_multipliers(*, batch, seq, n_local, head0, p, seed, offset):
    """Dropout multipliers D[b, l, i, j] = keep * scale for the rank's local
    heads l (global head head0 + l), every query i and key j < seq."""
    thr = keep_threshold(p)
    scale = keep_scale(p)
    nkb = (seq + 31) // 32
    i = np.arange(seq, dtype=np.uint64)[:, None, None]
    kb = np.arange(nkb, dtype=np.uint64)[None, :, None]
    g = np.arange(2, dtype=np.uint64)[None, None, :]
    D = np.zeros((batch, n_local, seq, seq))
    for b in range(batch):
        for l in range(n_local):
            hk = np.uint64((b << 32) | (head0 + l))
            words = philox4x64_10(i, kb, hk, g, seed, offset)  # each [seq, nkb, 2]
            for q in range(16):
                u = (words[q >> 2] >> np.uint64(16 * (q & 3))) & np.uint64(0xFFFF)
                keep = (u >= np.uint64(thr)).astype(np.float64) * scale  # [seq, nkb, 2]
                for gg in range(2):
                    j = 32 * np.arange(nkb) + 8 * (q >> 2) + 4 * gg + (q & 3)
                    ok = j < seq
                    D[b, l][:, j[ok]] = keep[:, ok, gg]
    return D


def residual_multipliers(*, tokens, hidden, p, seed, offset):
    """Dropout multipliers R[t, j] = keep * scale on a block output before the
    residual add (the same on every rank)."""
    thr = keep_threshold(p)
    scale = keep_scale(p)
    t = np.arange(tokens, dtype=np.uint64)[:, None]
    c = np.arange((hidden + 15) // 16, dtype=np.uint64)[None, :]
    words = philox4x64_10(t, c, np.uint64(0), np.uint64(2), seed, offset)  # each [T, ceil(h/16)]
    R = np.zeros((tokens, (hidden + 15) // 16 * 16))
    for q in range(16):
        u = (words[q >> 2] >> np.uint64(16 * (q & 3))) & np.uint64(0xFFFF)
        R[:, q::16] = (u >= np.uint64(thr)).astype(np.float64) * scale
    return R[:, :hidden]
