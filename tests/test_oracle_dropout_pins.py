"""Pins of the oracle's counter-based generator and attention dropout to
things other than itself: numpy's own Philox4x64-10 bit generator, torch
float64 autograd of attention with the same multipliers, central finite
differences, binomial bounds on the kept fraction, and the p = 0 reduction to
attention without dropout. CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_philox_matches_numpy_bit_generator():
    # numpy's Philox advances its 256-bit counter before each block of four
    # 64-bit outputs, so its first block is the function at counter + 1
    rng = np.random.default_rng(0)
    for _ in range(25):
        key = rng.integers(0, 2 ** 63, size=2, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=2, dtype=np.uint64)
        ctr = rng.integers(0, 2 ** 63, size=4, dtype=np.uint64)
        ctr[0] = ctr[0] & np.uint64(0x7FFFFFFFFFFFFFF0)  # no carry out of word 0 in the next few blocks
        bg = np.random.Philox(key=key, counter=ctr)
        want = bg.random_raw(12).reshape(3, 4)
        for blk in range(3):
            got = oracle.philox4x64_10(ctr[0] + np.uint64(blk + 1), ctr[1], ctr[2], ctr[3], key[0], key[1])
            np.testing.assert_array_equal(np.array([int(w) for w in got], dtype=np.uint64), want[blk])


def test_philox_vectorised_equals_scalar_calls():
    c0 = np.arange(7, dtype=np.uint64)[:, None]
    c1 = np.arange(5, dtype=np.uint64)[None, :]
    words = oracle.philox4x64_10(c0, c1, np.uint64(3), np.uint64(1), 11, 12)
    for a in range(7):
        for b in range(5):
            one = oracle.philox4x64_10(np.uint64(a), np.uint64(b), np.uint64(3), np.uint64(1), 11, 12)
            assert [int(w[a, b]) for w in words] == [int(w) for w in one]


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_kept_fraction_within_binomial_bounds(p):
    D = oracle.attention_multipliers(batch=1, seq=200, n_local=3, head0=5, p=p, seed=7, offset=1)
    n = D.size
    kept = (D > 0).mean()
    want = 1.0 - oracle.keep_threshold(p) / 65536.0
    assert abs(kept - want) < 6 * math.sqrt(want * (1 - want) / n)
    np.testing.assert_allclose(D[D > 0], oracle.keep_scale(p))
    assert abs(D.mean() - 1.0) < 6 * math.sqrt((oracle.keep_scale(p) - 1.0) / n)


def test_masks_depend_on_head_seed_offset_not_on_rank_of_the_call():
    kw = dict(batch=2, seq=70, p=0.3)
    a = oracle.attention_multipliers(n_local=4, head0=0, seed=1, offset=2, **kw)
    # the same global heads seen by another rank layout: rank 1 of 2 owns heads 2, 3
    b = oracle.attention_multipliers(n_local=2, head0=2, seed=1, offset=2, **kw)
    np.testing.assert_array_equal(a[:, 2:], b)
    assert not np.array_equal(a[:, 0], a[:, 1])  # heads independent
    assert not np.array_equal(a[0], a[1])        # batch elements independent
    c = oracle.attention_multipliers(n_local=4, head0=0, seed=1, offset=3, **kw)
    d = oracle.attention_multipliers(n_local=4, head0=0, seed=9, offset=2, **kw)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    z = oracle.attention_multipliers(n_local=4, head0=0, seed=1, offset=2, batch=2, seq=70, p=0.0)
    np.testing.assert_array_equal(z, 1.0)


def _layer(T_b, s, h, nh, tp, seed):
    g = np.random.default_rng(seed)
    X = g.normal(size=(T_b * s, h))
    Wqkv = g.normal(scale=0.3, size=(h, 3 * h // tp))
    bqkv = g.normal(scale=0.1, size=3 * h // tp)
    Wo = g.normal(scale=0.3, size=(h // tp, h))
    dO = g.normal(size=(T_b * s, h))
    return X, Wqkv, bqkv, Wo, dO


@pytest.mark.parametrize("alibi", [False, True])
def test_dropout_attention_matches_torch_autograd(alibi):
    b, s, h, nh, tp, rank = 2, 9, 16, 4, 2, 1
    X, Wqkv, bqkv, Wo, dO = _layer(b, s, h, nh, tp, 3)
    n_l, d = nh // tp, h // nh
    D = oracle.attention_multipliers(batch=b, seq=s, n_local=n_l, head0=rank * n_l, p=0.4, seed=5, offset=0)
    kw = dict(batch=b, seq=s, n_heads=nh, tp_size=tp, tp_rank=rank, alibi=alibi, dropout=D)
    _, ctx, lse, O = oracle.attn_fwd(X, Wqkv, bqkv, Wo, **kw)
    dX, dWqkv, dbqkv, dWo, _ = oracle.attn_bwd(X, Wqkv, bqkv, Wo, dO, **kw)
    # torch: the same layer from library routines (softmax, matmul, autograd)
    Xt, Wt, bt, Wot = (torch.tensor(a, requires_grad=True) for a in (X, Wqkv, bqkv, Wo))
    hl = h // tp
    qkv = Xt @ Wt + bt
    i = torch.arange(s)[:, None]
    j = torch.arange(s)[None, :]
    outs = []
    for bi in range(b):
        heads = []
        for l in range(n_l):
            q = qkv[bi * s:(bi + 1) * s, l * d:(l + 1) * d]
            k = qkv[bi * s:(bi + 1) * s, hl + l * d:hl + (l + 1) * d]
            v = qkv[bi * s:(bi + 1) * s, 2 * hl + l * d:2 * hl + (l + 1) * d]
            S = q @ k.T / math.sqrt(d)
            if alibi:
                S = S - 2.0 ** (-8.0 * (rank * n_l + l + 1) / nh) * (i - j).double()
            S = S.masked_fill(j > i, float("-inf"))
            P = torch.softmax(S, dim=-1) * torch.tensor(D[bi, l])
            heads.append(P @ v)
        outs.append(torch.cat(heads, dim=1))
    ctx_t = torch.cat(outs, dim=0)
    O_t = ctx_t @ Wot
    np.testing.assert_allclose(ctx, ctx_t.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O, O_t.detach().numpy(), rtol=1e-12, atol=1e-12)
    (O_t * torch.tensor(dO)).sum().backward()
    for got, ref in ((dX, Xt.grad), (dWqkv, Wt.grad), (dbqkv, bt.grad), (dWo, Wot.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-11)


def test_dropout_attention_finite_differences():
    b, s, h, nh, tp = 1, 6, 8, 2, 1
    X, Wqkv, bqkv, Wo, dO = _layer(b, s, h, nh, tp, 8)
    D = oracle.attention_multipliers(batch=b, seq=s, n_local=nh, head0=0, p=0.5, seed=2, offset=4)
    kw = dict(batch=b, seq=s, n_heads=nh, tp_size=tp, tp_rank=0, dropout=D)
    _, dWqkv, _, _, _ = oracle.attn_bwd(X, Wqkv, bqkv, Wo, dO, **kw)
    e = 1e-6
    fd = np.zeros_like(Wqkv)
    for idx in np.ndindex(Wqkv.shape):
        Wqkv[idx] += e
        hi = (oracle.attn_fwd(X, Wqkv, bqkv, Wo, **kw)[3] * dO).sum()
        Wqkv[idx] -= 2 * e
        lo = (oracle.attn_fwd(X, Wqkv, bqkv, Wo, **kw)[3] * dO).sum()
        Wqkv[idx] += e
        fd[idx] = (hi - lo) / (2 * e)
    np.testing.assert_allclose(dWqkv, fd, rtol=1e-6, atol=1e-7)


def test_p_zero_is_attention_without_dropout():
    b, s, h, nh, tp = 2, 11, 16, 4, 2
    X, Wqkv, bqkv, Wo, dO = _layer(b, s, h, nh, tp, 4)
    D = oracle.attention_multipliers(batch=b, seq=s, n_local=2, head0=2, p=0.0, seed=1, offset=1)
    kw = dict(batch=b, seq=s, n_heads=nh, tp_size=tp, tp_rank=1)
    a = oracle.attn_fwd(X, Wqkv, bqkv, Wo, **kw) + oracle.attn_bwd(X, Wqkv, bqkv, Wo, dO, **kw)
    c = oracle.attn_fwd(X, Wqkv, bqkv, Wo, dropout=D, **kw) + oracle.attn_bwd(X, Wqkv, bqkv, Wo, dO, dropout=D, **kw)
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


def test_documented_element_mapping():
    # element (b, k, i, j): counter (i, j // 32, (b << 32) | k, ((j % 32) >> 2) & 1), key (seed, offset),
    # 16-bit lane q = 4 ((j % 32) >> 3) + j % 4; kept iff that lane >= thr
    p, seed, offset = 0.37, 123, 45
    D = oracle.attention_multipliers(batch=2, seq=100, n_local=3, head0=6, p=p, seed=seed, offset=offset)
    thr = oracle.keep_threshold(p)
    rng = np.random.default_rng(3)
    for _ in range(200):
        b, l, i, j = (int(rng.integers(0, n)) for n in (2, 3, 100, 100))
        words = oracle.philox4x64_10(np.uint64(i), np.uint64(j // 32), np.uint64((b << 32) | (6 + l)),
                                     np.uint64(((j % 32) >> 2) & 1), seed, offset)
        q = 4 * ((j % 32) >> 3) + (j % 4)
        u = (int(words[q >> 2]) >> (16 * (q & 3))) & 0xFFFF
        assert (D[b, l, i, j] > 0) == (u >= thr)


# ----------------------------------------------------------------------------
# residual dropout (before the residual add; identical on every rank)
# ----------------------------------------------------------------------------

def test_residual_mask_mapping_and_statistics():
    T, h, p, seed, offset = 37, 100, 0.25, 77, 3
    R = oracle.residual_multipliers(tokens=T, hidden=h, p=p, seed=seed, offset=offset)
    thr = oracle.keep_threshold(p)
    for t, j in ((0, 0), (5, 15), (5, 16), (36, 99), (17, 42)):
        w = oracle.philox4x64_10(np.uint64(t), np.uint64(j // 16), np.uint64(0), np.uint64(2), seed, offset)
        u = (int(w[(j % 16) >> 2]) >> (16 * (j % 4))) & 0xFFFF
        assert (R[t, j] > 0) == (u >= thr)
    kept = (R > 0).mean()
    assert abs(kept - (1 - thr / 65536)) < 6 * math.sqrt(p * (1 - p) / R.size)
    # the residual counter space (last word 2) never meets the attention one (last word 0 or 1)
    A = oracle.attention_multipliers(batch=1, seq=T, n_local=1, head0=0, p=p, seed=seed, offset=offset)
    assert not np.array_equal((A[0, 0, :, :T] > 0), (R[:, :T] > 0))


def test_residual_dropout_ln_matches_torch_autograd():
    g = np.random.default_rng(6)
    T, h = 7, 40
    resid, parts = g.normal(size=(T, h)), [g.normal(size=(T, h)) for _ in range(2)]
    bias, gamma, beta = g.normal(size=h), 1 + 0.1 * g.normal(size=h), 0.1 * g.normal(size=h)
    dy, dr_in = g.normal(size=(T, h)), g.normal(size=(T, h))
    R = oracle.residual_multipliers(tokens=T, hidden=h, p=0.3, seed=1, offset=2)
    r, y, _, _ = oracle.ln_residual_fwd(resid, parts, bias, gamma, beta, 1e-5, dropout=R)
    dr, d_block, dg, db, dbias = oracle.ln_residual_bwd_dropout(r, gamma, 1e-5, dy, dr_in, R)
    tr, tparts = torch.tensor(resid, requires_grad=True), [torch.tensor(q, requires_grad=True) for q in parts]
    tb, tg, tbe = (torch.tensor(a, requires_grad=True) for a in (bias, gamma, beta))
    rt = tr + (sum(tparts) + tb) * torch.tensor(R)
    yt = torch.nn.functional.layer_norm(rt, (h,), tg, tbe, 1e-5)
    np.testing.assert_allclose(r, rt.detach().numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    ((yt * torch.tensor(dy)).sum() + (rt * torch.tensor(dr_in)).sum()).backward()
    tol = dict(rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dr, tr.grad.numpy(), **tol)
    for q in tparts:
        np.testing.assert_allclose(d_block, q.grad.numpy(), **tol)
    np.testing.assert_allclose(dbias, tb.grad.numpy(), **tol)
    np.testing.assert_allclose(dg, tg.grad.numpy(), **tol)
    np.testing.assert_allclose(db, tbe.grad.numpy(), **tol)
    # p = 0 is the step without dropout
    R0 = oracle.residual_multipliers(tokens=T, hidden=h, p=0.0, seed=1, offset=2)
    a = oracle.ln_residual_fwd(resid, parts, bias, gamma, beta, 1e-5, dropout=R0)
    b = oracle.ln_residual_fwd(resid, parts, bias, gamma, beta, 1e-5)
    for x, z in zip(a, b):
        np.testing.assert_array_equal(x, z)
