"""Pins of the fp64 oracle to things other than itself: torch float64 library
routines on the unsharded layer, central finite differences, closed forms and
the parameter counts the pages print. CPU only."""
import csv
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# torch float64 reference of the UNSHARDED layer (library routines + autograd)
# ----------------------------------------------------------------------------

def torch_mlp(X, A, b1, B, b2):
    return F.gelu(X @ A + b1, approximate="tanh") @ B + b2


def torch_attention(X, Wqkv, bqkv, Wo, bo, *, batch, seq, n_heads, alibi):
    T, h = X.shape
    d = h // n_heads
    qkv = X @ Wqkv + bqkv
    q, k, v = qkv[:, :h], qkv[:, h:2 * h], qkv[:, 2 * h:]

    def heads(t):
        return t.reshape(batch, seq, n_heads, d).permute(0, 2, 1, 3).contiguous()

    i = torch.arange(seq)[:, None]
    j = torch.arange(seq)[None, :]
    mask = torch.zeros(n_heads, seq, seq, dtype=X.dtype)
    if alibi:
        slopes = torch.tensor([2.0 ** (-8.0 * (hh + 1) / n_heads) for hh in range(n_heads)], dtype=X.dtype)
        mask = mask - slopes[:, None, None] * (i - j).to(X.dtype)
    mask = mask.masked_fill(j > i, float("-inf"))
    ctx = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), attn_mask=mask)
    ctx = ctx.permute(0, 2, 1, 3).reshape(T, h)
    scores = heads(q) @ heads(k).transpose(-1, -2) / math.sqrt(d) + mask
    lse = torch.logsumexp(scores, dim=-1)  # [batch, heads, seq]
    return ctx @ Wo + bo, ctx, lse


def tt(a):
    return torch.tensor(a, dtype=torch.float64, requires_grad=True)


# ----------------------------------------------------------------------------
# GeLU
# ----------------------------------------------------------------------------

def test_gelu_matches_torch_tanh_gelu():
    x = np.linspace(-12, 12, 20001)
    ref = F.gelu(torch.tensor(x), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu(x), ref, rtol=1e-14, atol=1e-15)


def test_gelu_grad_matches_autograd_and_fd():
    x = np.linspace(-8, 8, 4001)
    xt = torch.tensor(x, requires_grad=True)
    F.gelu(xt, approximate="tanh").sum().backward()
    np.testing.assert_allclose(oracle.gelu_grad(x), xt.grad.numpy(), rtol=1e-13, atol=1e-14)
    eps = 1e-6
    fd = (oracle.gelu(x + eps) - oracle.gelu(x - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.gelu_grad(x), fd, rtol=1e-7, atol=1e-8)


def test_gelu_closed_forms():
    assert oracle.gelu(np.array(0.0)) == 0.0
    assert oracle.gelu_grad(np.array(0.0)) == 0.5
    x = np.linspace(-6, 6, 101)
    # 0.5 x (1 + tanh u) - (-0.5 x (1 - tanh u)) = x for any odd u
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, atol=1e-14)
    assert abs(oracle.gelu(np.array(30.0)) - 30.0) < 1e-12
    assert abs(oracle.gelu(np.array(-30.0))) < 1e-12
    # a GeLU: within 1e-3 of the erf form everywhere
    erf_gelu = F.gelu(torch.tensor(x)).numpy()
    assert np.max(np.abs(oracle.gelu(x) - erf_gelu)) < 1e-3


# ----------------------------------------------------------------------------
# MLP block: sum over column/row shards equals the unsharded GeLU(XA+b1)B+b2
# ----------------------------------------------------------------------------

def _mlp_full(r, T=12, h=16, f=64, bias=0.3):
    X = r.standard_normal((T, h))
    A = r.standard_normal((h, f)) * 0.3
    b1 = r.standard_normal(f) * bias
    B = r.standard_normal((f, h)) * 0.3
    b2 = r.standard_normal(h) * bias
    dZ = r.standard_normal((T, h))
    return X, A, b1, B, b2, dZ


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_mlp_sum_over_shards_equals_unsharded(tp):
    X, A, b1, B, b2, _ = _mlp_full(rng(tp))
    parts = []
    for r in range(tp):
        _, _, Z_r = oracle.mlp_fwd(X, oracle.column_shard(A, r, tp), oracle.column_shard(b1, r, tp),
                                   oracle.row_shard(B, r, tp))
        parts.append(Z_r)
    Z = oracle.sum_partials(parts, b2)
    ref = torch_mlp(*(torch.tensor(a) for a in (X, A, b1, B, b2))).numpy()
    np.testing.assert_allclose(Z, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_mlp_bwd_matches_autograd(tp):
    X, A, b1, B, b2, dZ = _mlp_full(rng(10 + tp))
    Xt, At, b1t, Bt, b2t = (tt(a) for a in (X, A, b1, B, b2))
    (torch_mlp(Xt, At, b1t, Bt, b2t) * torch.tensor(dZ)).sum().backward()
    dX = []
    for r in range(tp):
        A_r, b1_r, B_r = oracle.column_shard(A, r, tp), oracle.column_shard(b1, r, tp), oracle.row_shard(B, r, tp)
        pre, y, _ = oracle.mlp_fwd(X, A_r, b1_r, B_r)
        dX_r, dA_r, db1_r, dB_r, db2 = oracle.mlp_bwd(X, A_r, B_r, pre, y, dZ)
        dX.append(dX_r)
        np.testing.assert_allclose(dA_r, oracle.column_shard(At.grad.numpy(), r, tp), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(db1_r, oracle.column_shard(b1t.grad.numpy(), r, tp), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dB_r, oracle.row_shard(Bt.grad.numpy(), r, tp), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(db2, b2t.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.sum_partials(dX), Xt.grad.numpy(), rtol=1e-12, atol=1e-12)


def _fd_check(f, arrays, grads, eps=1e-6, rtol=1e-7):
    """Central differences of scalar f over every entry of every array."""
    for a, g in zip(arrays, grads):
        num = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = a[idx]
            a[idx] = old + eps
            fp = f()
            a[idx] = old - eps
            fm = f()
            a[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        scale = max(1.0, np.abs(num).max())
        assert np.max(np.abs(num - g)) <= rtol * scale, (np.max(np.abs(num - g)), scale)


def test_mlp_bwd_finite_differences():
    r = rng(3)
    tp, rank = 2, 1
    X, A, b1, B, b2, dZ = _mlp_full(r, T=5, h=4, f=8, bias=0.5)
    A_r, b1_r, B_r = [np.array(a) for a in (oracle.column_shard(A, rank, tp), oracle.column_shard(b1, rank, tp),
                                            oracle.row_shard(B, rank, tp))]

    def loss():
        _, _, Z_r = oracle.mlp_fwd(X, A_r, b1_r, B_r)
        return float(np.sum((Z_r + b2) * dZ))

    pre, y, _ = oracle.mlp_fwd(X, A_r, b1_r, B_r)
    dX_r, dA_r, db1_r, dB_r, db2 = oracle.mlp_bwd(X, A_r, B_r, pre, y, dZ)
    _fd_check(loss, [X, A_r, b1_r, B_r, b2], [dX_r, dA_r, db1_r, dB_r, db2])


# ----------------------------------------------------------------------------
# Attention block: per-head split equals full multi-head attention
# ----------------------------------------------------------------------------

def _attn_full(r, batch=2, seq=7, n_heads=4, d=4, bias=0.3):
    h = n_heads * d
    T = batch * seq
    X = r.standard_normal((T, h))
    Wqkv = r.standard_normal((h, 3 * h)) * 0.5
    bqkv = r.standard_normal(3 * h) * bias
    Wo = r.standard_normal((h, h)) * 0.5
    bo = r.standard_normal(h) * bias
    dO = r.standard_normal((T, h))
    return X, Wqkv, bqkv, Wo, bo, dO


def _rank_attn(X, Wqkv, bqkv, Wo, r, tp, **kw):
    return (X, oracle.qkv_weight_shard(Wqkv, r, tp), oracle.qkv_bias_shard(bqkv, r, tp),
            oracle.row_shard(Wo, r, tp)), dict(tp_size=tp, tp_rank=r, **kw)


@pytest.mark.parametrize("tp,alibi", [(1, False), (2, False), (4, False), (2, True), (4, True)])
def test_attn_heads_concat_equals_torch_mha(tp, alibi):
    batch, seq, nh = 2, 9, 4
    X, Wqkv, bqkv, Wo, bo, _ = _attn_full(rng(20 + tp), batch=batch, seq=seq, n_heads=nh)
    O_ref, ctx_ref, lse_ref = torch_attention(*(torch.tensor(a) for a in (X, Wqkv, bqkv, Wo, bo)),
                                              batch=batch, seq=seq, n_heads=nh, alibi=alibi)
    parts, ctxs, lses = [], [], []
    for r in range(tp):
        args, kw = _rank_attn(X, Wqkv, bqkv, Wo, r, tp, batch=batch, seq=seq, n_heads=nh, alibi=alibi)
        qkv, ctx, lse, O_r = oracle.attn_fwd(*args, **kw)
        parts.append(O_r)
        ctxs.append(ctx)
        lses.append(lse)
    np.testing.assert_allclose(np.concatenate(ctxs, axis=1), ctx_ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(lses, axis=1), lse_ref.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.sum_partials(parts, bo), O_ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tp,alibi", [(1, False), (2, False), (2, True), (4, True)])
def test_attn_bwd_matches_autograd(tp, alibi):
    batch, seq, nh = 2, 6, 4
    X, Wqkv, bqkv, Wo, bo, dO = _attn_full(rng(30 + tp), batch=batch, seq=seq, n_heads=nh)
    ts = [tt(a) for a in (X, Wqkv, bqkv, Wo, bo)]
    O, _, _ = torch_attention(*ts, batch=batch, seq=seq, n_heads=nh, alibi=alibi)
    (O * torch.tensor(dO)).sum().backward()
    Xg, Wqkvg, bqkvg, Wog, bog = (t.grad.numpy() for t in ts)
    dX = []
    for r in range(tp):
        args, kw = _rank_attn(X, Wqkv, bqkv, Wo, r, tp, batch=batch, seq=seq, n_heads=nh, alibi=alibi)
        dX_r, dWqkv_r, dbqkv_r, dWo_r, dbo = oracle.attn_bwd(*args, dO, **kw)
        dX.append(dX_r)
        np.testing.assert_allclose(dWqkv_r, oracle.qkv_weight_shard(Wqkvg, r, tp), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dbqkv_r, oracle.qkv_bias_shard(bqkvg, r, tp), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dWo_r, oracle.row_shard(Wog, r, tp), rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(dbo, bog, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.sum_partials(dX), Xg, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("alibi", [False, True])
def test_attn_bwd_finite_differences(alibi):
    tp, rank, batch, seq, nh = 2, 1, 2, 4, 4
    X, Wqkv, bqkv, Wo, bo, dO = _attn_full(rng(40), batch=batch, seq=seq, n_heads=nh, d=2)
    args, kw = _rank_attn(X, Wqkv, bqkv, Wo, rank, tp, batch=batch, seq=seq, n_heads=nh, alibi=alibi)
    X_, W_, b_, Wo_ = [np.array(a) for a in args]

    def loss():
        *_, O_r = oracle.attn_fwd(X_, W_, b_, Wo_, **kw)
        return float(np.sum((O_r + bo) * dO))

    dX_r, dWqkv_r, dbqkv_r, dWo_r, dbo = oracle.attn_bwd(X_, W_, b_, Wo_, dO, **kw)
    _fd_check(loss, [X_, W_, b_, Wo_, bo], [dX_r, dWqkv_r, dbqkv_r, dWo_r, dbo])


def test_attn_closed_forms():
    """Row 0 attends only to itself; with zero queries the weights are uniform
    over the causal prefix; with ALiBi they are geometric, e^{-m (i-j)}."""
    batch, seq, nh, d = 1, 6, 2, 3
    h = nh * d
    r = rng(50)
    X = r.standard_normal((seq, h))
    Wqkv = r.standard_normal((h, 3 * h))
    Wqkv[:, :h] = 0.0  # W_q = 0 and b_q = 0 -> all scores 0 before ALiBi
    bqkv = np.concatenate([np.zeros(h), r.standard_normal(2 * h)])
    Wo = np.eye(h)
    kw = dict(batch=batch, seq=seq, n_heads=nh, tp_size=1, tp_rank=0)
    qkv, ctx, lse, _ = oracle.attn_fwd(X, Wqkv, bqkv, Wo, **kw)
    v = qkv[:, 2 * h:]
    np.testing.assert_allclose(ctx[0], v[0], rtol=0, atol=1e-15)
    cummean = np.cumsum(v, axis=0) / np.arange(1, seq + 1)[:, None]
    np.testing.assert_allclose(ctx, cummean, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, seq + 1)), rtol=1e-14, atol=1e-14)
    # ALiBi: head k (1-based) of nh=2 has slope 2^(-8k/2) -> 1/16, 1/256
    qkv, ctx, lse, _ = oracle.attn_fwd(X, Wqkv, bqkv, Wo, alibi=True, **kw)
    for k in (1, 2):
        m = 2.0 ** (-4.0 * k)
        cols = slice((k - 1) * d, k * d)
        for i in range(seq):
            w = np.exp(-m * (i - np.arange(i + 1)))
            np.testing.assert_allclose(ctx[i, cols], (w[:, None] * v[:i + 1, cols]).sum(0) / w.sum(),
                                       rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[0, k - 1, i], np.log(w.sum()), rtol=1e-13, atol=1e-13)


def test_zero_grad_out_gives_zero_grads():
    X, Wqkv, bqkv, Wo, bo, _ = _attn_full(rng(60))
    outs = oracle.attn_bwd(X, Wqkv, bqkv, Wo, np.zeros((X.shape[0], Wo.shape[1])),
                           batch=2, seq=7, n_heads=4, tp_size=1, tp_rank=0)
    assert all(np.all(o == 0) for o in outs)
    X, A, b1, B, b2, _ = _mlp_full(rng(61))
    pre, y, _ = oracle.mlp_fwd(X, A, b1, B)
    outs = oracle.mlp_bwd(X, A, B, pre, y, np.zeros((X.shape[0], B.shape[1])))
    assert all(np.all(o == 0) for o in outs)


def test_alibi_slopes_of_176b_shard():
    # 112 heads: slope of global head k is 2^(-k/14); rank 0 of 8 owns k = 1..14
    s = [oracle.alibi_slope(k, 112) for k in range(1, 15)]
    assert abs(s[0] - 2 ** (-1 / 14)) < 1e-15 and abs(s[-1] - 0.5) < 1e-15
    assert all(a > b for a, b in zip(s, s[1:]))
    assert abs(oracle.alibi_slope(112, 112) - 2 ** -8) < 1e-18


# ----------------------------------------------------------------------------
# Weight shapes vs the parameter counts the pages print
# ----------------------------------------------------------------------------

def _golden_rows():
    with open(os.path.join(HERE, "golden", "param_counts.csv")) as fh:
        rows = [ln for ln in fh if ln.strip() and not ln.startswith("#")]
    return list(csv.reader(rows))


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: f"{r[0]}-h{r[1]}")
@pytest.mark.parametrize("tp", [1, 8])
def test_param_counts_match_pages(row, tp):
    src, hidden, heads, layers, head_dim, seq, params, unit = row
    hidden, heads, layers, seq = int(hidden), int(heads), int(layers), int(seq)
    params, unit = float(params), float(unit)
    if head_dim:
        assert hidden == heads * int(head_dim)
    shapes = oracle.layer_weight_shapes(hidden, 4 * hidden, tp)
    replicated = {"bo", "b2"}
    per_layer = sum(math.prod(s) * (1 if n in replicated else tp) for n, s in shapes.items())
    per_layer += 4 * hidden  # two LayerNorms (gain + bias) outside the tensor-parallel region
    total = layers * per_layer + 51200 * hidden + seq * hidden  # token + position embeddings
    # the printed figure is rounded or truncated to its last digit
    assert abs(total - params) < unit, (total, params)


def test_sum_partials_adds_bias_once():
    parts = [np.full((3, 4), float(i + 1)) for i in range(4)]
    out = oracle.sum_partials(parts, np.arange(4.0))
    np.testing.assert_array_equal(out, np.full((3, 4), 10.0) + np.arange(4.0))
