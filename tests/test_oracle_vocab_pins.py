"""Pins of the oracle's vocabulary-parallel logits + cross-entropy to things
other than itself: torch float64 cross_entropy and autograd on the UNSHARDED
output layer, central finite differences, and closed forms. CPU only."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def draw(T, h, V, seed=0, w_std=0.5):
    g = np.random.default_rng(seed)
    X = g.normal(size=(T, h))
    W = g.normal(scale=w_std, size=(V, h))
    labels = g.integers(0, V, size=T)
    dloss = g.normal(size=T)
    return X, W, labels, dloss


def sharded(X, W, labels, dloss, tp):
    """The oracle's per-rank path, combined over all ranks."""
    n = W.shape[0] // tp
    stats = [oracle.ce_partial_stats(oracle.logits_fwd(X, oracle.vocab_shard(W, r, tp)), labels, r * n)
             for r in range(tp)]
    loss, lse = oracle.ce_combine(stats)
    outs = [oracle.ce_bwd(X, oracle.vocab_shard(W, r, tp), labels, r * n, lse, dloss) for r in range(tp)]
    dX = sum(o[1] for o in outs)
    dW = np.concatenate([o[2] for o in outs], axis=0)
    return loss, lse, dX, dW


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_sharded_loss_and_grads_match_torch_unsharded(tp):
    X, W, labels, dloss = draw(37, 24, 64, seed=tp)
    loss, lse, dX, dW = sharded(X, W, labels, dloss, tp)
    Xt = torch.tensor(X, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    logits = Xt @ Wt.T
    ref = F.cross_entropy(logits, torch.tensor(labels), reduction="none")
    np.testing.assert_allclose(loss, ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=1).detach().numpy(), rtol=1e-13, atol=1e-13)
    (ref * torch.tensor(dloss)).sum().backward()
    np.testing.assert_allclose(dX, Xt.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_finite_differences():
    X, W, labels, dloss = draw(4, 5, 12, seed=9)

    def L(X_, W_):
        loss, _, _, _ = sharded(X_, W_, labels, dloss, 3)
        return float((loss * dloss).sum())

    _, _, dX, dW = sharded(X, W, labels, dloss, 3)
    e = 1e-6
    for arr, want in ((X, dX), (W, dW)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            arr[idx] += e
            hi = L(X, W)
            arr[idx] -= 2 * e
            lo = L(X, W)
            arr[idx] += e
            fd[idx] = (hi - lo) / (2 * e)
        np.testing.assert_allclose(want, fd, rtol=1e-7, atol=1e-8)


def test_closed_forms():
    T, h, V, tp = 9, 6, 40, 4
    X, W, labels, dloss = draw(T, h, V, seed=2)
    # all-zero table: uniform softmax, loss = log V, dlogits = (1/V - onehot) dloss
    Z = np.zeros((V, h))
    loss, lse, _, _ = sharded(X, Z, labels, dloss, tp)
    np.testing.assert_allclose(loss, math.log(V), rtol=1e-15)
    np.testing.assert_allclose(lse, math.log(V), rtol=1e-15)
    n = V // tp
    for r in range(tp):
        d, _, _ = oracle.ce_bwd(X, oracle.vocab_shard(Z, r, tp), labels, r * n, lse, dloss)
        want = np.full((T, n), 1.0 / V)
        for t, lab in enumerate(labels):
            if r * n <= lab < (r + 1) * n:
                want[t, lab - r * n] -= 1.0
        np.testing.assert_allclose(d, want * dloss[:, None], rtol=1e-14, atol=1e-15)
    # labels on slice boundaries are owned by exactly one rank
    lab_b = np.array([0, n - 1, n, 2 * n - 1, V - 1, n, 0, 3 * n, 2 * n])
    stats = [oracle.ce_partial_stats(oracle.logits_fwd(X, oracle.vocab_shard(W, r, tp)), lab_b, r * n)
             for r in range(tp)]
    logits = X @ W.T
    _, lse = oracle.ce_combine(stats)
    loss, _ = oracle.ce_combine(stats)
    np.testing.assert_allclose(loss, lse - logits[np.arange(T), lab_b], rtol=1e-13)
    # a label outside [0, V) is owned by no rank: its loss is the log-sum-exp
    stats = [oracle.ce_partial_stats(oracle.logits_fwd(X, oracle.vocab_shard(W, r, tp)), np.full(T, V), r * n)
             for r in range(tp)]
    loss, lse = oracle.ce_combine(stats)
    np.testing.assert_array_equal(loss, lse)
    # the softmax gradient sums to zero over the full vocabulary (dloss = 1)
    d = np.concatenate([oracle.ce_bwd(X, oracle.vocab_shard(W, r, tp), labels, r * n, lse, np.ones(T))[0]
                        for r in range(tp)], axis=1)
    np.testing.assert_allclose(d.sum(axis=1), 0.0, atol=1e-14)


def test_combine_is_order_and_shift_stable():
    # large logits: the combine subtracts the global max, so shifting every logit
    # of a token by a constant shifts lse by that constant and leaves the loss
    X, W, labels, dloss = draw(6, 4, 16, seed=4, w_std=30.0)
    tp, n = 4, 4
    base = [oracle.ce_partial_stats(oracle.logits_fwd(X, oracle.vocab_shard(W, r, tp)), labels, r * n)
            for r in range(tp)]
    loss0, lse0 = oracle.ce_combine(base)
    c = np.linspace(-500.0, 800.0, X.shape[0])
    shifted = [(m + c, s, np.where(z != 0, z + c, 0.0)) for (m, s, z) in base]
    loss1, lse1 = oracle.ce_combine(shifted)
    np.testing.assert_allclose(lse1, lse0 + c, rtol=1e-13)
    np.testing.assert_allclose(loss1, loss0, rtol=1e-9, atol=1e-9)
    assert np.all(np.isfinite(loss0)) and np.all(loss0 >= 0)
    loss2, _ = oracle.ce_combine(base[::-1])
    np.testing.assert_allclose(loss2, loss0, rtol=1e-13)
