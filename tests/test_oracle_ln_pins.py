"""Pins of the oracle's residual add + LayerNorm to things other than itself:
torch float64 `layer_norm` and autograd (library routines), central finite
differences, and closed forms of layer normalization. CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

EPS = 1e-5


def draw(T, h, n_parts, seed=0, bias=True):
    g = np.random.default_rng(seed)
    d = {
        "resid_in": g.normal(size=(T, h)),
        "parts": [g.normal(size=(T, h)) for _ in range(n_parts)],
        "bias": g.normal(scale=0.5, size=h) if bias else None,
        "gamma": 1.0 + 0.1 * g.normal(size=h),
        "beta": 0.1 * g.normal(size=h),
        "dy": g.normal(size=(T, h)),
        "dr_in": g.normal(size=(T, h)),
    }
    return d


def tt(a):
    return torch.tensor(a, dtype=torch.float64, requires_grad=True)


def torch_ln_residual(d, eps=EPS):
    """The same layer from torch library routines: returns r, y and the
    leaf tensors, for autograd."""
    leaves = {"resid_in": tt(d["resid_in"]), "gamma": tt(d["gamma"]), "beta": tt(d["beta"]),
              "parts": [tt(p) for p in d["parts"]]}
    r = leaves["resid_in"] + sum(leaves["parts"])
    if d["bias"] is not None:
        leaves["bias"] = tt(d["bias"])
        r = r + leaves["bias"]
    y = F.layer_norm(r, (r.shape[1],), leaves["gamma"], leaves["beta"], eps)
    return r, y, leaves


@pytest.mark.parametrize("n_parts,bias", [(1, False), (2, True), (4, True)])
def test_ln_fwd_matches_torch_layer_norm(n_parts, bias):
    d = draw(6, 40, n_parts, seed=n_parts, bias=bias)
    r, y, mu, rstd = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    rt, yt, _ = torch_ln_residual(d)
    np.testing.assert_allclose(r, rt.detach().numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    var_t = torch.var(rt.detach(), dim=1, unbiased=False).numpy()
    np.testing.assert_allclose(mu, rt.detach().mean(dim=1).numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(var_t + EPS), rtol=1e-12)


@pytest.mark.parametrize("n_parts,bias,with_dr_in", [(1, False, False), (2, True, True), (3, True, False)])
def test_ln_bwd_matches_autograd(n_parts, bias, with_dr_in):
    d = draw(5, 48, n_parts, seed=10 + n_parts, bias=bias)
    dr_in = d["dr_in"] if with_dr_in else None
    r, _, _, _ = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    dr, dgamma, dbeta, dbias = oracle.ln_residual_bwd(r, d["gamma"], EPS, d["dy"], dr_in)
    rt, yt, lv = torch_ln_residual(d)
    loss = (yt * torch.tensor(d["dy"])).sum()
    if dr_in is not None:
        loss = loss + (rt * torch.tensor(dr_in)).sum()
    loss.backward()
    tol = dict(rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dr, lv["resid_in"].grad.numpy(), **tol)
    for p in lv["parts"]:  # every part receives the same gradient
        np.testing.assert_allclose(dr, p.grad.numpy(), **tol)
    np.testing.assert_allclose(dgamma, lv["gamma"].grad.numpy(), **tol)
    np.testing.assert_allclose(dbeta, lv["beta"].grad.numpy(), **tol)
    if bias:
        np.testing.assert_allclose(dbias, lv["bias"].grad.numpy(), **tol)


def test_ln_bwd_finite_differences():
    d = draw(3, 8, 2, seed=3)

    def loss(resid_in, gamma, beta, bias):
        r, y, _, _ = oracle.ln_residual_fwd(resid_in, d["parts"], bias, gamma, beta, EPS)
        return float((y * d["dy"]).sum() + (r * d["dr_in"]).sum())

    r, _, _, _ = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    dr, dgamma, dbeta, dbias = oracle.ln_residual_bwd(r, d["gamma"], EPS, d["dy"], d["dr_in"])
    args = {"resid_in": d["resid_in"], "gamma": d["gamma"], "beta": d["beta"], "bias": d["bias"]}
    want = {"resid_in": dr, "gamma": dgamma, "beta": dbeta, "bias": dbias}
    e = 1e-6
    for name, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hi = {k: v.copy() for k, v in args.items()}
            lo = {k: v.copy() for k, v in args.items()}
            hi[name][idx] += e
            lo[name][idx] -= e
            fd[idx] = (loss(**hi) - loss(**lo)) / (2 * e)
        np.testing.assert_allclose(want[name], fd, rtol=1e-7, atol=1e-7, err_msg=name)


def test_ln_worked_row():
    # one row [1, 2, 3, 4]: mean 5/2, biased variance 5/4, so with eps -> 0 the
    # normalized row is (-3, -1, 1, 3) / sqrt(5); gamma and beta then scale and shift
    r0 = np.array([[1.0, 2.0, 3.0, 4.0]])
    gamma = np.array([1.0, 2.0, 0.5, -1.0])
    beta = np.array([0.0, 1.0, -1.0, 0.25])
    _, y, mu, rstd = oracle.ln_residual_fwd(r0, [], None, gamma, beta, 0.0)
    xhat = np.array([-3.0, -1.0, 1.0, 3.0]) / np.sqrt(5.0)
    np.testing.assert_allclose(mu, [2.5], rtol=0, atol=0)
    np.testing.assert_allclose(rstd, [1.0 / np.sqrt(1.25)], rtol=1e-15)
    np.testing.assert_allclose(y[0], xhat * gamma + beta, rtol=1e-15, atol=1e-15)


def test_ln_closed_forms():
    T, h = 7, 33
    d = draw(T, h, 2, seed=5)
    ones, zeros = np.ones(h), np.zeros(h)
    r, y, _, rstd = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], ones, zeros, EPS)
    var = 1.0 / rstd ** 2 - EPS
    # gamma = 1, beta = 0: every row has mean 0 and mean square var / (var + eps)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + EPS), rtol=1e-13)
    # a constant row normalizes to beta exactly; there xhat = 0, so its gradient
    # is (g - mean g) / sqrt(eps) with g = dy * gamma
    c = np.full((2, h), 3.25)
    _, yc, _, _ = oracle.ln_residual_fwd(c, [], None, d["gamma"], d["beta"], EPS)
    np.testing.assert_array_equal(yc, np.broadcast_to(d["beta"], yc.shape))
    drc, dgc, _, _ = oracle.ln_residual_bwd(c, d["gamma"], EPS, d["dy"][:2], None)
    gc = d["dy"][:2] * d["gamma"]
    np.testing.assert_allclose(drc, (gc - gc.mean(axis=1, keepdims=True)) / np.sqrt(EPS), rtol=1e-13, atol=1e-12)
    np.testing.assert_array_equal(dgc, 0.0)
    # a per-row shift of the residual input changes neither y nor the gradients
    shift = np.arange(T, dtype=np.float64)[:, None] * 7.5
    _, y2, _, _ = oracle.ln_residual_fwd(d["resid_in"] + shift, d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    _, y1, _, _ = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-12)
    # scaling r by s with eps scaled by s^2 leaves y unchanged
    s = 3.0
    _, y3, _, _ = oracle.ln_residual_fwd(s * r, [], None, d["gamma"], d["beta"], s * s * EPS)
    _, y4, _, _ = oracle.ln_residual_fwd(r, [], None, d["gamma"], d["beta"], EPS)
    np.testing.assert_allclose(y3, y4, rtol=1e-12, atol=1e-12)


def test_ln_bwd_invariants():
    # the norm's share of dr sums to zero over each row (the mean is removed),
    # and its projection on xhat is rstd * h * b * eps / (var + eps) with
    # b = mean(dy * gamma * xhat) (zero as eps -> 0); a dropped term breaks one
    T, h = 6, 24
    d = draw(T, h, 1, seed=7)
    r, _, mu, rstd = oracle.ln_residual_fwd(d["resid_in"], d["parts"], d["bias"], d["gamma"], d["beta"], EPS)
    dr, _, _, dbias = oracle.ln_residual_bwd(r, d["gamma"], EPS, d["dy"], d["dr_in"])
    ln_part = dr - d["dr_in"]
    xhat = (r - mu[:, None]) * rstd[:, None]
    var = (r - mu[:, None]).var(axis=1)
    b = (d["dy"] * d["gamma"] * xhat).mean(axis=1)
    scale = np.abs(ln_part).sum(axis=1)
    assert np.all(np.abs(ln_part.sum(axis=1)) <= 1e-13 * scale)
    np.testing.assert_allclose((ln_part * xhat).sum(axis=1), rstd * h * b * EPS / (var + EPS), rtol=1e-6,
                               atol=1e-13 * scale.max())
    np.testing.assert_allclose(dbias, dr.sum(axis=0), rtol=1e-15)
    # zero incoming gradients give zero gradients
    z = np.zeros((T, h))
    dr0, dg0, db0, dbias0 = oracle.ln_residual_bwd(r, d["gamma"], EPS, z, None)
    for a in (dr0, dg0, db0, dbias0):
        np.testing.assert_array_equal(a, 0.0)
