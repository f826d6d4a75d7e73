"""Pins of the gradient oracle (oracle/grad.py): its forward equals the C
oracle's, its written-out layer-norm L2 gradient equals autograd of the loss it
differentiates, every gradient matches central finite differences of the C
oracle's forward (an independent implementation), and eta = 0 reduces to the
textbook layer-norm backward of a static linear layer."""
import numpy as np
import pytest
import torch

import oracle
from oracle import grad as OG


def _case(seed, B=2, H=2, L=13, d=8, mb=4, scale_w=0.3):
    rng = np.random.default_rng(seed)
    XQ, XK, XV = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    eta = 0.05 + 0.1 * rng.random((B, H, L))
    W0 = scale_w * rng.standard_normal((B, H, d, d))
    b0 = 0.1 * rng.standard_normal((B, H, d))
    gamma = 1 + 0.2 * rng.standard_normal((H, d))
    beta = 0.2 * rng.standard_normal((H, d))
    dO = rng.standard_normal((B, H, L, d))
    dW = rng.standard_normal((B, H, d, d))
    db = rng.standard_normal((B, H, d))
    return dict(XQ=XQ, XK=XK, XV=XV, eta=eta, W0=W0, b0=b0, gamma=gamma, beta=beta), dO, dW, db, mb


def _fd(x, name, V, dO, dW, db, mb, h=1e-5):
    """Directional derivative of the C oracle's loss along V: central
    differences at h and h/2 combined by Richardson extrapolation (error O(h^4))."""
    def D(hh):
        xp = dict(x); xp[name] = x[name] + hh * V
        xm = dict(x); xm[name] = x[name] - hh * V
        return (_c_loss(xp, dO, dW, db, mb) - _c_loss(xm, dO, dW, db, mb)) / (2 * hh)
    return (4 * D(h / 2) - D(h)) / 3


def _c_loss(x, dO, dW, db, mb, eps=1e-6):
    O, W, b = oracle.linear_forward(x["XQ"], x["XK"], x["XV"], x["eta"], x["W0"], x["b0"],
                                    x["gamma"], x["beta"], eps, mb=mb, w0_batched=True)
    return float((O * dO).sum() + (W * dW).sum() + (b * db).sum())


def test_forward_matches_c_oracle():
    x, dO, dW, db, mb = _case(1)
    ts = [torch.tensor(x[k]) for k in ("XQ", "XK", "XV", "eta", "W0", "b0", "gamma", "beta")]
    O, W, b = OG.linear_primal(*ts, 1e-6, mb)
    ref = oracle.linear_forward(x["XQ"], x["XK"], x["XV"], x["eta"], x["W0"], x["b0"], x["gamma"],
                                x["beta"], 1e-6, mb=mb, w0_batched=True)
    for got, want in zip((O, W, b), ref):
        got = got.detach().numpy()
        assert np.abs(got - want).max() <= 1e-12 * max(1.0, np.abs(want).max())


def test_ln_l2_grad_formula_is_the_gradient_of_its_loss():
    rng = np.random.default_rng(2)
    z = torch.tensor(rng.standard_normal((5, 16)), requires_grad=True)
    tau = torch.tensor(rng.standard_normal((5, 16)))
    g = torch.tensor(1 + 0.3 * rng.standard_normal(16))
    bt = torch.tensor(0.3 * rng.standard_normal(16))
    loss = 0.5 * ((OG.ln(z, g, bt, 1e-6) - tau) ** 2).sum()
    (auto,) = torch.autograd.grad(loss, z)
    formula = OG.ln_l2_grad(z, tau, g, bt, 1e-6)
    assert torch.allclose(formula, auto, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["XQ", "XK", "XV", "eta", "W0", "b0", "gamma", "beta"])
def test_gradients_match_central_differences(name):
    x, dO, dW, db, mb = _case(3)
    g = OG.linear_backward(x["XQ"], x["XK"], x["XV"], x["eta"], x["W0"], x["b0"], x["gamma"],
                           x["beta"], 1e-6, mb, dO, dW, db)["d" + name]
    rng = np.random.default_rng(30)
    V = rng.standard_normal(x[name].shape)
    fd = _fd(x, name, V, dO, dW, db, mb)
    an = float((g * V).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_partial_last_chunk_and_mb1():
    """L % mb != 0 and mb = 1 (per-token TTT) against finite differences in eta."""
    for mb, L in ((5, 11), (1, 6)):
        x, dO, dW, db, _ = _case(4, L=L, mb=mb)
        g = OG.linear_backward(x["XQ"], x["XK"], x["XV"], x["eta"], x["W0"], x["b0"], x["gamma"],
                               x["beta"], 1e-6, mb, dO, dW, db)
        for name in ("eta", "XK"):
            V = np.random.default_rng(5).standard_normal(x[name].shape)
            fd = _fd(x, name, V, dO, dW, db, mb)
            an = float((g["d" + name] * V).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (mb, name, fd, an)


def test_eta_zero_is_the_layer_norm_backward_of_a_static_layer():
    """eta = 0 freezes the state: O = XQ + LN(XQ W0 + b0), whose gradients are
    the textbook layer-norm backward; XK and XV then get no gradient."""
    x, dO, _, _, mb = _case(6)
    x["eta"] = np.zeros_like(x["eta"])
    g = OG.linear_backward(x["XQ"], x["XK"], x["XV"], x["eta"], x["W0"], x["b0"], x["gamma"],
                           x["beta"], 1e-6, mb, dO)
    Z = x["XQ"] @ x["W0"] + x["b0"][:, :, None, :]
    mu = Z.mean(-1, keepdims=True)
    sig = np.sqrt(((Z - mu) ** 2).mean(-1, keepdims=True) + 1e-6)
    xh = (Z - mu) / sig
    gd = x["gamma"][None, :, None, :] * dO
    dZ = (gd - gd.mean(-1, keepdims=True) - xh * (gd * xh).mean(-1, keepdims=True)) / sig
    tol = lambda a: 1e-12 * max(1.0, np.abs(a).max())
    assert np.abs(g["dXQ"] - (dO + dZ @ np.swapaxes(x["W0"], -1, -2))).max() <= tol(g["dXQ"])
    assert np.abs(g["dW0"] - np.swapaxes(x["XQ"], -1, -2) @ dZ).max() <= tol(g["dW0"])
    assert np.abs(g["db0"] - dZ.sum(2)).max() <= tol(g["db0"])
    assert np.abs(g["dgamma"] - (dO * xh).sum((0, 2))).max() <= tol(g["dgamma"])
    assert np.abs(g["dbeta"] - dO.sum((0, 2))).max() <= tol(g["dbeta"])
    assert np.abs(g["dXK"]).max() == 0 and np.abs(g["dXV"]).max() == 0
