"""Pins of the oracle's Modular-TTT options (the Modular-TTT page lists the
loss, MSE or inner product, and weight decay on the fast weights as design
axes): oracle.linear_forward_opts against an autograd implementation of the
definition, closed forms for weight decay and for the inner-product loss, and
reduction to the default layer."""
import numpy as np
import pytest

import oracle
from tests import torch_ref


def _case(seed, L=23, d=8, H=2):
    rng = np.random.default_rng(seed)
    XQ, XK, XV = (rng.standard_normal((1, H, L, d)) for _ in range(3))
    eta = 0.05 + 0.1 * rng.random((1, H, L))
    W0 = 0.3 * rng.standard_normal((H, d, d))
    b0 = 0.1 * rng.standard_normal((H, d))
    gamma = 1 + 0.2 * rng.standard_normal((H, d))
    beta = 0.2 * rng.standard_normal((H, d))
    return XQ, XK, XV, eta, W0, b0, gamma, beta


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.3])
@pytest.mark.parametrize("mb", [1, 4, 16])
def test_matches_autograd_of_the_definition(loss, wd, mb):
    XQ, XK, XV, eta, W0, b0, g, be = _case(20 + mb)
    O, W, b = oracle.linear_forward_opts(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=mb, loss=loss,
                                         weight_decay=wd)
    for h in range(2):
        Or, Wr, br = torch_ref.linear_autograd_opts(XQ[0, h], XK[0, h], XV[0, h], eta[0, h], W0[h],
                                                    b0[h], g[h], be[h], 1e-6, mb, loss, wd)
        for got, ref in ((O[0, h], Or), (W[0, h], Wr), (b[0, h], br)):
            assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_defaults_equal_the_plain_layer():
    XQ, XK, XV, eta, W0, b0, g, be = _case(30)
    a = oracle.linear_forward(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=4)
    b = oracle.linear_forward_opts(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=4)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_weight_decay_alone_scales_the_state():
    """Zero keys: the reconstruction gradient of W (xk^T G) vanishes, so each
    chunk only scales W by 1 - lambda * (sum of the chunk's eta)."""
    XQ, XK, XV, eta, W0, b0, g, be = _case(31)
    XK = np.zeros_like(XK)
    lam, mb = 0.7, 5
    _, W, _ = oracle.linear_forward_opts(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=mb, loss="mse",
                                         weight_decay=lam)
    for h in range(2):
        f = 1.0
        for c0 in range(0, eta.shape[2], mb):
            f *= 1.0 - lam * eta[0, h, c0:c0 + mb].sum()
        assert np.abs(W[0, h] - f * W0[h]).max() <= 1e-13


def test_inner_product_loss_with_zero_values_is_static():
    """The inner-product gradient is linear in XV: XV = 0 leaves the state at
    (W0, b0) and the output is the static layer XQ + LN(XQ W0 + b0)."""
    XQ, XK, XV, eta, W0, b0, g, be = _case(32)
    O, W, b = oracle.linear_forward_opts(XQ, XK, np.zeros_like(XV), eta, W0, b0, g, be, 1e-6,
                                         mb=4, loss="inner_product")
    assert np.array_equal(W[0], W0) and np.array_equal(b[0], b0)
    for h in range(2):
        Z = XQ[0, h] @ W0[h] + b0[h]
        mu = Z.mean(-1, keepdims=True)
        sd = np.sqrt(((Z - mu) ** 2).mean(-1, keepdims=True) + 1e-6)
        assert np.abs(O[0, h] - (XQ[0, h] + g[h] * (Z - mu) / sd + be[h])).max() <= 1e-13


def test_inner_product_gradient_is_linear_in_the_values():
    """One token, b = 1: the inner-product update is linear in XV (doubling
    XV doubles W - W0 and b - b0), unlike the squared error's."""
    XQ, XK, XV, eta, W0, b0, g, be = _case(33, L=1)
    _, W1, b1 = oracle.linear_forward_opts(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=1,
                                           loss="inner_product")
    _, W2, b2 = oracle.linear_forward_opts(XQ, XK, 2 * XV, eta, W0, b0, g, be, 1e-6, mb=1,
                                           loss="inner_product")
    assert np.abs((W2[0] - W0) - 2 * (W1[0] - W0)).max() <= 1e-13
    assert np.abs((b2[0] - b0) - 2 * (b1[0] - b0)).max() <= 1e-13


def _mlp_case(seed, L=11, d=4, H=2):
    rng = np.random.default_rng(seed)
    m = 4 * d
    XQ, XK, XV = (rng.standard_normal((1, H, L, d)) for _ in range(3))
    eta = 0.05 + 0.1 * rng.random((1, H, L))
    W1 = rng.standard_normal((H, d, m)) / np.sqrt(d)
    b1 = 0.1 * rng.standard_normal((H, m))
    W2 = rng.standard_normal((H, m, d)) / np.sqrt(m)
    b2 = 0.1 * rng.standard_normal((H, d))
    gamma = 1 + 0.2 * rng.standard_normal((H, d))
    beta = 0.2 * rng.standard_normal((H, d))
    return XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.4])
@pytest.mark.parametrize("mb", [1, 4])
def test_mlp_matches_autograd_of_the_definition(loss, wd, mb):
    XQ, XK, XV, eta, W1, b1, W2, b2, g, be = _mlp_case(40 + mb)
    got = oracle.mlp_forward_opts(XQ, XK, XV, eta, W1, b1, W2, b2, g, be, 1e-6, mb=mb, loss=loss,
                                  weight_decay=wd)
    for h in range(2):
        ref = torch_ref.mlp_autograd_opts(XQ[0, h], XK[0, h], XV[0, h], eta[0, h], W1[h], b1[h],
                                          W2[h], b2[h], g[h], be[h], 1e-6, mb, loss, wd)
        for x, r in zip(got, ref):
            assert np.abs(x[0, h] - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


def test_mlp_defaults_equal_the_plain_layer():
    c = _mlp_case(50)
    a = oracle.mlp_forward(*c, 1e-6, mb=4)
    b = oracle.mlp_forward_opts(*c, 1e-6, mb=4)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_mlp_weight_decay_alone_scales_both_weights():
    """XV = 0 under the inner-product loss makes the loss gradient vanish, so
    with decay each chunk scales W1 and W2 by 1 - lambda * (sum of the chunk's
    eta) and leaves b1, b2 alone."""
    XQ, XK, XV, eta, W1, b1, W2, b2, g, be = _mlp_case(51, L=13)
    lam, mb = 0.6, 4
    _, W1o, b1o, W2o, b2o = oracle.mlp_forward_opts(XQ, XK, np.zeros_like(XV), eta, W1, b1, W2,
                                                    b2, g, be, 1e-6, mb=mb,
                                                    loss="inner_product", weight_decay=lam)
    for h in range(2):
        f = 1.0
        for c0 in range(0, eta.shape[2], mb):
            f *= 1.0 - lam * eta[0, h, c0:c0 + mb].sum()
        assert np.abs(W1o[0, h] - f * W1[h]).max() <= 1e-13
        assert np.abs(W2o[0, h] - f * W2[h]).max() <= 1e-13
        assert np.array_equal(b1o[0, h], b1[h]) and np.array_equal(b2o[0, h], b2[h])


def test_mlp_inner_product_second_layer_step_is_closed_form():
    """One token, b = 1, inner-product loss: the gradient at the second
    layer's output is g = -(gamma * v) pushed back through the layer norm,
    i.e. -(gamma v - mean(gamma v) - yhat * mean(gamma v * yhat)) / sigma with
    yhat the normalised z2, so b2' = b2 - eta g and W2' = W2 - eta a g^T with
    a = gelu(xk W1 + b1)."""
    from math import erf, sqrt
    XQ, XK, XV, eta, W1, b1, W2, b2, g, be = _mlp_case(52, L=1)
    eps = 1e-6
    _, _, _, W2o, b2o = oracle.mlp_forward_opts(XQ, XK, XV, eta, W1, b1, W2, b2, g, be, eps,
                                                mb=1, loss="inner_product")
    for h in range(2):
        k, v, e = XK[0, h, 0], XV[0, h, 0], eta[0, h, 0]
        z1 = k @ W1[h] + b1[h]
        a = np.array([0.5 * x * (1 + erf(x / sqrt(2))) for x in z1])
        z2 = a @ W2[h] + b2[h]
        mu = z2.mean()
        sig = np.sqrt(((z2 - mu) ** 2).mean() + eps)
        yh = (z2 - mu) / sig
        u = g[h] * v
        grad = -(u - u.mean() - yh * (u * yh).mean()) / sig
        assert np.abs(b2o[0, h] - (b2[h] - e * grad)).max() <= 1e-13
        assert np.abs(W2o[0, h] - (W2[h] - e * np.outer(a, grad))).max() <= 1e-13
