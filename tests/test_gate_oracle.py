"""Pins of the learning-rate gate in the oracle (the lryc.cn article §2.2,
eta = eta_base * logistic(theta_lr . x), x := the head's key): special values
of the logistic function, its symmetry, SciPy's logistic routine, and central
finite differences of the C oracle's forward for the gradients through it."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import grad as OG
from test_sequence_layer_ttt_amd import gen


def _xk(seed, B=2, H=3, L=7, d=8):
    return np.random.default_rng(seed).standard_normal((B, H, L, d))


def test_zero_weights_give_half_the_base_rate():
    XK = _xk(1)
    eta = oracle.eta_gate(XK, np.zeros((3, 8)), 0.25)
    assert np.all(eta == 0.125)


def test_symmetry_and_limits():
    XK = _xk(2)
    th = np.random.default_rng(3).standard_normal((3, 8))
    a, b = oracle.eta_gate(XK, th, 0.5), oracle.eta_gate(XK, -th, 0.5)
    assert np.abs(a + b - 0.5).max() <= 1e-15          # logistic(s) + logistic(-s) = 1
    assert np.all((a > 0) & (a < 0.5))
    big = oracle.eta_gate(np.full((1, 1, 2, 4), 1.0), np.array([[1e3, 1e3, 1e3, 1e3]]), 0.5)
    small = oracle.eta_gate(np.full((1, 1, 2, 4), 1.0), np.array([[-1e3, -1e3, -1e3, -1e3]]), 0.5)
    assert np.all(big == 0.5) and np.all(small == 0.0)


def test_matches_scipy_logistic_per_head():
    """The gate reads theta_lr[h] with the keys of head h (not another head)."""
    XK = _xk(4)
    th = np.random.default_rng(5).standard_normal((3, 8))
    eta = oracle.eta_gate(XK, th, 1 / 64)
    for h in range(3):
        s = np.einsum("bld,d->bl", XK[:, h], th[h])
        assert np.abs(eta[:, h] - expit(s) / 64).max() <= 1e-17


def test_gated_workload_draws_only_the_gate_weights():
    x = gen.make_workload(1)
    assert x.eta is None and x.theta_lr.shape == (1, 16) and x.eta_base == 1 / 16
    eta = oracle.eta_gate(x.XK, x.theta_lr, x.eta_base)
    assert np.all(eta > 0) and np.all(eta < 1 / 16)


def _case(seed, B=2, H=2, L=13, d=8, mb=4):
    rng = np.random.default_rng(seed)
    XQ, XK, XV = (rng.standard_normal((B, H, L, d)) for _ in range(3))
    theta = 0.5 * rng.standard_normal((H, d))
    W0 = 0.3 * rng.standard_normal((B, H, d, d))
    b0 = 0.1 * rng.standard_normal((B, H, d))
    gamma = 1 + 0.2 * rng.standard_normal((H, d))
    beta = 0.2 * rng.standard_normal((H, d))
    dO = rng.standard_normal((B, H, L, d))
    dW = rng.standard_normal((B, H, d, d))
    db = rng.standard_normal((B, H, d))
    x = dict(XQ=XQ, XK=XK, XV=XV, theta=theta, W0=W0, b0=b0, gamma=gamma, beta=beta)
    return x, dO, dW, db, mb


ETA_BASE = 0.125


def _c_loss(x, dO, dW, db, mb, eps=1e-6):
    O, W, b = oracle.linear_forward_gated(x["XQ"], x["XK"], x["XV"], x["theta"], ETA_BASE,
                                          x["W0"], x["b0"], x["gamma"], x["beta"], eps, mb=mb,
                                          w0_batched=True)
    return float((O * dO).sum() + (W * dW).sum() + (b * db).sum())


def _fd(x, name, V, dO, dW, db, mb, h=1e-5):
    def D(hh):
        xp = dict(x); xp[name] = x[name] + hh * V
        xm = dict(x); xm[name] = x[name] - hh * V
        return (_c_loss(xp, dO, dW, db, mb) - _c_loss(xm, dO, dW, db, mb)) / (2 * hh)
    return (4 * D(h / 2) - D(h)) / 3


@pytest.mark.parametrize("name", ["theta", "XK", "XQ"])
def test_gated_gradients_match_central_differences(name):
    x, dO, dW, db, mb = _case(11)
    g = OG.linear_backward_gated(x["XQ"], x["XK"], x["XV"], x["theta"], ETA_BASE, x["W0"],
                                 x["b0"], x["gamma"], x["beta"], 1e-6, mb, dO, dW, db)
    V = np.random.default_rng(12).standard_normal(x[name].shape)
    fd = _fd(x, name, V, dO, dW, db, mb)
    an = float((g["d" + name] * V).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_chain_rule_split():
    """The gated gradients equal the ungated ones at the gated eta plus the
    gate's own backward driven by deta (the split the GPU path takes)."""
    x, dO, dW, db, mb = _case(13)
    full = OG.linear_backward_gated(x["XQ"], x["XK"], x["XV"], x["theta"], ETA_BASE, x["W0"],
                                    x["b0"], x["gamma"], x["beta"], 1e-6, mb, dO, dW, db)
    eta = oracle.eta_gate(x["XK"], x["theta"], ETA_BASE)
    part = OG.linear_backward(x["XQ"], x["XK"], x["XV"], eta, x["W0"], x["b0"], x["gamma"],
                              x["beta"], 1e-6, mb, dO, dW, db)
    gate = OG.eta_gate_backward(x["XK"], x["theta"], ETA_BASE, part["deta"])
    tol = lambda a: 1e-12 * max(1.0, np.abs(a).max())
    assert np.abs(full["eta"] - eta).max() <= 1e-15
    assert np.abs(full["dXK"] - (part["dXK"] + gate["dXK"])).max() <= tol(full["dXK"])
    assert np.abs(full["dtheta"] - gate["dtheta"].sum(0)).max() <= tol(full["dtheta"])
    for k in ("dXQ", "dXV", "dW0", "db0", "dgamma", "dbeta"):
        assert np.abs(full[k] - part[k]).max() <= tol(full[k]), k


def test_gate_backward_against_central_differences():
    XK = _xk(14)
    th = np.random.default_rng(15).standard_normal((3, 8))
    deta = np.random.default_rng(16).standard_normal((2, 3, 7))
    g = OG.eta_gate_backward(XK, th, 0.3, deta)
    f = lambda xk, t: float((oracle.eta_gate(xk, t, 0.3) * deta).sum())
    for V, which in ((np.random.default_rng(17).standard_normal(XK.shape), "dXK"),
                     (np.random.default_rng(18).standard_normal(th.shape), "dtheta")):
        h = 1e-5
        if which == "dXK":
            D = lambda hh: (f(XK + hh * V, th) - f(XK - hh * V, th)) / (2 * hh)
            an = float((g["dXK"] * V).sum())
        else:
            D = lambda hh: (f(XK, th + hh * V) - f(XK, th - hh * V)) / (2 * hh)
            an = float((g["dtheta"].sum(0) * V).sum())
        fd = (4 * D(h / 2) - D(h)) / 3
        assert abs(fd - an) <= 1e-8 * max(1.0, abs(an)), (which, fd, an)
