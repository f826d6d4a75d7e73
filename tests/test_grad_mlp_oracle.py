"""Pins of the TTT-MLP gradient oracle (oracle/grad.py mlp_primal,
mlp_backward): its forward equals the C oracle's TTT-MLP primal, its written-out
GELU derivative is the derivative of GELU, every gradient matches central
finite differences of the C oracle's forward (an independent implementation),
and eta = 0 reduces to the textbook backward of a static two-layer GELU MLP
followed by a layer norm."""
import numpy as np
import pytest
import torch

import oracle
from oracle import grad as OG

NAMES = ("XQ", "XK", "XV", "eta", "W1", "b1", "W2", "b2", "gamma", "beta")


def _case(seed, B=2, H=2, L=11, d=4, mb=4):
    rng = np.random.default_rng(seed)
    m = 4 * d
    x = {n: rng.standard_normal((B, H, L, d)) for n in ("XQ", "XK", "XV")}
    x["eta"] = 0.05 + 0.2 * rng.random((B, H, L))
    x["W1"] = 0.4 * rng.standard_normal((B, H, d, m))
    x["b1"] = 0.2 * rng.standard_normal((B, H, m))
    x["W2"] = 0.3 * rng.standard_normal((B, H, m, d))
    x["b2"] = 0.1 * rng.standard_normal((B, H, d))
    x["gamma"] = 1 + 0.2 * rng.standard_normal((H, d))
    x["beta"] = 0.2 * rng.standard_normal((H, d))
    adj = dict(dO=rng.standard_normal((B, H, L, d)), dW1=rng.standard_normal((B, H, d, m)),
               db1=rng.standard_normal((B, H, m)), dW2=rng.standard_normal((B, H, m, d)),
               db2=rng.standard_normal((B, H, d)))
    return x, adj, mb


def _c_loss(x, adj, mb, eps=1e-6):
    O, W1, b1, W2, b2 = oracle.mlp_forward(*(x[n] for n in NAMES), eps, mb=mb, w0_batched=True)
    return float((O * adj["dO"]).sum() + (W1 * adj["dW1"]).sum() + (b1 * adj["db1"]).sum()
                 + (W2 * adj["dW2"]).sum() + (b2 * adj["db2"]).sum())


def _fd(x, name, V, adj, mb, h=1e-5):
    """Directional derivative of the C oracle's loss along V (central
    differences at h and h/2, Richardson-extrapolated, error O(h^4))."""
    def D(hh):
        xp = dict(x); xp[name] = x[name] + hh * V
        xm = dict(x); xm[name] = x[name] - hh * V
        return (_c_loss(xp, adj, mb) - _c_loss(xm, adj, mb)) / (2 * hh)
    return (4 * D(h / 2) - D(h)) / 3


def _grads(x, adj, mb):
    return OG.mlp_backward(*(x[n] for n in NAMES), 1e-6, mb, adj["dO"], adj["dW1"], adj["db1"],
                           adj["dW2"], adj["db2"])


def test_forward_matches_c_oracle():
    x, _, mb = _case(1)
    got = OG.mlp_primal(*(torch.tensor(x[n]) for n in NAMES), 1e-6, mb)
    ref = oracle.mlp_forward(*(x[n] for n in NAMES), 1e-6, mb=mb, w0_batched=True)
    for g, r in zip(got, ref):
        assert np.abs(g.numpy() - r).max() <= 1e-12 * max(1.0, np.abs(r).max())


def test_gelu_prime_is_the_derivative_of_gelu():
    z = torch.linspace(-8, 8, 1001, dtype=torch.float64, requires_grad=True)
    (auto,) = torch.autograd.grad(OG.gelu(z).sum(), z)
    assert torch.allclose(OG.gelu_prime(z.detach()), auto, rtol=0, atol=1e-14)
    # and gelu itself is x Phi(x): Phi(0) = 1/2, Phi(1.959963984540054) = 0.975
    assert float(OG.gelu(torch.tensor(1.959963984540054, dtype=torch.float64))) == pytest.approx(
        0.975 * 1.959963984540054, rel=1e-12)


@pytest.mark.parametrize("name", NAMES)
def test_gradients_match_central_differences(name):
    x, adj, mb = _case(3)
    g = _grads(x, adj, mb)["d" + name]
    V = np.random.default_rng(31).standard_normal(x[name].shape)
    fd = _fd(x, name, V, adj, mb)
    an = float((g * V).sum())
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_partial_last_chunk_and_mb1():
    """L % mb != 0 and mb = 1 (per-token TTT) against finite differences."""
    for mb, L in ((5, 11), (1, 5)):
        x, adj, _ = _case(4, L=L, mb=mb)
        g = _grads(x, adj, mb)
        for name in ("eta", "XK", "W2"):
            V = np.random.default_rng(6).standard_normal(x[name].shape)
            fd = _fd(x, name, V, adj, mb)
            an = float((g["d" + name] * V).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (mb, name, fd, an)


def test_eta_zero_is_the_backward_of_a_static_mlp():
    """eta = 0 freezes the state: O = XQ + LN(gelu(XQ W1 + b1) W2 + b2); its
    gradients are the chain rule through LN, the second layer, GELU and the
    first layer written out in NumPy; XK and XV get no gradient."""
    from scipy.special import erf
    x, adj, mb = _case(7)
    x["eta"] = np.zeros_like(x["eta"])
    g = OG.mlp_backward(*(x[n] for n in NAMES), 1e-6, mb, adj["dO"])
    dO = adj["dO"]
    Z1 = x["XQ"] @ x["W1"] + x["b1"][:, :, None, :]
    Phi = 0.5 * (1 + erf(Z1 / np.sqrt(2)))
    A = Z1 * Phi
    Z2 = A @ x["W2"] + x["b2"][:, :, None, :]
    mu = Z2.mean(-1, keepdims=True)
    sig = np.sqrt(((Z2 - mu) ** 2).mean(-1, keepdims=True) + 1e-6)
    xh = (Z2 - mu) / sig
    gd = x["gamma"][None, :, None, :] * dO
    dZ2 = (gd - gd.mean(-1, keepdims=True) - xh * (gd * xh).mean(-1, keepdims=True)) / sig
    T = lambda a: np.swapaxes(a, -1, -2)
    dA = dZ2 @ T(x["W2"])
    dZ1 = dA * (Phi + Z1 * np.exp(-0.5 * Z1 ** 2) / np.sqrt(2 * np.pi))
    tol = lambda a: 1e-12 * max(1.0, np.abs(a).max())
    want = {"dXQ": dO + dZ1 @ T(x["W1"]), "dW1": T(x["XQ"]) @ dZ1, "db1": dZ1.sum(2),
            "dW2": T(A) @ dZ2, "db2": dZ2.sum(2), "dgamma": (dO * xh).sum((0, 2)),
            "dbeta": dO.sum((0, 2))}
    for k, w in want.items():
        assert np.abs(g[k] - w).max() <= tol(w), k
    assert np.abs(g["dXK"]).max() == 0 and np.abs(g["dXV"]).max() == 0
