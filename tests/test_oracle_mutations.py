"""The oracle's pins reject plausible mistakes. Each case plants one mistake
in a temporary copy of the C oracle (a dropped term, a wrong sign, a
transposed operand, epsilon outside the root, a missing update, the decay
taken at the wrong state, a wrong GELU derivative), rebuilds the copy, and
checks that the autograd comparison the pins use rejects it. The shipped
oracle passes the same comparisons (test_oracle_pins.py,
test_variant_oracle.py). CPU only."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import torch_ref

SRC = os.path.join(os.path.dirname(oracle.__file__), "ttt_oracle.c")

# name -> (text in the oracle source, its replacement, replace every occurrence?, pin)
MUTATIONS = {
    "ln_backward_drops_the_xhat_term": (
        "G[j] = (gh - m1 - xh * m2) / sigma;", "G[j] = (gh - m1) / sigma;", False, "linear"),
    "ln_backward_eps_outside_the_root": (
        "double sigma = sqrt(var + eps);\n    double m1 = 0.0, m2 = 0.0;\n    for (int j = 0; j < d; ++j) {\n"
        "        double xh = (z[j] - mu) / sigma;\n        double y = gamma[j] * xh + beta[j];",
        "double sigma = sqrt(var) + eps;\n    double m1 = 0.0, m2 = 0.0;\n    for (int j = 0; j < d; ++j) {\n"
        "        double xh = (z[j] - mu) / sigma;\n        double y = gamma[j] * xh + beta[j];",
        False, "linear"),
    "update_with_the_wrong_sign": (
        "W[(size_t)i * d + jj] -= e * gw;", "W[(size_t)i * d + jj] += e * gw;", False, "linear"),
    "bias_never_updated": (
        "for (int jj = 0; jj < d; ++jj) b[jj] -= e * g[jj];", "", False, "linear"),
    "key_forward_transposes_W": (
        "for (int i = 0; i < d; ++i) acc += k[i] * W[(size_t)i * d + jj];",
        "for (int i = 0; i < d; ++i) acc += k[i] * W[(size_t)jj * d + i];", False, "linear"),
    "target_with_the_wrong_sign": (
        "tau[jj] = v[jj] - k[jj];", "tau[jj] = k[jj] - v[jj];", False, "linear"),
    "decay_at_the_current_state": (
        "gw += j->wd * Wc[(size_t)i * d + jj];", "gw += j->wd * W[(size_t)i * d + jj];", False,
        "linear_decay"),
    "inner_product_gradient_sign": (
        "double gh = -gamma[j] * v[j];", "double gh = gamma[j] * v[j];", True, "linear_ip"),
    "gelu_derivative_drops_x_phi": ("return Phi + x * phi;", "return Phi;", False, "mlp"),
    "mlp_backward_transposes_W2": (
        "acc += G2[(size_t)s * d + jj] * W2[(size_t)q * d + jj];",
        "acc += G2[(size_t)s * d + jj] * W2[(size_t)jj * m + q];", False, "mlp"),
}


def _build(tmp_path, name, old, new, every):
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    src = src.replace(old, new) if every else src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-o", str(so),
                    str(c), "-lm", "-lpthread"], check=True)
    return str(so)


def _pin_error(pin):
    """Largest difference between the oracle and the autograd definition."""
    rng = np.random.default_rng(7)
    H = 2
    if pin == "mlp":
        L, d = 11, 4
        m = 4 * d
        XQ, XK, XV = (rng.standard_normal((1, H, L, d)) for _ in range(3))
        eta = 0.05 + 0.1 * rng.random((1, H, L))
        W1 = rng.standard_normal((H, d, m)) / np.sqrt(d)
        b1 = 0.1 * rng.standard_normal((H, m))
        W2 = rng.standard_normal((H, m, d)) / np.sqrt(m)
        b2 = 0.1 * rng.standard_normal((H, d))
        g = 1 + 0.2 * rng.standard_normal((H, d))
        be = 0.2 * rng.standard_normal((H, d))
        got = oracle.mlp_forward(XQ, XK, XV, eta, W1, b1, W2, b2, g, be, 1e-6, mb=4)
        err = 0.0
        for h in range(H):
            ref = torch_ref.mlp_autograd(XQ[0, h], XK[0, h], XV[0, h], eta[0, h], W1[h], b1[h],
                                         W2[h], b2[h], g[h], be[h], 1e-6, 4)
            err = max(err, max(np.abs(x[0, h] - r).max() for x, r in zip(got, ref)))
        return err
    L, d = 23, 8
    XQ, XK, XV = (rng.standard_normal((1, H, L, d)) for _ in range(3))
    eta = 0.05 + 0.1 * rng.random((1, H, L))
    W0 = 0.3 * rng.standard_normal((H, d, d))
    b0 = 0.1 * rng.standard_normal((H, d))
    g = 1 + 0.2 * rng.standard_normal((H, d))
    be = 0.2 * rng.standard_normal((H, d))
    loss = "inner_product" if pin == "linear_ip" else "mse"
    wd = 0.3 if pin == "linear_decay" else 0.0
    got = oracle.linear_forward_opts(XQ, XK, XV, eta, W0, b0, g, be, 1e-6, mb=4, loss=loss,
                                     weight_decay=wd)
    err = 0.0
    for h in range(H):
        ref = torch_ref.linear_autograd_opts(XQ[0, h], XK[0, h], XV[0, h], eta[0, h], W0[h], b0[h],
                                             g[h], be[h], 1e-6, 4, loss, wd)
        err = max(err, max(np.abs(x[0, h] - r).max() for x, r in zip(got, ref)))
    return err


@pytest.mark.parametrize("pin", ["linear", "linear_decay", "linear_ip", "mlp"])
def test_the_shipped_oracle_passes(pin):
    assert _pin_error(pin) <= 1e-11


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_planted_mistake_fails_the_pin(name, tmp_path, monkeypatch):
    old, new, every, pin = MUTATIONS[name]
    so = _build(tmp_path, name, old, new, every)
    monkeypatch.setattr(oracle, "_LIB_PATH", so)
    monkeypatch.setattr(oracle, "_lib", None)
    err = _pin_error(pin)
    assert err > 1e-6, (name, err)
