"""Independent references used to pin the oracle (tests only).

These take every gradient by torch autograd (fp64, CPU) or by finite /
complex-step differences of the loss, never by the oracle's hand-derived
layer-norm backward, so a dropped term, a wrong sign or a transposed operand in
the oracle fails against them.

Definition followed ([D] = damodev.csdn.net TTT deep-dive, [Y] = lryc.cn TTT
article): update then apply, [D] §3.1; reconstruction target XV - XK and
forward XK W + b, [D] §4.2; output f(x) = x + LN(f_res(x)), [Y] §2.1;
mini-batch: gradients at the chunk-start state, [D] §4.1.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def chunk_schedule(L, mb):
    s = [mb] * (L // mb)
    if L % mb:
        s.append(L % mb)
    return s


def linear_autograd(XQ, XK, XV, eta, W0, b0, gamma, beta, eps, mb):
    """Mini-batch TTT-Linear for one sequence via autograd. Inputs [L,d]."""
    xq, xk, xv, et = _t(XQ), _t(XK), _t(XV), _t(eta)
    W = _t(W0).clone()
    b = _t(b0).clone()
    g_, be_ = _t(gamma), _t(beta)
    L, d = xq.shape
    O = torch.zeros(L, d, dtype=torch.float64)
    t0 = 0
    for n in chunk_schedule(L, mb):
        Wc = W.clone().requires_grad_(True)
        bc = b.clone().requires_grad_(True)
        grads = []
        for s in range(t0, t0 + n):
            z = xk[s] @ Wc + bc
            y = F.layer_norm(z, (d,), g_, be_, eps)
            loss = 0.5 * ((y - (xv[s] - xk[s])) ** 2).sum()
            gW, gb = torch.autograd.grad(loss, (Wc, bc))
            grads.append((gW, gb))
        for i, s in enumerate(range(t0, t0 + n)):
            W = W - et[s] * grads[i][0]
            b = b - et[s] * grads[i][1]
            zb = xq[s] @ W + b
            O[s] = xq[s] + F.layer_norm(zb, (d,), g_, be_, eps)
        t0 += n
    return O.numpy(), W.detach().numpy(), b.detach().numpy()


def linear_autograd_opts(XQ, XK, XV, eta, W0, b0, gamma, beta, eps, mb, loss="mse", wd=0.0):
    """linear_autograd with the Modular-TTT options: per-token loss "mse"
    (1/2 ||LN(z) - (xv - xk)||^2) or "inner_product" (-< xk + LN(z), xv >),
    plus wd/2 ||W||^2; every gradient by autograd at the chunk-start state."""
    xq, xk, xv, et = _t(XQ), _t(XK), _t(XV), _t(eta)
    W = _t(W0).clone()
    b = _t(b0).clone()
    g_, be_ = _t(gamma), _t(beta)
    L, d = xq.shape
    O = torch.zeros(L, d, dtype=torch.float64)
    t0 = 0
    for n in chunk_schedule(L, mb):
        Wc = W.clone().requires_grad_(True)
        bc = b.clone().requires_grad_(True)
        grads = []
        for s in range(t0, t0 + n):
            y = F.layer_norm(xk[s] @ Wc + bc, (d,), g_, be_, eps)
            if loss == "mse":
                ls = 0.5 * ((y - (xv[s] - xk[s])) ** 2).sum()
            else:
                ls = -((xk[s] + y) * xv[s]).sum()
            ls = ls + 0.5 * wd * (Wc ** 2).sum()
            grads.append(torch.autograd.grad(ls, (Wc, bc)))
        for i, s in enumerate(range(t0, t0 + n)):
            W = W - et[s] * grads[i][0]
            b = b - et[s] * grads[i][1]
            O[s] = xq[s] + F.layer_norm(xq[s] @ W + b, (d,), g_, be_, eps)
        t0 += n
    return O.numpy(), W.detach().numpy(), b.detach().numpy()


def mlp_autograd(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps, mb):
    """Mini-batch TTT-MLP (d -> 4d exact GELU -> d) via autograd. Inputs [L,d]."""
    xq, xk, xv, et = _t(XQ), _t(XK), _t(XV), _t(eta)
    P = [_t(W1).clone(), _t(b1).clone(), _t(W2).clone(), _t(b2).clone()]
    g_, be_ = _t(gamma), _t(beta)
    L, d = xq.shape

    def f_res(x, p):
        return F.gelu(x @ p[0] + p[1], approximate="none") @ p[2] + p[3]

    O = torch.zeros(L, d, dtype=torch.float64)
    t0 = 0
    for n in chunk_schedule(L, mb):
        Pc = [p.clone().requires_grad_(True) for p in P]
        grads = []
        for s in range(t0, t0 + n):
            y = F.layer_norm(f_res(xk[s], Pc), (d,), g_, be_, eps)
            loss = 0.5 * ((y - (xv[s] - xk[s])) ** 2).sum()
            grads.append(torch.autograd.grad(loss, Pc))
        for i, s in enumerate(range(t0, t0 + n)):
            P = [p - et[s] * g for p, g in zip(P, grads[i])]
            O[s] = xq[s] + F.layer_norm(f_res(xq[s], P), (d,), g_, be_, eps)
        t0 += n
    return (O.numpy(),) + tuple(p.detach().numpy() for p in P)


def mlp_autograd_opts(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps, mb, loss="mse",
                      wd=0.0):
    """mlp_autograd with the Modular-TTT options: per-token loss "mse" or
    "inner_product" (-< xk + LN(f_res(xk)), xv >), plus
    wd/2 (||W1||^2 + ||W2||^2); every gradient by autograd at the chunk-start
    state."""
    xq, xk, xv, et = _t(XQ), _t(XK), _t(XV), _t(eta)
    P = [_t(W1).clone(), _t(b1).clone(), _t(W2).clone(), _t(b2).clone()]
    g_, be_ = _t(gamma), _t(beta)
    L, d = xq.shape

    def f_res(x, p):
        return F.gelu(x @ p[0] + p[1], approximate="none") @ p[2] + p[3]

    O = torch.zeros(L, d, dtype=torch.float64)
    t0 = 0
    for n in chunk_schedule(L, mb):
        Pc = [p.clone().requires_grad_(True) for p in P]
        grads = []
        for s in range(t0, t0 + n):
            y = F.layer_norm(f_res(xk[s], Pc), (d,), g_, be_, eps)
            if loss == "mse":
                ls = 0.5 * ((y - (xv[s] - xk[s])) ** 2).sum()
            else:
                ls = -((xk[s] + y) * xv[s]).sum()
            ls = ls + 0.5 * wd * ((Pc[0] ** 2).sum() + (Pc[2] ** 2).sum())
            grads.append(torch.autograd.grad(ls, Pc))
        for i, s in enumerate(range(t0, t0 + n)):
            P = [p - et[s] * g for p, g in zip(P, grads[i])]
            O[s] = xq[s] + F.layer_norm(f_res(xq[s], P), (d,), g_, be_, eps)
        t0 += n
    return (O.numpy(),) + tuple(p.detach().numpy() for p in P)


def token_loss_np(z, tau, gamma, beta, eps):
    """l(z) = 1/2 ||LN(z) - tau||^2 written with plain NumPy operations that
    also accept complex arguments (for complex-step differentiation)."""
    d = z.shape[-1]
    mu = z.sum(-1, keepdims=True) / d
    var = ((z - mu) * (z - mu)).sum(-1, keepdims=True) / d
    y = gamma * (z - mu) / np.sqrt(var + eps) + beta
    r = y - tau
    return 0.5 * (r * r).sum(-1)


def complex_step_grad(z, tau, gamma, beta, eps, h=1e-30):
    """d l / d z for each row of z by complex-step differentiation."""
    z = np.asarray(z, dtype=np.float64)
    G = np.empty_like(z)
    for j in range(z.shape[-1]):
        zc = z.astype(np.complex128)
        zc[..., j] += 1j * h
        G[..., j] = token_loss_np(zc, tau, gamma, beta, eps).imag / h
    return G


def linear_bruteforce_fd(XQ, XK, XV, eta, W0, b0, gamma, beta, eps, mb, h=1e-6):
    """Mini-batch TTT-Linear for one sequence where every gradient (with
    respect to W and b) comes from central differences of the loss; the
    output layer norm is plain NumPy. No analytic gradient at all."""
    XQ, XK, XV = (np.asarray(a, np.float64) for a in (XQ, XK, XV))
    W = np.array(W0, np.float64)
    b = np.array(b0, np.float64)
    L, d = XQ.shape
    O = np.zeros((L, d))

    def loss(Wm, bv, s):
        z = XK[s] @ Wm + bv
        return token_loss_np(z, XV[s] - XK[s], gamma, beta, eps)

    def ln(z):
        mu = z.mean()
        v = ((z - mu) ** 2).mean()
        return gamma * (z - mu) / np.sqrt(v + eps) + beta

    t0 = 0
    for n in chunk_schedule(L, mb):
        grads = []
        for s in range(t0, t0 + n):
            gW = np.zeros((d, d))
            gb = np.zeros(d)
            for i in range(d):
                for j in range(d):
                    Wp = W.copy(); Wp[i, j] += h
                    Wm = W.copy(); Wm[i, j] -= h
                    gW[i, j] = (loss(Wp, b, s) - loss(Wm, b, s)) / (2 * h)
            for j in range(d):
                bp = b.copy(); bp[j] += h
                bm = b.copy(); bm[j] -= h
                gb[j] = (loss(W, bp, s) - loss(W, bm, s)) / (2 * h)
            grads.append((gW, gb))
        for i, s in enumerate(range(t0, t0 + n)):
            W = W - eta[s] * grads[i][0]
            b = b - eta[s] * grads[i][1]
            O[s] = XQ[s] + ln(XQ[s] @ W + b)
        t0 += n
    return O, W, b
