"""fp64 gradients of the TTT-Linear and TTT-MLP inner loops -- TEST INFRASTRUCTURE ONLY.

Only the tests and the benchmark's CPU baseline may import this module; the
GPU path never does, and it shares nothing with the GPU path.

The forward below is the primal mini-batch recurrence (the definition: the
per-token update-then-apply rule of the damodev.csdn.net TTT deep-dive §3.1
with every token of a chunk taking its gradient at the chunk-start state,
§4.1-4.2, and the LN-residual output of the lryc.cn TTT article §2.1), written
with PyTorch CPU float64 tensor operations. Reverse-mode automatic
differentiation of

    loss = <dO, O> + <dW_out, W_L> + <db_out, b_L>

then gives, to rounding, the gradients a training step needs from this layer
(the deep-dive's §6 / §7.1 train the outer-loop parameters through the inner
loop): with respect to XQ, XK, XV, eta, W0, b0, gamma and beta.

The layer-norm L2 gradient G is written out (the same closed form as the C
oracle's ln_l2_bwd) so that autograd differentiates through it; the tests pin
that formula against autograd of the loss it is the gradient of, and the whole
forward against the C oracle.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

_F64 = torch.float64


def _t(a, grad: bool = False) -> torch.Tensor:
    return torch.tensor(np.asarray(a, dtype=np.float64), dtype=_F64, requires_grad=grad)


def ln(z: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float) -> torch.Tensor:
    """LN_{gamma,beta}(z) over the last axis, biased variance, eps inside the root."""
    mu = z.mean(-1, keepdim=True)
    var = ((z - mu) ** 2).mean(-1, keepdim=True)
    return gamma * (z - mu) / torch.sqrt(var + eps) + beta


def ln_l2_grad(z: torch.Tensor, tau: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor,
               eps: float) -> torch.Tensor:
    """G = d/dz 1/2 || LN_{gamma,beta}(z) - tau ||^2, row-wise (the deep-dive §4.2 step)."""
    mu = z.mean(-1, keepdim=True)
    sigma = torch.sqrt(((z - mu) ** 2).mean(-1, keepdim=True) + eps)
    xhat = (z - mu) / sigma
    ghat = gamma * (gamma * xhat + beta - tau)
    return (ghat - ghat.mean(-1, keepdim=True) - xhat * (ghat * xhat).mean(-1, keepdim=True)) / sigma


def linear_primal(XQ, XK, XV, eta, W0, b0, gamma, beta, eps: float, mb: int):
    """Primal forward on torch tensors. XQ, XK, XV [B,H,L,d]; eta [B,H,L];
    W0 [B,H,d,d]; b0 [B,H,d]; gamma, beta [H,d]. Returns O, W_L, b_L."""
    B, H, L, d = XQ.shape
    g = gamma[None, :, :]
    bt = beta[None, :, :]
    W, b = W0, b0
    outs = []
    for c0 in range(0, L, mb):
        sl = slice(c0, min(L, c0 + mb))
        xq, xk, xv, et = XQ[:, :, sl], XK[:, :, sl], XV[:, :, sl], eta[:, :, sl]
        # every token of the chunk takes its gradient at the chunk-start state
        Z = xk @ W + b[:, :, None, :]
        G = ln_l2_grad(Z, xv - xk, g[:, :, None, :], bt[:, :, None, :], eps)
        for t in range(xq.shape[2]):
            # update with token t, then apply to token t
            W = W - et[:, :, t, None, None] * xk[:, :, t, :, None] * G[:, :, t, None, :]
            b = b - et[:, :, t, None] * G[:, :, t, :]
            zb = (xq[:, :, t, None, :] @ W)[:, :, 0, :] + b
            outs.append(xq[:, :, t, :] + ln(zb, g, bt, eps))
    O = torch.stack(outs, 2) if outs else XQ * 0.0
    return O, W, b


def linear_backward(XQ, XK, XV, eta, W0, b0, gamma, beta, eps: float, mb: int, dO,
                    dW_out: Optional[np.ndarray] = None, db_out: Optional[np.ndarray] = None) -> dict:
    """Gradients of <dO, O> + <dW_out, W_L> + <db_out, b_L> (float64 NumPy).

    W0 and b0 are per sequence ([B,H,d,d], [B,H,d]); gamma and beta are per
    head ([H,d]), so their gradients are summed over the batch."""
    B, H, L, d = np.shape(XQ)
    W0 = np.broadcast_to(W0, (B, H, d, d))
    b0 = np.broadcast_to(b0, (B, H, d))
    names = ("XQ", "XK", "XV", "eta", "W0", "b0", "gamma", "beta")
    ts = [_t(a, True) for a in (XQ, XK, XV, eta, W0, b0, gamma, beta)]
    O, W, b = linear_primal(*ts, eps, mb)
    loss = (O * _t(dO)).sum()
    if dW_out is not None:
        loss = loss + (W * _t(dW_out)).sum()
    if db_out is not None:
        loss = loss + (b * _t(db_out)).sum()
    grads = torch.autograd.grad(loss, ts, allow_unused=True)
    out = {}
    for n, t, gr in zip(names, ts, grads):
        out["d" + n] = np.zeros(t.shape) if gr is None else gr.detach().numpy()
    out["O"] = O.detach().numpy()
    out["W"] = W.detach().numpy()
    out["b"] = b.detach().numpy()
    return out


def eta_gate_t(XK: torch.Tensor, theta: torch.Tensor, eta_base: float) -> torch.Tensor:
    """eta = eta_base * logistic(theta . x) per token with x := the head's key
    (the lryc.cn article §2.2 gate). XK [B,H,L,d]; theta [B,H,d] or [H,d]."""
    th = theta if theta.dim() == 3 else theta[None]
    s = (XK * th[:, :, None, :]).sum(-1)
    return eta_base / (1.0 + torch.exp(-s))


def eta_gate_backward(XK, theta_lr, eta_base: float, deta) -> dict:
    """Gradients of <deta, eta_gate(XK, theta_lr)>: dXK [B,H,L,d] (the gate's
    share only) and dtheta per sequence [B,H,d] (sum over B for the per-head
    parameter)."""
    B, H, L, d = np.shape(XK)
    xk = _t(XK, True)
    th = _t(np.broadcast_to(theta_lr, (B, H, d)), True)
    loss = (eta_gate_t(xk, th, eta_base) * _t(deta)).sum()
    gx, gt = torch.autograd.grad(loss, (xk, th), allow_unused=True)
    zero = lambda t: np.zeros(t.shape)
    return {"dXK": zero(xk) if gx is None else gx.detach().numpy(),
            "dtheta": zero(th) if gt is None else gt.detach().numpy()}


def linear_backward_gated(XQ, XK, XV, theta_lr, eta_base: float, W0, b0, gamma, beta,
                          eps: float, mb: int, dO, dW_out: Optional[np.ndarray] = None,
                          db_out: Optional[np.ndarray] = None) -> dict:
    """Gradients of <dO, O> + <dW_out, W_L> + <db_out, b_L> when eta comes from
    the gate: dXK includes the path through eta, and dtheta ([H,d], summed
    over the batch) replaces deta. Also returns O, W, b and the gated eta."""
    B, H, L, d = np.shape(XQ)
    W0 = np.broadcast_to(W0, (B, H, d, d))
    b0 = np.broadcast_to(b0, (B, H, d))
    names = ("XQ", "XK", "XV", "theta", "W0", "b0", "gamma", "beta")
    ts = [_t(a, True) for a in (XQ, XK, XV, theta_lr, W0, b0, gamma, beta)]
    eta = eta_gate_t(ts[1], ts[3], eta_base)
    O, W, b = linear_primal(ts[0], ts[1], ts[2], eta, *ts[4:], eps, mb)
    loss = (O * _t(dO)).sum()
    if dW_out is not None:
        loss = loss + (W * _t(dW_out)).sum()
    if db_out is not None:
        loss = loss + (b * _t(db_out)).sum()
    grads = torch.autograd.grad(loss, ts, allow_unused=True)
    out = {}
    for n, t, gr in zip(names, ts, grads):
        out["d" + n] = np.zeros(t.shape) if gr is None else gr.detach().numpy()
    out["O"] = O.detach().numpy()
    out["W"] = W.detach().numpy()
    out["b"] = b.detach().numpy()
    out["eta"] = eta.detach().numpy()
    return out


# ----------------------------------------------------------------------------
# TTT-MLP (the lryc.cn TTT article §2.1: d -> 4d -> d with exact GELU, the
# same LN-residual output; the same mini-batch rule as TTT-Linear)
# ----------------------------------------------------------------------------

_SQRT2 = 2.0 ** 0.5
_INV_SQRT_2PI = (2.0 * np.pi) ** -0.5


def gelu(z: torch.Tensor) -> torch.Tensor:
    """Exact GELU z Phi(z), Phi the standard normal CDF."""
    return 0.5 * z * (1.0 + torch.erf(z / _SQRT2))


def gelu_prime(z: torch.Tensor) -> torch.Tensor:
    """d/dz gelu(z) = Phi(z) + z phi(z), written out so that autograd can take
    its own derivative (the inner gradient G1 contains it)."""
    return 0.5 * (1.0 + torch.erf(z / _SQRT2)) + z * _INV_SQRT_2PI * torch.exp(-0.5 * z * z)


def mlp_primal(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps: float, mb: int):
    """Primal forward of TTT-MLP on torch tensors. XQ, XK, XV [B,H,L,d];
    eta [B,H,L]; W1 [B,H,d,4d]; b1 [B,H,4d]; W2 [B,H,4d,d]; b2 [B,H,d];
    gamma, beta [H,d]. Every token of a chunk takes its gradient of
    1/2 ||LN(gelu(k W1 + b1) W2 + b2) - (v - k)||^2 at the chunk-start state;
    the updates then apply one token at a time, and token t's output is
    q_t + LN(gelu(q_t W1_t + b1_t) W2_t + b2_t). Returns O, W1, b1, W2, b2."""
    B, H, L, d = XQ.shape
    g = gamma[None, :, :]
    bt = beta[None, :, :]
    outs = []
    for c0 in range(0, L, mb):
        sl = slice(c0, min(L, c0 + mb))
        xq, xk, xv, et = XQ[:, :, sl], XK[:, :, sl], XV[:, :, sl], eta[:, :, sl]
        Z1 = xk @ W1 + b1[:, :, None, :]
        A = gelu(Z1)
        Z2 = A @ W2 + b2[:, :, None, :]
        G2 = ln_l2_grad(Z2, xv - xk, g[:, :, None, :], bt[:, :, None, :], eps)
        G1 = (G2 @ W2.transpose(-1, -2)) * gelu_prime(Z1)
        for t in range(xq.shape[2]):
            e = et[:, :, t]
            W1 = W1 - e[..., None, None] * xk[:, :, t, :, None] * G1[:, :, t, None, :]
            b1 = b1 - e[..., None] * G1[:, :, t, :]
            W2 = W2 - e[..., None, None] * A[:, :, t, :, None] * G2[:, :, t, None, :]
            b2 = b2 - e[..., None] * G2[:, :, t, :]
            a = gelu((xq[:, :, t, None, :] @ W1)[:, :, 0, :] + b1)
            zb = (a[:, :, None, :] @ W2)[:, :, 0, :] + b2
            outs.append(xq[:, :, t, :] + ln(zb, g, bt, eps))
    O = torch.stack(outs, 2) if outs else XQ * 0.0
    return O, W1, b1, W2, b2


def mlp_backward(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps: float, mb: int, dO,
                 dW1_out=None, db1_out=None, dW2_out=None, db2_out=None) -> dict:
    """Gradients of <dO, O> + <dW1_out, W1_L> + <db1_out, b1_L>
    + <dW2_out, W2_L> + <db2_out, b2_L> (float64 NumPy) with respect to XQ,
    XK, XV, eta, the initial state W1, b1, W2, b2 (per sequence) and gamma,
    beta (per head, summed over the batch). Also returns the forward."""
    B, H, L, d = np.shape(XQ)
    m = 4 * d
    W1 = np.broadcast_to(W1, (B, H, d, m))
    b1 = np.broadcast_to(b1, (B, H, m))
    W2 = np.broadcast_to(W2, (B, H, m, d))
    b2 = np.broadcast_to(b2, (B, H, d))
    names = ("XQ", "XK", "XV", "eta", "W1", "b1", "W2", "b2", "gamma", "beta")
    ts = [_t(a, True) for a in (XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta)]
    O, W1L, b1L, W2L, b2L = mlp_primal(*ts, eps, mb)
    loss = (O * _t(dO)).sum()
    for fin, adj in ((W1L, dW1_out), (b1L, db1_out), (W2L, dW2_out), (b2L, db2_out)):
        if adj is not None:
            loss = loss + (fin * _t(adj)).sum()
    grads = torch.autograd.grad(loss, ts, allow_unused=True)
    out = {}
    for n, t, gr in zip(names, ts, grads):
        out["d" + n] = np.zeros(t.shape) if gr is None else gr.detach().numpy()
    out["O"] = O.detach().numpy()
    out["W1"], out["b1"] = W1L.detach().numpy(), b1L.detach().numpy()
    out["W2"], out["b2"] = W2L.detach().numpy(), b2L.detach().numpy()
    return out
