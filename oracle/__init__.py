"""fp64 CPU oracle for the TTT inner loop -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package. The GPU path never imports it, and it imports nothing
from the GPU path. Inputs are NumPy arrays (any float dtype; widened to
float64 here); outputs are float64.

Citation key: [D] damodev.csdn.net TTT deep-dive; [Y] lryc.cn "测试时学习
（TTT）" article; [X] xiaohu.ai TTT summary.

The functions compute the mini-batch TTT recurrence of [D] §3.1 / §4.1-4.2
with the LN-residual output of [Y] §2.1, in primal form (the definition), and
the dual form of [D] §4.2 / [X] (used to pin the primal form). Chunks are
aligned at t = 0; `schedule` lists the chunk lengths (default: mb-sized
chunks with a partial last chunk when L % mb != 0).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libttt_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build_oracle()
    lib = ctypes.CDLL(_LIB_PATH)
    lin_args = [ctypes.c_int] * 5 + [_I, ctypes.c_double] + [_D] * 6 + [ctypes.c_int] \
        + [_D] * 2 + [_D] * 3 + [ctypes.c_int]
    for name in ("oracle_linear_forward", "oracle_linear_dual"):
        f = getattr(lib, name)
        f.argtypes = lin_args
        f.restype = ctypes.c_int
    mlp_args = [ctypes.c_int] * 5 + [_I, ctypes.c_double] + [_D] * 8 + [ctypes.c_int] \
        + [_D] * 2 + [_D] * 5 + [ctypes.c_int]
    for name in ("oracle_mlp_forward", "oracle_mlp_dual"):
        f = getattr(lib, name)
        f.argtypes = mlp_args
        f.restype = ctypes.c_int
    lib.oracle_linear_forward_opts.argtypes = [ctypes.c_int] * 5 + [_I, ctypes.c_double] \
        + [_D] * 6 + [ctypes.c_int] + [_D] * 2 + [ctypes.c_int, ctypes.c_double] + [_D] * 3 \
        + [ctypes.c_int]
    lib.oracle_linear_forward_opts.restype = ctypes.c_int
    lib.oracle_mlp_forward_opts.argtypes = [ctypes.c_int] * 5 + [_I, ctypes.c_double] \
        + [_D] * 8 + [ctypes.c_int] + [_D] * 2 + [ctypes.c_int, ctypes.c_double] + [_D] * 5 \
        + [ctypes.c_int]
    lib.oracle_mlp_forward_opts.restype = ctypes.c_int
    lib.oracle_ln_l2_bwd.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, _D, _D,
                                     ctypes.c_double, _D]
    lib.oracle_ln_l2_bwd.restype = None
    lib.oracle_ln_fwd.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, _D, ctypes.c_double, _D]
    lib.oracle_qkv_project.argtypes = [ctypes.c_int] * 5 + [_D] * 5
    lib.oracle_qkv_project_at.argtypes = [ctypes.c_int] * 5 + [_D, _D, ctypes.c_int, _I, _D]
    lib.oracle_ln_fwd.restype = None
    lib.oracle_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


def default_threads() -> int:
    return max(1, os.cpu_count() or 1)


def chunk_schedule(L: int, mb: int) -> list:
    """Chunks of mb tokens aligned at t = 0; the last may be partial."""
    s = [mb] * (L // mb)
    if L % mb:
        s.append(L % mb)
    return s


def _sched(L, mb, schedule):
    s = list(schedule) if schedule is not None else chunk_schedule(L, mb)
    arr = np.ascontiguousarray(s, dtype=np.int32)
    return arr, len(s)


def ln_l2_bwd(Z, target, gamma, beta, eps: float) -> np.ndarray:
    """dl/dZ of l = 1/2 ||LN(Z) - target||^2 row-wise. Z, target [rows, d]."""
    lib = _load()
    Z = _f64(Z)
    rows, d = Z.shape
    T = _f64(target)
    g = _f64(gamma)
    b = _f64(beta)
    G = np.empty_like(Z)
    lib.oracle_ln_l2_bwd(rows, d, _p(Z), _p(T), _p(g), _p(b), float(eps), _p(G))
    return G


def ln_fwd(Z, gamma, beta, eps: float) -> np.ndarray:
    lib = _load()
    Z = _f64(Z)
    rows, d = Z.shape
    Y = np.empty_like(Z)
    lib.oracle_ln_fwd(rows, d, _p(Z), _p(_f64(gamma)), _p(_f64(beta)), float(eps), _p(Y))
    return Y


def linear_forward(XQ, XK, XV, eta, W0, b0, gamma, beta, eps: float, mb: int = 16,
                   schedule: Optional[Sequence[int]] = None, w0_batched: bool = False,
                   dual: bool = False, nthreads: Optional[int] = None):
    """TTT-Linear over [B,H,L,d] inputs. Returns (O, W_out, b_out) in float64.

    W0 is [H,d,d] (shared over B) unless w0_batched, then [B,H,d,d]; b0 is
    [H,d] or [B,H,d] likewise.
    """
    lib = _load()
    XQ, XK, XV, eta = _f64(XQ), _f64(XK), _f64(XV), _f64(eta)
    B, H, L, d = XQ.shape
    W0, b0, gamma, beta = _f64(W0), _f64(b0), _f64(gamma), _f64(beta)
    sched, nch = _sched(L, mb, schedule)
    O = np.zeros((B, H, L, d))
    Wo = np.zeros((B, H, d, d))
    bo = np.zeros((B, H, d))
    f = lib.oracle_linear_dual if dual else lib.oracle_linear_forward
    st = f(B, H, L, d, nch, sched.ctypes.data_as(_I), float(eps), _p(XQ), _p(XK), _p(XV),
           _p(eta), _p(W0), _p(b0), int(bool(w0_batched)), _p(gamma), _p(beta), _p(O),
           _p(Wo), _p(bo), nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle linear returned {st}")
    return O, Wo, bo


def linear_forward_opts(XQ, XK, XV, eta, W0, b0, gamma, beta, eps: float, mb: int = 16,
                        loss: str = "mse", weight_decay: float = 0.0,
                        schedule: Optional[Sequence[int]] = None, w0_batched: bool = False,
                        nthreads: Optional[int] = None):
    """TTT-Linear with the Modular-TTT options (primal form): loss "mse" (the
    squared reconstruction error of linear_forward) or "inner_product"
    (-< XK + LN(XK W + b), XV > per token), and weight decay lambda/2 ||W||^2
    added to every token's loss (W only). Returns (O, W_out, b_out)."""
    lib = _load()
    XQ, XK, XV, eta = _f64(XQ), _f64(XK), _f64(XV), _f64(eta)
    B, H, L, d = XQ.shape
    W0, b0, gamma, beta = _f64(W0), _f64(b0), _f64(gamma), _f64(beta)
    sched, nch = _sched(L, mb, schedule)
    O = np.zeros((B, H, L, d))
    Wo = np.zeros((B, H, d, d))
    bo = np.zeros((B, H, d))
    code = {"mse": 0, "inner_product": 1}[loss]
    st = lib.oracle_linear_forward_opts(B, H, L, d, nch, sched.ctypes.data_as(_I), float(eps),
                                        _p(XQ), _p(XK), _p(XV), _p(eta), _p(W0), _p(b0),
                                        int(bool(w0_batched)), _p(gamma), _p(beta), code,
                                        float(weight_decay), _p(O), _p(Wo), _p(bo),
                                        nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle linear (options) returned {st}")
    return O, Wo, bo


def mlp_forward(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps: float, mb: int = 16,
                schedule: Optional[Sequence[int]] = None, w0_batched: bool = False,
                dual: bool = False, nthreads: Optional[int] = None):
    """TTT-MLP (hidden 4d, exact GELU). Returns (O, W1, b1, W2, b2) in float64."""
    lib = _load()
    XQ, XK, XV, eta = _f64(XQ), _f64(XK), _f64(XV), _f64(eta)
    B, H, L, d = XQ.shape
    m = 4 * d
    W1, b1, W2, b2 = _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    gamma, beta = _f64(gamma), _f64(beta)
    sched, nch = _sched(L, mb, schedule)
    O = np.zeros((B, H, L, d))
    W1o = np.zeros((B, H, d, m))
    b1o = np.zeros((B, H, m))
    W2o = np.zeros((B, H, m, d))
    b2o = np.zeros((B, H, d))
    f = lib.oracle_mlp_dual if dual else lib.oracle_mlp_forward
    st = f(B, H, L, d, nch, sched.ctypes.data_as(_I), float(eps), _p(XQ), _p(XK), _p(XV),
           _p(eta), _p(W1), _p(b1), _p(W2), _p(b2), int(bool(w0_batched)), _p(gamma),
           _p(beta), _p(O), _p(W1o), _p(b1o), _p(W2o), _p(b2o), nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle mlp returned {st}")
    return O, W1o, b1o, W2o, b2o


def mlp_forward_opts(XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta, eps: float, mb: int = 16,
                     loss: str = "mse", weight_decay: float = 0.0,
                     schedule: Optional[Sequence[int]] = None, w0_batched: bool = False,
                     nthreads: Optional[int] = None):
    """TTT-MLP with the Modular-TTT options (primal form): loss "mse" (as
    mlp_forward) or "inner_product" (-< XK + LN(f_res(XK)), XV > per token),
    and weight decay lambda/2 (||W1||^2 + ||W2||^2) added to every token's
    loss (not the biases). Returns (O, W1, b1, W2, b2) in float64."""
    lib = _load()
    XQ, XK, XV, eta = _f64(XQ), _f64(XK), _f64(XV), _f64(eta)
    B, H, L, d = XQ.shape
    m = 4 * d
    W1, b1, W2, b2 = _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    gamma, beta = _f64(gamma), _f64(beta)
    sched, nch = _sched(L, mb, schedule)
    O = np.zeros((B, H, L, d))
    W1o = np.zeros((B, H, d, m))
    b1o = np.zeros((B, H, m))
    W2o = np.zeros((B, H, m, d))
    b2o = np.zeros((B, H, d))
    code = {"mse": 0, "inner_product": 1}[loss]
    st = lib.oracle_mlp_forward_opts(B, H, L, d, nch, sched.ctypes.data_as(_I), float(eps),
                                     _p(XQ), _p(XK), _p(XV), _p(eta), _p(W1), _p(b1), _p(W2),
                                     _p(b2), int(bool(w0_batched)), _p(gamma), _p(beta), code,
                                     float(weight_decay), _p(O), _p(W1o), _p(b1o), _p(W2o),
                                     _p(b2o), nthreads or default_threads())
    if st != 0:
        raise RuntimeError(f"oracle mlp (options) returned {st}")
    return O, W1o, b1o, W2o, b2o


def decode_step(xq, xk, xv, eta, W, b, gamma, beta, eps: float, nthreads: Optional[int] = None):
    """One single-token step (b = 1) for a batch of independent states.

    xq/xk/xv [B,H,d], eta [B,H], W [B,H,d,d], b [B,H,d]. Returns (o, W', b').
    """
    xq = _f64(xq)
    B, H, d = xq.shape
    O, Wn, bn = linear_forward(xq.reshape(B, H, 1, d), _f64(xk).reshape(B, H, 1, d),
                               _f64(xv).reshape(B, H, 1, d), _f64(eta).reshape(B, H, 1),
                               W, b, gamma, beta, eps, mb=1, w0_batched=True,
                               nthreads=nthreads)
    return O.reshape(B, H, d), Wn, bn


def eta_gate(XK, theta_lr, eta_base: float) -> np.ndarray:
    """Per-token learning rate of the lryc.cn article §2.2: eta = eta_base
    times the logistic sigmoid of theta_lr . x, per token and per head.

    The article leaves the gate input x open; this oracle takes x := that
    head's key XK_t. XK [B,H,L,d]; theta_lr [H,d]. Returns eta [B,H,L] in
    float64 (exp overflow for a very negative theta . x gives eta = 0)."""
    XK, th = _f64(XK), _f64(theta_lr)
    B, H, L, d = XK.shape
    eta = np.empty((B, H, L))
    with np.errstate(over="ignore"):
        for h in range(H):
            s = XK[:, h] @ th[h]                       # theta_lr . x per token
            eta[:, h] = float(eta_base) / (1.0 + np.exp(-s))
    return eta


def linear_forward_gated(XQ, XK, XV, theta_lr, eta_base: float, W0, b0, gamma, beta,
                         eps: float, mb: int = 16, **kw):
    """TTT-Linear with eta from the gate (eta_gate), then linear_forward."""
    return linear_forward(XQ, XK, XV, eta_gate(XK, theta_lr, eta_base), W0, b0, gamma,
                          beta, eps, mb=mb, **kw)


def qkv_project(X, theta, H: int):
    """Key, value and query views of the layer input ([Y] §2.2 projections
    theta_Q, theta_K, theta_V; [D] §4.2 inputs XQ, XK, XV): with theta
    [3, H*d, d_model] stored output-major, XQ[b,h,t,j] = sum_k X[b,t,k]
    theta[0][h*d+j][k] (XK: theta[1], XV: theta[2]). X [B,L,d_model].
    Returns (XQ, XK, XV), each [B,H,L,d] in float64."""
    X, th = _f64(X), _f64(theta)
    B, L, dm = X.shape
    if th.shape[0] != 3 or th.shape[2] != dm or th.shape[1] % H:
        raise ValueError("theta must be [3, H*d, d_model]")
    d = th.shape[1] // H
    outs = [np.empty((B, H, L, d)) for _ in range(3)]
    st = _load().oracle_qkv_project(B, L, dm, H, d, _p(X), _p(th), *(_p(o) for o in outs))
    if st:
        raise ValueError(f"oracle_qkv_project: error {st}")
    return tuple(outs)


def qkv_project_at(X, theta, H: int, idx) -> np.ndarray:
    """qkv_project at chosen outputs only: idx [n,5] rows (view, b, h, t, j)
    with view 0 = XQ, 1 = XK, 2 = XV. Returns the n values in float64."""
    X, th = _f64(X), _f64(theta)
    B, L, dm = X.shape
    d = th.shape[1] // H
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(-1, 5))
    out = np.empty(idx.shape[0])
    st = _load().oracle_qkv_project_at(B, L, dm, H, d, _p(X), _p(th), idx.shape[0],
                                       idx.ctypes.data_as(_I), _p(out))
    if st:
        raise ValueError(f"oracle_qkv_project_at: error {st}")
    return out
