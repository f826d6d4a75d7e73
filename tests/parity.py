"""Helpers for GPU-vs-oracle parity tests: move seeded inputs to the device,
run the HIP path through the C ABI binding and the fp64 oracle on the same
values, and measure the error.

Error metric (per output tensor): for each (n,h) slice, max|got - ref| /
max|ref|, then the maximum over slices. Elementwise ratios are undefined near
zero, so the slice maximum is the scale.
Tolerances: 1e-4 for fp32 storage, 2e-2 for bf16 inputs with fp32 state.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from test_sequence_layer_ttt_amd import ttt

TOL = {"f32": 1e-4, "bf16": 2e-2}


def max_rel(got, ref, nseq: int) -> float:
    g = np.asarray(got, np.float64).reshape(nseq, -1)
    r = np.asarray(ref, np.float64).reshape(nseq, -1)
    if g.size == 0:
        return 0.0
    num = np.abs(g - r).max(1)
    den = np.maximum(np.abs(r).max(1), 1e-30)
    return float((num / den).max())


def elem_rel(got, ref, nseq: int) -> float:
    """Secondary log of the per-output metric: the largest elementwise ratio
    |got - ref| / max(|ref|, 1e-3 max|ref|), the floor taken per (n,h) slice
    (elementwise ratios are undefined near zero without one)."""
    g = np.asarray(got, np.float64).reshape(nseq, -1)
    r = np.asarray(ref, np.float64).reshape(nseq, -1)
    if g.size == 0:
        return 0.0
    floor = np.maximum(1e-3 * np.abs(r).max(1, keepdims=True), 1e-30)
    return float((np.abs(g - r) / np.maximum(np.abs(r), floor)).max())


def elem_errors(got, ref, nseq, names):
    return {n: elem_rel(g, r, nseq) for n, g, r in zip(names, got, ref)}


def dev(a, dtype=torch.float32, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(dtype)


def io_dtype(io: str):
    return torch.bfloat16 if io == "bf16" else torch.float32


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def linear_gpu(x, mb=None, W0=None, b0=None, stream=None):
    """Run ttt_linear_forward on inputs `x` (gen.LinearInputs). Returns numpy
    (O, W_out, b_out)."""
    dt = io_dtype(x.io)
    W0 = x.W0 if W0 is None else W0
    b0 = x.b0 if b0 is None else b0
    if x.eta is None:  # gated inputs: the kernel evaluates the gate
        O, Wo, bo = ttt.ttt_linear_forward_gated(dev(x.XQ, dt), dev(x.XK, dt), dev(x.XV, dt),
                                                 dev(x.theta_lr), x.eta_base, dev(W0), dev(b0),
                                                 dev(x.gamma), dev(x.beta), mb=mb or x.mb,
                                                 ln_eps=x.eps, stream=stream)
    else:
        O, Wo, bo = ttt.ttt_linear_forward(dev(x.XQ, dt), dev(x.XK, dt), dev(x.XV, dt),
                                           dev(x.eta), dev(W0), dev(b0), dev(x.gamma),
                                           dev(x.beta), mb=mb or x.mb, ln_eps=x.eps,
                                           stream=stream)
    torch.cuda.synchronize()
    return to_np(O), to_np(Wo), to_np(bo)


def linear_oracle(x, mb=None, W0=None, b0=None, schedule=None):
    W0 = x.W0 if W0 is None else W0
    b0 = x.b0 if b0 is None else b0
    eta = x.eta if x.eta is not None else oracle.eta_gate(x.XK, x.theta_lr, x.eta_base)
    return oracle.linear_forward(x.XQ, x.XK, x.XV, eta, W0, b0, x.gamma, x.beta, x.eps,
                                 mb=mb or x.mb, w0_batched=np.ndim(W0) == 4, schedule=schedule)


def mlp_gpu(x, mb=None):
    dt = io_dtype(x.io)
    out = ttt.ttt_mlp_forward(dev(x.XQ, dt), dev(x.XK, dt), dev(x.XV, dt), dev(x.eta),
                              dev(x.W1), dev(x.b1), dev(x.W2), dev(x.b2), dev(x.gamma),
                              dev(x.beta), mb=mb or x.mb, ln_eps=x.eps)
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in out)


def mlp_oracle(x, mb=None):
    return oracle.mlp_forward(x.XQ, x.XK, x.XV, x.eta, x.W1, x.b1, x.W2, x.b2, x.gamma,
                              x.beta, x.eps, mb=mb or x.mb)


def errors(got, ref, nseq, names):
    return {n: max_rel(g, r, nseq) for n, g, r in zip(names, got, ref)}
