"""Seeded synthetic inputs for the TTT inner loop.

This module is shared by the oracle-side tests and the GPU path. It only
*draws* inputs; it holds none of the inner loop's arithmetic (no loss, no
gradient, no state update, no layer norm).

Sources for the shapes and distributions:
  * fast-weight init W ~ N(0, 0.02^2), b = 0, per head  -- damodev.csdn.net,
    "TTT-LM" deep-dive, section 4.3 (TTTLinear initialisation excerpt).
  * per-token learning rate eta(x) = eta_base * sigmoid(theta_lr . x)  --
    lryc.cn article, section 2.2 (dynamic learning-rate formula). Where a
    workload gates eta, only theta_lr and eta_base are drawn here; the
    oracle and the kernels evaluate the gate. Elsewhere eta itself is drawn
    from the distribution the gate gives for a standard-normal
    pre-activation: (1/d) times a logit-normal variate.
  * mini-batch size b = 16  -- lryc.cn article, section 2.4.
  * TTT-MLP hidden width 4d with GELU  -- lryc.cn article, section 2.1.

The pages train on Pile / Books3 activations; those are not available, so
standard-normal draws of the same shapes stand in for them.

Conventions
  * NumPy ``default_rng(seed)`` (PCG64), ``standard_normal`` in float64,
    cast to float32, then (for bf16 workloads) rounded to bfloat16 with
    round-to-nearest-even. Float arrays returned here always hold the exact
    value the device sees (bf16 values widened to float32).
  * Fixed draw order: XQ, XK, XV, eta logits (or theta_lr), W0 (or W1, W2),
    then decode XQ, XK, XV, eta logits.
  * Layouts: XQ/XK/XV [B,H,L,d]; eta [B,H,L]; W0 [H,d,d] (row i = input
    feature, column j = output feature); b0 [H,d]; gamma/beta [H,d].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

LN_EPS = 1e-6
MINI_BATCH = 16


# ----------------------------------------------------------------------------
# bfloat16 helpers (storage format only)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (round to nearest, ties to even); return the
    16-bit patterns as uint16. Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


def _normal_f32(rng: np.random.Generator, shape, scale: float = 1.0,
                block: int = 1 << 24) -> np.ndarray:
    """Draw float64 standard normals in blocks (same stream as one big draw),
    scale, and cast to float32 without holding the whole float64 array."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, block):
        e = min(n, s + block)
        out[s:e] = (rng.standard_normal(e - s) * scale).astype(np.float32)
    return out.reshape(shape)


def _logit_normal64(z: np.ndarray) -> np.ndarray:
    """Map standard-normal draws z to logit-normal variates in (0, 1)."""
    return 1.0 / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------
# Input bundles
# ----------------------------------------------------------------------------
@dataclass
class LinearInputs:
    B: int
    H: int
    L: int
    d: int
    io: str                      # "f32" or "bf16": storage type of XQ/XK/XV/O
    XQ: np.ndarray               # [B,H,L,d] float32 (exact device values)
    XK: np.ndarray
    XV: np.ndarray
    eta: Optional[np.ndarray]    # [B,H,L] float32; None when the gate below gives it
    W0: np.ndarray               # [H,d,d] float32 (broadcast over B)
    b0: np.ndarray               # [H,d]   float32
    gamma: np.ndarray            # [H,d]   float32
    beta: np.ndarray             # [H,d]   float32
    eps: float = LN_EPS
    mb: int = MINI_BATCH
    theta_lr: Optional[np.ndarray] = None  # [H,d] float32 gate weights (gated inputs)
    eta_base: float = 0.0                  # gate scale (gated inputs)


@dataclass
class MLPInputs:
    B: int
    H: int
    L: int
    d: int
    io: str
    XQ: np.ndarray
    XK: np.ndarray
    XV: np.ndarray
    eta: np.ndarray
    W1: np.ndarray               # [H,d,4d]
    b1: np.ndarray               # [H,4d]
    W2: np.ndarray               # [H,4d,d]
    b2: np.ndarray               # [H,d]
    gamma: np.ndarray
    beta: np.ndarray
    eps: float = LN_EPS
    mb: int = MINI_BATCH


@dataclass
class DecodeInputs:
    steps: int
    B: int                       # independent sequences
    H: int
    d: int
    io: str
    XQ: np.ndarray               # [steps,B,H,d] (step-major)
    XK: np.ndarray
    XV: np.ndarray
    eta: np.ndarray              # [steps,B,H]


def _finish_io(x: np.ndarray, io: str) -> np.ndarray:
    if io == "bf16":
        return round_bf16(x)
    if io == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"unknown io dtype {io!r}")


def _rms_normalise(x32: np.ndarray) -> np.ndarray:
    """x / sqrt(mean_d x^2) per (n,h,t) row, computed in float64."""
    x = x32.astype(np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    return (x / r).astype(np.float32)


def _eta_from_logits(rng, shape, d) -> np.ndarray:
    logits = rng.standard_normal(int(np.prod(shape))).reshape(shape)
    return ((1.0 / d) * _logit_normal64(logits)).astype(np.float32)


def make_linear(seed: int, B: int, H: int, L: int, d: int, io: str = "bf16",
                rms_norm: bool = False, gate: str = "logits",
                ln_random: bool = False, w_std: float = 0.02,
                b_random: bool = False) -> LinearInputs:
    """TTT-Linear inputs.

    gate="logits": eta = (1/d) * logit-normal draw per token.
    gate="theta":  eta is left to the gate: theta_lr ~ N(0, 0.02^2) of shape
                   [H,d] and eta_base = 1/d are drawn/set here, eta = None.
    ln_random:     gamma ~ 1 + N(0,0.1^2), beta ~ N(0,0.1^2) (drawn last).
    b_random:      b0 ~ N(0, 0.02^2) instead of zeros (drawn last).
    """
    rng = np.random.default_rng(seed)
    shp = (B, H, L, d)
    XQ = _normal_f32(rng, shp)
    XK = _normal_f32(rng, shp)
    XV = _normal_f32(rng, shp)
    if rms_norm:
        XQ, XK, XV = (_rms_normalise(a) for a in (XQ, XK, XV))
    XQ, XK, XV = (_finish_io(a, io) for a in (XQ, XK, XV))
    if gate == "logits":
        eta = _eta_from_logits(rng, (B, H, L), d)
    elif gate == "theta":
        theta = (rng.standard_normal(H * d).reshape(H, d) * 0.02).astype(np.float32)
        eta = None
    else:
        raise ValueError(gate)
    W0 = (rng.standard_normal(H * d * d) * w_std).reshape(H, d, d).astype(np.float32)
    b0 = np.zeros((H, d), np.float32)
    gamma = np.ones((H, d), np.float32)
    beta = np.zeros((H, d), np.float32)
    if ln_random:
        gamma = (1.0 + 0.1 * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
        beta = (0.1 * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
    if b_random:
        b0 = (w_std * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
    x = LinearInputs(B, H, L, d, io, XQ, XK, XV, eta, W0, b0, gamma, beta)
    if gate == "theta":
        x.theta_lr, x.eta_base = theta, 1.0 / d
    return x


def make_mlp(seed: int, B: int, H: int, L: int, d: int, io: str = "bf16",
             ln_random: bool = False, w_std: float = 0.02,
             b_random: bool = False) -> MLPInputs:
    """TTT-MLP inputs: hidden width 4d, W1 [H,d,4d], W2 [H,4d,d]."""
    rng = np.random.default_rng(seed)
    m = 4 * d
    shp = (B, H, L, d)
    XQ = _finish_io(_normal_f32(rng, shp), io)
    XK = _finish_io(_normal_f32(rng, shp), io)
    XV = _finish_io(_normal_f32(rng, shp), io)
    eta = _eta_from_logits(rng, (B, H, L), d)
    W1 = (rng.standard_normal(H * d * m) * w_std).reshape(H, d, m).astype(np.float32)
    W2 = (rng.standard_normal(H * m * d) * w_std).reshape(H, m, d).astype(np.float32)
    b1 = np.zeros((H, m), np.float32)
    b2 = np.zeros((H, d), np.float32)
    gamma = np.ones((H, d), np.float32)
    beta = np.zeros((H, d), np.float32)
    if ln_random:
        gamma = (1.0 + 0.1 * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
        beta = (0.1 * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
    if b_random:
        b1 = (w_std * rng.standard_normal(H * m)).reshape(H, m).astype(np.float32)
        b2 = (w_std * rng.standard_normal(H * d)).reshape(H, d).astype(np.float32)
    return MLPInputs(B, H, L, d, io, XQ, XK, XV, eta, W1, b1, W2, b2, gamma, beta)


def make_decode(rng: np.random.Generator, steps: int, B: int, H: int, d: int,
                io: str = "bf16") -> DecodeInputs:
    """Decode-step inputs, step-major, drawn from an existing stream."""
    shp = (steps, B, H, d)
    XQ = _finish_io(_normal_f32(rng, shp), io)
    XK = _finish_io(_normal_f32(rng, shp), io)
    XV = _finish_io(_normal_f32(rng, shp), io)
    eta = _eta_from_logits(rng, (steps, B, H), d)
    return DecodeInputs(steps, B, H, d, io, XQ, XK, XV, eta)


# ----------------------------------------------------------------------------
# The five workloads (seed = workload number)
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    num: int
    name: str
    kind: str                    # "linear" | "mlp" | "long+decode"
    B: int
    H: int
    L: int
    d: int
    io: str
    rms_norm: bool = False
    gate: str = "logits"
    decode_steps: int = 0
    decode_B: int = 0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(1, "ttt_linear_fp32_B1_H1_L64_d16", "linear", 1, 1, 64, 16, "f32",
                gate="theta"),
    2: Workload(2, "ttt_linear_bf16_B4_H12_L2048_d64_rms", "linear", 4, 12, 2048, 64,
                "bf16", rms_norm=True),
    3: Workload(3, "ttt_linear_bf16_B2_H32_L8192_d64", "linear", 2, 32, 8192, 64, "bf16"),
    4: Workload(4, "ttt_mlp_bf16_B2_H12_L8192_d64", "mlp", 2, 12, 8192, 64, "bf16"),
    5: Workload(5, "ttt_linear_bf16_B1_H32_L32768_d64+decode64x1024", "long+decode",
                1, 32, 32768, 64, "bf16", decode_steps=1024, decode_B=64),
}


def make_workload(num: int, L: Optional[int] = None, B: Optional[int] = None,
                  H: Optional[int] = None, decode_steps: Optional[int] = None):
    """Inputs of workload `num` (seed = num). L/B/H/decode_steps may shrink
    the shape while keeping the distribution (for oracle-sized tests).

    Returns LinearInputs / MLPInputs, or for workload 5 a tuple
    (LinearInputs prefill, DecodeInputs decode) drawn from one stream.
    """
    w = WORKLOADS[num]
    B = w.B if B is None else B
    H = w.H if H is None else H
    L = w.L if L is None else L
    if w.kind == "mlp":
        return make_mlp(num, B, H, L, w.d, w.io)
    if w.kind == "linear":
        return make_linear(num, B, H, L, w.d, w.io, rms_norm=w.rms_norm, gate=w.gate)
    # long context + decode: prefill then decode draws continue the stream.
    rng = np.random.default_rng(num)
    shp = (B, H, L, w.d)
    XQ = _finish_io(_normal_f32(rng, shp), w.io)
    XK = _finish_io(_normal_f32(rng, shp), w.io)
    XV = _finish_io(_normal_f32(rng, shp), w.io)
    eta = _eta_from_logits(rng, (B, H, L), w.d)
    W0 = (rng.standard_normal(H * w.d * w.d) * 0.02).reshape(H, w.d, w.d).astype(np.float32)
    pre = LinearInputs(B, H, L, w.d, w.io, XQ, XK, XV, eta, W0,
                       np.zeros((H, w.d), np.float32), np.ones((H, w.d), np.float32),
                       np.zeros((H, w.d), np.float32))
    steps = w.decode_steps if decode_steps is None else decode_steps
    dec = make_decode(rng, steps, w.decode_B, H, w.d, w.io)
    return pre, dec


def head_tokens(num: int) -> int:
    w = WORKLOADS[num]
    return w.B * w.H * w.L


# ----------------------------------------------------------------------------
# Layer input and projections (the views XQ, XK, XV are made from X)
# ----------------------------------------------------------------------------
@dataclass
class ProjInputs:
    B: int
    L: int
    dm: int                      # model width d_model
    H: int
    d: int
    X: np.ndarray                # [B, L, dm], bf16 values widened to float32
    theta: np.ndarray            # [3, H*d, dm]: theta_Q, theta_K, theta_V (output-major)


def make_proj(seed: int, B: int, L: int, dm: int, H: int, d: int) -> ProjInputs:
    """Layer input X ~ N(0, 1) and the three projections theta ~ N(0, 0.02^2)
    (the initialisation scale of the damodev deep-dive, section 4.3, stands in
    for trained outer-loop weights), both rounded to bfloat16. Draw order: X,
    then theta_Q, theta_K, theta_V."""
    rng = np.random.default_rng(seed)
    X = round_bf16(_normal_f32(rng, (B, L, dm)))
    theta = round_bf16(_normal_f32(rng, (3, H * d, dm), 0.02))
    return ProjInputs(B, L, dm, H, d, X, theta)


def make_proj_workload(num: int, L: Optional[int] = None, B: Optional[int] = None) -> ProjInputs:
    """Projection inputs at a Linear workload's shape: model width H*d (the
    configs name it: 768 for workload 2, 2048 for workload 3). Seed 100 + num."""
    w = WORKLOADS[num]
    return make_proj(100 + num, w.B if B is None else B, w.L if L is None else L, w.H * w.d, w.H, w.d)
