"""GPU parity on the layer norm's edge cases: rows whose mean is large against
their spread, and rows of constant value.

The layer norm is the one inside the LN-residual output f(x) = x + LN(f_res(x))
(lryc.cn TTT article, §2.1) and the fused LN + L2 backward of the inner loss
(damodev.csdn.net TTT deep-dive, §4.2). Its statistics must not come from
E[z^2] - mean(z)^2 in fp32: with a row mean m and spread s that formula loses
about (m / s)^2 * 2^-24 of the variance. The gradient rows sum to zero, so an
offset in b0 (or in W0's row means) stays in z along the whole sequence.

Cases: b0 = c 1 + N(0, 0.02^2) with c in {10, 100}; W0 with per-row offsets;
W0 = 0 with a constant b0 (every row of z constant in the first chunk: zero
variance, the 1/sqrt(eps) scale). Besides O, W_out and b_out, the tests compare
the state's change (W_out - W0, b_out - b0), whose scale a large offset would
otherwise hide. Tolerances: 1e-4 for fp32 storage, 2e-2 for bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu


def _report(tag, err):
    print(f"[ln-edge] {tag}: " + " ".join(f"{k}={v:.3e}" for k, v in err.items()), flush=True)


def _state_errors(got, ref, W0, b0, nseq):
    """Errors of O, W_out, b_out and of the state changes W_out - W0, b_out - b0."""
    O, W, b = got
    rO, rW, rb = ref
    W0b = np.broadcast_to(W0, rW.shape) if W0.ndim < rW.ndim else W0
    b0b = np.broadcast_to(b0, rb.shape) if b0.ndim < rb.ndim else b0
    return {"O": P.max_rel(O, rO, nseq), "W_out": P.max_rel(W, rW, nseq),
            "b_out": P.max_rel(b, rb, nseq),
            "dW": P.max_rel(W - W0b, rW - W0b, nseq), "db": P.max_rel(b - b0b, rb - b0b, nseq)}


def _offset_linear(seed, io, c, ln_random, L=16 * 20 + 5, row_offsets=False):
    x = gen.make_linear(seed, 1, 3, L, 64, io=io, ln_random=ln_random)
    rng = np.random.default_rng(seed + 1)
    x.b0 = (c + 0.02 * rng.standard_normal((3, 64))).astype(np.float32)
    if row_offsets:  # every input row of W0 offset: mean(z_t) = XK_t . offsets + c
        x.W0 = (x.W0 + rng.standard_normal((3, 64, 1))).astype(np.float32)
    return x


@pytest.mark.parametrize("ln", ["ident", "random"])
@pytest.mark.parametrize("c", [10.0, 100.0])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_linear_prefill_offset_bias(io, c, ln):
    """b0 = c + N(0, 0.02^2): bf16 runs the MFMA prefill, fp32 the VALU one."""
    x = _offset_linear(900 + int(c), io, c, ln == "random")
    got = P.linear_gpu(x)
    ref = P.linear_oracle(x)
    err = _state_errors(got, ref, x.W0, x.b0, 3)
    _report(f"linear {io} b0 offset {c:g} {ln}", err)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_linear_prefill_offset_rows_of_w0(io):
    """W0 rows offset by N(0, 1) each and b0 offset by 30: every token's z
    has its own large mean."""
    x = _offset_linear(950, io, 30.0, False, row_offsets=True)
    got = P.linear_gpu(x)
    ref = P.linear_oracle(x)
    err = _state_errors(got, ref, x.W0, x.b0, 3)
    _report(f"linear {io} W0 row offsets", err)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
def test_linear_prefill_offset_with_weight_decay(loss):
    """Weight decay scales W's row means with W; the MFMA kernel holds the
    state centred and must restore the decayed offset."""
    x = _offset_linear(960, "bf16", 10.0, False, L=16 * 12 + 3, row_offsets=True)
    dt = torch.bfloat16
    O, W, b = ttt.ttt_linear_forward_opts(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt),
                                          P.dev(x.eta), P.dev(x.W0), P.dev(x.b0), P.dev(x.gamma),
                                          P.dev(x.beta), inner_loss=loss, weight_decay=0.5,
                                          ln_eps=x.eps)
    torch.cuda.synchronize()
    ref = oracle.linear_forward_opts(x.XQ, x.XK, x.XV, x.eta, x.W0, x.b0, x.gamma, x.beta, x.eps,
                                     mb=16, loss=loss, weight_decay=0.5)
    err = _state_errors((P.to_np(O), P.to_np(W), P.to_np(b)), ref, x.W0, x.b0, 3)
    _report(f"linear opts {loss} wd=0.5 offsets", err)
    assert max(err.values()) <= P.TOL["bf16"], err


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_linear_prefill_constant_rows(io):
    """W0 = 0 and a constant b0: z is a constant row in the first chunk (zero
    variance, so the gradient carries the 1/sqrt(eps) scale)."""
    x = gen.make_linear(970, 1, 3, 48, 64, io=io)
    x.W0 = np.zeros_like(x.W0)
    x.b0 = np.full_like(x.b0, 0.7)
    got = P.linear_gpu(x)
    ref = P.linear_oracle(x)
    err = _state_errors(got, ref, x.W0, x.b0, 3)
    _report(f"linear {io} W0 = 0, constant b0", err)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("c", [10.0, 100.0])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_mlp_prefill_offset_bias(io, c):
    """b2 = c + N(0, 0.02^2) offsets every row of Z2 = GELU(Z1) W2 + b2."""
    x = gen.make_mlp(980 + int(c), 1, 2, 16 * 8 + 3, 64, io=io)
    rng = np.random.default_rng(981)
    x.b2 = (c + 0.02 * rng.standard_normal(x.b2.shape)).astype(np.float32)
    got = P.mlp_gpu(x)
    ref = P.mlp_oracle(x)
    names = ("O", "W1", "b1", "W2", "b2")
    err = P.errors(got, ref, 2, names)
    err["db2"] = P.max_rel(got[4] - x.b2, ref[4] - x.b2, 2)
    _report(f"mlp {io} b2 offset {c:g}", err)
    assert max(err.values()) <= P.TOL[io], err


def _decode_inputs(seed, io, c, ln, steps=40, B=3, H=2):
    rng = np.random.default_rng(seed)
    dec = gen.make_decode(rng, steps, B, H, 64, io)
    W0 = (0.3 * rng.standard_normal((B, H, 64, 64))).astype(np.float32)
    b0 = (c + 0.02 * rng.standard_normal((B, H, 64))).astype(np.float32)
    if ln == "ident":
        gamma, beta = np.ones((H, 64), np.float32), np.zeros((H, 64), np.float32)
    else:
        gamma = (1 + 0.1 * rng.standard_normal((H, 64))).astype(np.float32)
        beta = (0.1 * rng.standard_normal((H, 64))).astype(np.float32)
    return dec, W0, b0, gamma, beta


def _decode_ref(W0, b0, dec, gamma, beta, mb=1):
    tr = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))
    return oracle.linear_forward(tr(dec.XQ), tr(dec.XK), tr(dec.XV), tr(dec.eta), W0, b0,
                                 gamma, beta, 1e-6, mb=mb, w0_batched=True)


@pytest.mark.parametrize("ln", ["ident", "random"])
@pytest.mark.parametrize("c", [10.0, 100.0])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_offset_bias(io, c, ln):
    """Resident multi-step decode (every state in registers) with b0 = c + N(0, 0.02^2)."""
    dec, W0, b0, gamma, beta = _decode_inputs(990 + int(c), io, c, ln)
    dt = P.io_dtype(io)
    W, b = P.dev(W0), P.dev(b0)
    o = ttt.ttt_decode_steps(P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt),
                             P.dev(dec.eta), W, b, P.dev(gamma), P.dev(beta))
    torch.cuda.synchronize()
    got = (np.ascontiguousarray(np.moveaxis(P.to_np(o), 0, 2)), P.to_np(W), P.to_np(b))
    ref = _decode_ref(W0, b0, dec, gamma, beta)
    err = _state_errors(got, ref, W0, b0, 6)
    _report(f"decode_steps {io} b0 offset {c:g} {ln}", err)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("c", [10.0, 100.0])
def test_decode_step_offset_bias(c):
    """The single-step kernel (one launch per token), fp32. Its state is the
    caller's fp32 array, read and rewritten by every step, so a bias held at
    c can only move in steps of the fp32 spacing at c (7.6e-6 at 100): the
    change b_out - b0 is checked by the multi-step kernels, which keep the
    state in registers, not here."""
    dec, W0, b0, gamma, beta = _decode_inputs(995 + int(c), "f32", c, "random", steps=12)
    W, b = P.dev(W0), P.dev(b0)
    xq, xk, xv, et = P.dev(dec.XQ), P.dev(dec.XK), P.dev(dec.XV), P.dev(dec.eta)
    outs = [ttt.ttt_decode_step(xq[s], xk[s], xv[s], et[s], W, b, P.dev(gamma), P.dev(beta))
            for s in range(dec.steps)]
    torch.cuda.synchronize()
    got = (np.stack([P.to_np(t) for t in outs], 2), P.to_np(W), P.to_np(b))
    ref = _decode_ref(W0, b0, dec, gamma, beta)
    err = P.errors(got, ref, 6, ("O", "W_out", "b_out"))
    err["dW"] = P.max_rel(got[1] - W0, ref[1] - W0, 6)
    _report(f"decode_step f32 b0 offset {c:g}", err)
    assert max(err.values()) <= P.TOL["f32"], err


@pytest.mark.parametrize("c", [10.0, 100.0])
def test_decode_steps_mb_offset_bias(c):
    """Mini-batch decode (b = 4, chunk-start state resident as a second copy), fp32."""
    dec, W0, b0, gamma, beta = _decode_inputs(997 + int(c), "f32", c, "ident", steps=22)
    W, b = P.dev(W0), P.dev(b0)
    Wc, bc = P.dev(W0), P.dev(b0)
    o = ttt.ttt_decode_steps_mb(P.dev(dec.XQ), P.dev(dec.XK), P.dev(dec.XV), P.dev(dec.eta),
                                Wc, bc, W, b, P.dev(gamma), P.dev(beta), mb=4, pos=0)
    torch.cuda.synchronize()
    got = (np.ascontiguousarray(np.moveaxis(P.to_np(o), 0, 2)), P.to_np(W), P.to_np(b))
    ref = _decode_ref(W0, b0, dec, gamma, beta, mb=4)
    err = _state_errors(got, ref, W0, b0, 6)
    _report(f"decode_steps_mb f32 b0 offset {c:g}", err)
    assert max(err.values()) <= P.TOL["f32"], err


@pytest.mark.parametrize("m", [10.0, 100.0, 1000.0])
def test_ln_l2_bwd_offset_rows(m):
    """The fused LN + L2 backward on rows with mean m and spread 0.2."""
    rng = np.random.default_rng(int(m))
    Z = (m + 0.2 * rng.standard_normal((300, 64))).astype(np.float32)
    T = rng.standard_normal((300, 64)).astype(np.float32)
    g = (1 + 0.2 * rng.standard_normal(64)).astype(np.float32)
    b = (0.2 * rng.standard_normal(64)).astype(np.float32)
    G = ttt.ttt_ln_l2_bwd(P.dev(Z), P.dev(T), P.dev(g), P.dev(b), ln_eps=1e-6)
    torch.cuda.synchronize()
    # the oracle sees the same fp32 rows
    ref = oracle.ln_l2_bwd(Z, T, g, b, 1e-6)
    err = np.abs(P.to_np(G) - ref).max(1) / np.abs(ref).max(1)
    print(f"[ln-edge] ln_l2_bwd mean {m:g}: {err.max():.3e}", flush=True)
    assert err.max() < 1e-4, err.max()
