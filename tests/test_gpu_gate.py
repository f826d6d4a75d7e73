"""GPU parity of the learning-rate gate (the lryc.cn article §2.2, x := the
head's key) through the C ABI: the fused gated TTT-Linear and TTT-MLP
prefills, the standalone gate,
its backward, and the gated training step composed from ttt_eta_gate,
ttt_linear_backward and ttt_eta_gate_backward, each against the fp64 oracle.

theta_lr is drawn wider here (std 0.3) than in the workloads (0.02) so that
theta . x spreads over several units and eta over most of (0, eta_base): a
gate that ignored the keys, or read another head's weights, would fail."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import grad as OG
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-5   # fp32 dot product, exp and divide against fp64


def _gated(seed, B, H, L, d, io, theta_std=0.3, **kw):
    x = gen.make_linear(seed, B, H, L, d, io=io, gate="theta", **kw)
    rng = np.random.default_rng(seed + 1000)
    x.theta_lr = (theta_std * rng.standard_normal((H, d))).astype(np.float32)
    return x


def _report(tag, err):
    print(f"[parity] gate {tag}: " + " ".join(f"{k}={v:.3e}" for k, v in err.items()), flush=True)


@pytest.mark.parametrize("io,d,mb,L", [("bf16", 64, 16, 16 * 12 + 7), ("bf16", 64, 16, 16),
                                       ("f32", 64, 16, 16 * 5 + 3), ("f32", 16, 5, 23),
                                       ("bf16", 16, 16, 40)])
def test_gated_prefill(io, d, mb, L):
    x = _gated(700 + d + L, 2, 3, L, d, io, ln_random=True, b_random=True)
    got = P.linear_gpu(x, mb=mb)
    ref = P.linear_oracle(x, mb=mb)
    err = P.errors(got, ref, x.B * x.H, ("O", "W_out", "b_out"))
    _report(f"prefill {io} d{d} mb{mb} L{L}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_gated_prefill_workload3_shape_sampled_heads():
    """Workload 3's shape (B=2, H=32, L=8192, bf16) with gated eta, in the
    launch configuration of the benchmark; the oracle checks batch 0, heads 0
    and 17 (the recurrence of each head is independent)."""
    full = gen.make_workload(3)
    x = dataclasses.replace(full, eta=None, eta_base=1.0 / full.d,
                            theta_lr=(0.3 * np.random.default_rng(33).standard_normal(
                                (full.H, full.d))).astype(np.float32))
    O, W, b = P.linear_gpu(x)
    hs = [0, 17]
    sl = lambda a: np.ascontiguousarray(a[:1, hs])
    xs = gen.LinearInputs(1, 2, x.L, x.d, x.io, sl(x.XQ), sl(x.XK), sl(x.XV), None,
                          np.ascontiguousarray(x.W0[hs]), np.ascontiguousarray(x.b0[hs]),
                          np.ascontiguousarray(x.gamma[hs]), np.ascontiguousarray(x.beta[hs]),
                          theta_lr=np.ascontiguousarray(x.theta_lr[hs]), eta_base=x.eta_base)
    ref = P.linear_oracle(xs)
    err = P.errors((sl(O), sl(W), sl(b)), ref, 2, ("O", "W_out", "b_out"))
    _report("prefill workload3 shape heads 0,17", err)
    assert max(err.values()) <= P.TOL["bf16"], err


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("L", [1, 37])
def test_eta_gate(io, d, L):
    x = _gated(800 + d + L, 2, 3, L, d, io)
    dt = P.io_dtype(io)
    eta = ttt.ttt_eta_gate(P.dev(x.XK, dt), P.dev(x.theta_lr), x.eta_base)
    torch.cuda.synchronize()
    ref = oracle.eta_gate(x.XK, x.theta_lr, x.eta_base)
    err = P.max_rel(P.to_np(eta), ref, x.B * x.H)
    assert err <= GATE_TOL, err


def test_eta_gate_workload3_shape():
    full = gen.make_workload(3)
    th = (0.3 * np.random.default_rng(34).standard_normal((full.H, full.d))).astype(np.float32)
    eta = ttt.ttt_eta_gate(P.dev(full.XK, torch.bfloat16), P.dev(th), 1.0 / full.d)
    torch.cuda.synchronize()
    ref = oracle.eta_gate(full.XK, th, 1.0 / full.d)
    err = P.max_rel(P.to_np(eta), ref, full.B * full.H)
    print(f"[parity] gate eta workload3 shape: {err:.3e}", flush=True)
    assert err <= GATE_TOL, err


def _gate_bwd_case(io, d, L, seed):
    x = _gated(seed, 2, 3, L, d, io)
    rng = np.random.default_rng(seed + 1)
    deta = rng.standard_normal((2, 3, L)).astype(np.float32)
    dXK0 = rng.standard_normal((2, 3, L, d)).astype(np.float32)
    return x, deta, dXK0


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("L", [0, 1, 45, 300])
def test_eta_gate_backward(io, d, L):
    x, deta, dXK0 = _gate_bwd_case(io, d, L, 850 + d + L)
    dt = P.io_dtype(io)
    XK, th, de = P.dev(x.XK, dt), P.dev(x.theta_lr), P.dev(deta)
    share = torch.zeros((2, 3, L, d), device="cuda")      # the gate's share alone
    dth = ttt.ttt_eta_gate_backward(XK, th, x.eta_base, de, share)
    acc = P.dev(dXK0)                                     # added onto a given dXK
    dth2 = ttt.ttt_eta_gate_backward(XK, th, x.eta_base, de, acc)
    torch.cuda.synchronize()
    assert torch.equal(dth, dth2)
    if L == 0:
        assert not torch.any(dth)
        return
    ref = OG.eta_gate_backward(x.XK, x.theta_lr, x.eta_base, deta)
    e_dth = P.max_rel(P.to_np(dth), ref["dtheta"], 6)
    e_share = P.max_rel(P.to_np(share), ref["dXK"], 6)
    want = dXK0 + ref["dXK"]
    e_acc = np.abs(P.to_np(acc) - want).max() / np.abs(want).max()
    print(f"[parity] gate bwd {io} d{d} L{L}: dtheta={e_dth:.2e} dXK share={e_share:.2e} "
          f"accumulated={e_acc:.2e}", flush=True)
    assert e_dth <= GATE_TOL and e_share <= GATE_TOL and e_acc <= 1e-6


def test_eta_gate_backward_repeatable():
    x, deta, dXK0 = _gate_bwd_case("bf16", 64, 1000, 860)
    outs = []
    for _ in range(2):
        dXK = P.dev(dXK0)
        dth = ttt.ttt_eta_gate_backward(P.dev(x.XK, torch.bfloat16), P.dev(x.theta_lr),
                                        x.eta_base, P.dev(deta), dXK)
        torch.cuda.synchronize()
        outs.append((P.to_np(dXK), P.to_np(dth)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("io,L", [("bf16", 40), ("f32", 23)])
def test_gated_training_step(io, L):
    """Gradients of the gated layer: ttt_eta_gate, then ttt_linear_backward at
    that eta, then ttt_eta_gate_backward adding the path through eta to dXK
    and giving dtheta, against autograd of the gated fp64 recurrence."""
    d, mb = 64, 16
    x = _gated(870 + L, 2, 3, L, d, io, ln_random=True, b_random=True, w_std=0.3)
    dt = P.io_dtype(io)
    rng = np.random.default_rng(871)
    dO = rng.standard_normal((2, 3, L, d)).astype(np.float32)
    dW = rng.standard_normal((2, 3, d, d)).astype(np.float32)
    db = rng.standard_normal((2, 3, d)).astype(np.float32)
    XQ, XK, XV = P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt)
    th = P.dev(x.theta_lr)
    eta = ttt.ttt_eta_gate(XK, th, x.eta_base)
    g = ttt.ttt_linear_backward(XQ, XK, XV, eta, P.dev(x.W0), P.dev(x.b0), P.dev(x.gamma),
                                P.dev(x.beta), P.dev(dO), P.dev(dW), P.dev(db), mb=mb,
                                ln_eps=x.eps)
    dth = ttt.ttt_eta_gate_backward(XK, th, x.eta_base, g["deta"], g["dXK"])
    torch.cuda.synchronize()
    got = {k: P.to_np(v) for k, v in g.items()}
    # theta, gamma and beta are per head: sum the per-sequence parts over B
    got["dtheta"] = P.to_np(dth).sum(0)
    got["dgamma"] = got["dgamma"].sum(0)
    got["dbeta"] = got["dbeta"].sum(0)
    ref = OG.linear_backward_gated(x.XQ, x.XK, x.XV, x.theta_lr, x.eta_base, x.W0, x.b0,
                                   x.gamma, x.beta, x.eps, mb, dO, dW, db)
    err = {}
    for k in ("dXQ", "dXK", "dXV", "dtheta", "dW0", "db0", "dgamma", "dbeta"):
        nseq = 3 if k in ("dtheta", "dgamma", "dbeta") else 6
        err[k] = P.max_rel(got[k], ref[k], nseq)
    _report(f"training step {io} L{L}", err)
    assert max(err.values()) <= 1e-4, err


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_gated_prefill_empty_sequence(io):
    """L = 0: no eta is formed and the final state is the initial one."""
    x = _gated(890, 2, 3, 0, 64, io, b_random=True)
    O, W, b = P.linear_gpu(x)
    assert O.shape == (2, 3, 0, 64)
    assert np.array_equal(W, np.broadcast_to(x.W0, W.shape))
    assert np.array_equal(b, np.broadcast_to(x.b0, b.shape))


# ---------------------------------------------------------------------------
# The gate inside the TTT-MLP prefill (ttt_mlp_forward_gated) against the
# oracle's gate followed by its MLP prefill.
# ---------------------------------------------------------------------------
MLP_NAMES = ("O", "W1_out", "b1_out", "W2_out", "b2_out")


def _mlp_gated(seed, B, H, L, io, theta_std=0.3, **kw):
    x = gen.make_mlp(seed, B, H, L, 64, io=io, **kw)
    th = (theta_std * np.random.default_rng(seed + 1000).standard_normal((H, 64))).astype(np.float32)
    return x, th, 1.0 / 64


def _mlp_gated_gpu(x, th, eta_base, mb):
    dt = P.io_dtype(x.io)
    out = ttt.ttt_mlp_forward_gated(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(th),
                                    eta_base, P.dev(x.W1), P.dev(x.b1), P.dev(x.W2), P.dev(x.b2),
                                    P.dev(x.gamma), P.dev(x.beta), mb=mb, ln_eps=x.eps)
    torch.cuda.synchronize()
    return tuple(P.to_np(t) for t in out)


def _mlp_gated_oracle(x, th, eta_base, mb):
    eta = oracle.eta_gate(x.XK, th, eta_base)
    return oracle.mlp_forward(x.XQ, x.XK, x.XV, eta, x.W1, x.b1, x.W2, x.b2, x.gamma, x.beta,
                              x.eps, mb=mb)


@pytest.mark.parametrize("io,mb,L", [("bf16", 16, 16 * 6 + 5), ("bf16", 16, 16),
                                     ("bf16", 16, 1), ("bf16", 16, 17),
                                     ("f32", 16, 16 * 3 + 7), ("bf16", 5, 23)])
def test_gated_mlp_prefill(io, mb, L):
    x, th, eb = _mlp_gated(900 + mb + L, 2, 3, L, io, ln_random=True, b_random=True)
    got, ref = _mlp_gated_gpu(x, th, eb, mb), _mlp_gated_oracle(x, th, eb, mb)
    err = P.errors(got, ref, x.B * x.H, MLP_NAMES)
    _report(f"mlp prefill {io} mb{mb} L{L}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_gated_mlp_prefill_workload4_shape_sampled_heads():
    """Workload 4's shape (B=2, H=12, L=8192, bf16) with the gate inside the
    MFMA kernel; the oracle checks batch 1, heads 4 and 9."""
    x = gen.make_workload(4)
    th = (0.3 * np.random.default_rng(44).standard_normal((x.H, x.d))).astype(np.float32)
    got = _mlp_gated_gpu(x, th, 1.0 / x.d, 16)
    hs = [4, 9]
    sl = lambda a: np.ascontiguousarray(a[1:2, hs])
    hp = lambda a: np.ascontiguousarray(a[hs])
    eta = oracle.eta_gate(sl(x.XK), hp(th), 1.0 / x.d)
    ref = oracle.mlp_forward(sl(x.XQ), sl(x.XK), sl(x.XV), eta, hp(x.W1), hp(x.b1), hp(x.W2),
                             hp(x.b2), hp(x.gamma), hp(x.beta), x.eps, mb=16)
    err = P.errors(tuple(sl(g) for g in got), ref, 2, MLP_NAMES)
    _report("mlp prefill workload4 shape heads 4,9", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_gated_mlp_prefill_equals_gate_then_prefill():
    """The fused gate against ttt_eta_gate followed by ttt_mlp_forward on the
    same inputs: the two differ only in the rounding of eta. The fp32 states
    agree to 1e-3; O is stored in bf16 (one rounding step is 2^-8 of a value),
    so an output may round the other way: two steps of the largest, 2^-7."""
    x, th, eb = _mlp_gated(950, 2, 3, 16 * 9 + 3, "bf16", b_random=True)
    dt = P.io_dtype(x.io)
    fused = _mlp_gated_gpu(x, th, eb, 16)
    eta = ttt.ttt_eta_gate(P.dev(x.XK, dt), P.dev(th), eb)
    two = ttt.ttt_mlp_forward(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), eta, P.dev(x.W1),
                              P.dev(x.b1), P.dev(x.W2), P.dev(x.b2), P.dev(x.gamma),
                              P.dev(x.beta), ln_eps=x.eps)
    torch.cuda.synchronize()
    err = P.errors(fused, tuple(P.to_np(t) for t in two), x.B * x.H, MLP_NAMES)
    _report("mlp fused vs two-pass", err)
    assert err["O"] <= 2.0 ** -7, err
    assert max(v for k, v in err.items() if k != "O") <= 1e-3, err


def test_gated_mlp_empty_sequence():
    x, th, eb = _mlp_gated(960, 2, 3, 0, "bf16", b_random=True)
    got = _mlp_gated_gpu(x, th, eb, 16)
    assert got[0].shape == (2, 3, 0, 64)
    for g_, r_ in zip(got[1:], (x.W1, x.b1, x.W2, x.b2)):
        assert np.array_equal(g_, np.broadcast_to(r_, g_.shape))


# ---------------------------------------------------------------------------
# The gate inside the decode kernels (ttt_decode_steps_gated): a gated prefill
# followed by gated decode calls equals the oracle's gate and prefill over the
# whole sequence.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("io,d", [("bf16", 64), ("f32", 64), ("f32", 16)])
@pytest.mark.parametrize("mb", [1, 4, 16])
def test_gated_decode_continues_the_gated_prefill(io, d, mb):
    B, H, L0 = 2, 3, 2 * mb
    splits = [mb // 2 + 1, mb + 1, max(mb - 2, 1)]
    T = sum(splits)
    x = _gated(1000 + 3 * d + mb, B, H, L0 + T, d, io, ln_random=True, b_random=True, w_std=0.3)
    dt = P.io_dtype(io)
    th = P.dev(x.theta_lr)
    O0, W, b = ttt.ttt_linear_forward_gated(*(P.dev(a[:, :, :L0], dt) for a in (x.XQ, x.XK, x.XV)),
                                            th, x.eta_base, P.dev(x.W0), P.dev(x.b0),
                                            P.dev(x.gamma), P.dev(x.beta), mb=mb, ln_eps=x.eps)
    Wc, bc = torch.full_like(W, float("nan")), torch.full_like(b, float("nan"))  # unread at pos 0
    step = lambda a: np.ascontiguousarray(np.moveaxis(a, 2, 0))   # [B,H,T,...] -> [T,B,H,...]
    outs, t, pos = [], L0, 0
    for n in splits:
        sl = slice(t, t + n)
        o = ttt.ttt_decode_steps_gated(*(P.dev(step(a[:, :, sl]), dt) for a in (x.XQ, x.XK, x.XV)),
                                       th, x.eta_base, W, b, P.dev(x.gamma), P.dev(x.beta), mb=mb,
                                       pos=pos, W_chunk=Wc if mb > 1 else None,
                                       b_chunk=bc if mb > 1 else None, ln_eps=x.eps)
        outs.append(np.moveaxis(P.to_np(o), 0, 2))
        t, pos = t + n, (pos + n) % mb
    torch.cuda.synchronize()
    eta = oracle.eta_gate(x.XK, x.theta_lr, x.eta_base)
    O_ref, W_ref, b_ref = oracle.linear_forward(x.XQ, x.XK, x.XV, eta, x.W0, x.b0, x.gamma, x.beta,
                                                x.eps, mb=mb)
    got = (np.concatenate(outs, 2), P.to_np(W), P.to_np(b))
    err = P.errors(got, (O_ref[:, :, L0:], W_ref, b_ref), B * H, ("o", "W", "b"))
    _report(f"decode mb={mb} {io} d{d}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_gated_decode_workload5_shape():
    """Workload 5's decode (1024 steps on 64 x 32 states of d = 64, bf16) with
    the gate inside the resident kernel, from the same start state per
    sequence, against the oracle's gate and b = 1 recurrence."""
    _, dec = gen.make_workload(5)
    rng = np.random.default_rng(55)
    th = (0.3 * rng.standard_normal((dec.H, dec.d))).astype(np.float32)
    W0 = (0.3 * rng.standard_normal((dec.B, dec.H, dec.d, dec.d))).astype(np.float32)
    b0 = (0.1 * rng.standard_normal((dec.B, dec.H, dec.d))).astype(np.float32)
    g, be = np.ones((dec.H, dec.d), np.float32), np.zeros((dec.H, dec.d), np.float32)
    dt = P.io_dtype(dec.io)
    W, b = P.dev(W0), P.dev(b0)
    o = ttt.ttt_decode_steps_gated(P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt),
                                   P.dev(th), 1.0 / dec.d, W, b, P.dev(g), P.dev(be))
    torch.cuda.synchronize()
    tr = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))  # step-major -> [B,H,T,...]
    eta = oracle.eta_gate(tr(dec.XK), th, 1.0 / dec.d)
    ref = oracle.linear_forward(tr(dec.XQ), tr(dec.XK), tr(dec.XV), eta, W0, b0, g, be, 1e-6,
                                mb=1, w0_batched=True)
    got = (tr(P.to_np(o)), P.to_np(W), P.to_np(b))
    err = P.errors(got, ref, dec.B * dec.H, ("o", "W", "b"))
    _report("decode workload5 shape 64x32x1024", err)
    assert max(err.values()) <= P.TOL["bf16"], err
