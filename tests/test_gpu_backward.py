"""GPU parity of ttt_linear_backward (through the C ABI) against the fp64
gradient oracle (autograd of the primal recurrence) on the same inputs. The
backward computes in fp32 throughout, so every case uses the fp32 bar (1e-4,
S18 metric per gradient) whatever the storage dtype of the inputs."""
import numpy as np
import pytest
import torch

from oracle import grad as OG
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ("dXQ", "dXK", "dXV", "deta", "dW0", "db0", "dgamma", "dbeta")
TOL = 1e-4


def _rel(got, ref, nseq):
    return P.max_rel(got, ref, nseq)


def _run(x, mb, dO, dW=None, db=None, batched_w0=None):
    dt = P.io_dtype(x.io)
    W0 = x.W0 if batched_w0 is None else batched_w0
    g = ttt.ttt_linear_backward(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta),
                                P.dev(W0), P.dev(x.b0), P.dev(x.gamma), P.dev(x.beta), P.dev(dO),
                                None if dW is None else P.dev(dW), None if db is None else P.dev(db),
                                mb=mb, ln_eps=x.eps)
    torch.cuda.synchronize()
    return {k: P.to_np(v) for k, v in g.items()}


def _check(x, mb, tag, dO_seed, with_state_grads=True, batched_w0=None):
    rng = np.random.default_rng(dO_seed)
    B, H, L, d = x.B, x.H, x.L, x.d
    dO = rng.standard_normal((B, H, L, d)).astype(np.float32)
    dW = rng.standard_normal((B, H, d, d)).astype(np.float32) if with_state_grads else None
    db = rng.standard_normal((B, H, d)).astype(np.float32) if with_state_grads else None
    got = _run(x, mb, dO, dW, db, batched_w0)
    W0 = x.W0 if batched_w0 is None else batched_w0
    ref = OG.linear_backward(x.XQ, x.XK, x.XV, x.eta, W0, x.b0, x.gamma, x.beta, x.eps, mb,
                             dO, dW, db)
    # gamma and beta are per head: the kernel returns per-sequence parts
    got["dgamma"] = got["dgamma"].sum(0)
    got["dbeta"] = got["dbeta"].sum(0)
    err = {}
    for k in NAMES:
        nseq = H if k in ("dgamma", "dbeta") else B * H
        err[k] = _rel(got[k], ref[k], nseq)
    print(f"[parity] backward {tag}: " + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= TOL, err
    return got


@pytest.mark.parametrize("io,d,mb,L,ln", [("f32", 16, 4, 23, "random"), ("f32", 64, 16, 40, "random"),
                                          ("bf16", 64, 16, 40, "random"), ("bf16", 64, 16, 48, "ident"),
                                          ("bf16", 64, 5, 21, "random"), ("f32", 64, 1, 9, "random")])
def test_backward_small(io, d, mb, L, ln):
    x = gen.make_linear(900 + d + mb + L, 2, 3, L, d, io=io, ln_random=(ln == "random"),
                        b_random=True, w_std=0.3)
    _check(x, mb, f"{io} d{d} mb{mb} L{L} {ln}", 950 + L)


def test_backward_per_sequence_w0_and_no_state_grads():
    """W0 given per sequence ([B,H,d,d]) and dW_out = db_out = NULL."""
    x = gen.make_linear(961, 2, 2, 37, 64, io="bf16", ln_random=True, b_random=True, w_std=0.3)
    rng = np.random.default_rng(962)
    W0b = (0.3 * rng.standard_normal((2, 2, 64, 64))).astype(np.float32)
    x = gen.LinearInputs(x.B, x.H, x.L, x.d, x.io, x.XQ, x.XK, x.XV, x.eta, W0b,
                         np.broadcast_to(x.b0, (2, 2, 64)).copy(), x.gamma, x.beta)
    _check(x, 16, "per-sequence W0, no state grads", 963, with_state_grads=False, batched_w0=W0b)


def test_backward_empty_sequence():
    """L = 0: all input gradients empty, dW0 = dW_out, db0 = db_out, no gamma/beta gradient."""
    x = gen.make_linear(970, 2, 3, 0, 64, io="bf16", b_random=True)
    rng = np.random.default_rng(971)
    dW = rng.standard_normal((2, 3, 64, 64)).astype(np.float32)
    db = rng.standard_normal((2, 3, 64)).astype(np.float32)
    got = _run(x, 16, np.zeros((2, 3, 0, 64), np.float32), dW, db)
    assert np.array_equal(got["dW0"], dW) and np.array_equal(got["db0"], db)
    assert not np.any(got["dgamma"]) and not np.any(got["dbeta"])
    assert got["dXQ"].shape == (2, 3, 0, 64)


def test_backward_repeatable():
    x = gen.make_linear(975, 2, 2, 64, 64, io="bf16", ln_random=True, b_random=True, w_std=0.3)
    dO = np.random.default_rng(976).standard_normal((2, 2, 64, 64)).astype(np.float32)
    a, b = _run(x, 16, dO), _run(x, 16, dO)
    for k in NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_backward_workload3_sampled_heads():
    """Workload 3's full length (L = 8192, 512 chunks) on two of its heads
    (batch 0, heads 0 and 17): the oracle's autograd runs on those two
    sequences only. Its 1,024 chunks exceed the pre-pass's resident
    workgroups (three per compute unit), so workgroups take a second chunk,
    of the other sequence, through the pre-pass's chunk loop."""
    full = gen.make_workload(3)
    hs = [0, 17]
    sl = lambda a: np.ascontiguousarray(a[:1, hs])
    x = gen.LinearInputs(1, 2, full.L, full.d, full.io, sl(full.XQ), sl(full.XK), sl(full.XV),
                         sl(full.eta), np.ascontiguousarray(full.W0[hs]),
                         np.ascontiguousarray(full.b0[hs]), np.ascontiguousarray(full.gamma[hs]),
                         np.ascontiguousarray(full.beta[hs]))
    _check(x, 16, "workload3 L8192 heads 0,17", 980)
