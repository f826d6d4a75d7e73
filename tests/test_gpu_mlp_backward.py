"""GPU parity of ttt_mlp_backward (through the C ABI) against the fp64
gradient oracle (autograd of the TTT-MLP primal recurrence, oracle/grad.py)
on the same inputs. The backward computes in fp32 throughout, so every case
uses the fp32 bar (1e-4, the per-sequence max |diff| / max |ref| of each
gradient) whatever the storage dtype of the inputs."""
import numpy as np
import pytest
import torch

from oracle import grad as OG
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ("dXQ", "dXK", "dXV", "deta", "dW1", "db1", "dW2", "db2", "dgamma", "dbeta")
STATE = ("dW1", "db1", "dW2", "db2")
TOL = 1e-4


def _state(x, batched):
    """Initial state as the kernel takes it: per head, or per sequence."""
    if not batched:
        return x.W1, x.b1, x.W2, x.b2
    return tuple(np.ascontiguousarray(np.broadcast_to(a, (x.B,) + a.shape)) for a in (x.W1, x.b1, x.W2, x.b2))


def _adjoints(rng, x, with_state_grads):
    m = 4 * x.d
    shp = {"dW1": (x.B, x.H, x.d, m), "db1": (x.B, x.H, m), "dW2": (x.B, x.H, m, x.d), "db2": (x.B, x.H, x.d)}
    if not with_state_grads:
        return {k: None for k in shp}
    return {k: rng.standard_normal(s).astype(np.float32) for k, s in shp.items()}


def _run(x, mb, dO, adj, state):
    dt = P.io_dtype(x.io)
    d = lambda a: None if a is None else P.dev(a)
    g = ttt.ttt_mlp_backward(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta),
                             *(P.dev(a) for a in state), P.dev(x.gamma), P.dev(x.beta), P.dev(dO),
                             d(adj["dW1"]), d(adj["db1"]), d(adj["dW2"]), d(adj["db2"]), mb=mb,
                             ln_eps=x.eps)
    torch.cuda.synchronize()
    return {k: P.to_np(v) for k, v in g.items()}


def _compare(got, ref, B, H, tag):
    got = dict(got)
    got["dgamma"] = got["dgamma"].sum(0)
    got["dbeta"] = got["dbeta"].sum(0)
    err = {}
    for k in NAMES:
        err[k] = P.max_rel(got[k], ref[k], H if k in ("dgamma", "dbeta") else B * H)
    print(f"[parity] mlp backward {tag}: " + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= TOL, err


def _check(x, mb, tag, seed, with_state_grads=True, batched=False):
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((x.B, x.H, x.L, x.d)).astype(np.float32)
    adj = _adjoints(rng, x, with_state_grads)
    state = _state(x, batched)
    print(f"[case] mlp backward {tag}: B={x.B} H={x.H} L={x.L} mb={mb} io={x.io}", flush=True)
    got = _run(x, mb, dO, adj, state)
    ref = OG.mlp_backward(x.XQ, x.XK, x.XV, x.eta, *state, x.gamma, x.beta, x.eps, mb, dO,
                          adj["dW1"], adj["db1"], adj["dW2"], adj["db2"])
    _compare(got, ref, x.B, x.H, tag)
    return got


def _small(seed, L, io, B=2, H=3):
    return gen.make_mlp(seed, B, H, L, 64, io=io, ln_random=True, w_std=0.1, b_random=True)


@pytest.mark.parametrize("io,mb,L", [("f32", 16, 40), ("bf16", 16, 48), ("f32", 5, 21), ("bf16", 16, 7),
                                     ("f32", 1, 6), ("f32", 16, 16)])
def test_mlp_backward_small(io, mb, L):
    """Several chunks with a ragged tail, one partial chunk, b = 1 (per-token
    TTT), a schedule with 5-token chunks, exactly one full chunk."""
    _check(_small(1100 + mb + L, L, io), mb, f"{io} mb{mb} L{L}", 1150 + L)


def test_mlp_backward_per_sequence_state_and_no_state_grads():
    """Initial state given per sequence and every state adjoint NULL (zero)."""
    x = _small(1170, 37, "bf16", B=2, H=2)
    _check(x, 16, "per-sequence state, no state grads", 1171, with_state_grads=False, batched=True)


def test_mlp_backward_empty_sequence():
    """L = 0: the state adjoints pass through unchanged; no other gradient."""
    x = _small(1180, 0, "bf16")
    rng = np.random.default_rng(1181)
    adj = _adjoints(rng, x, True)
    got = _run(x, 16, np.zeros((2, 3, 0, 64), np.float32), adj, _state(x, False))
    for k in STATE:
        assert np.array_equal(got[k], adj[k]), k
    assert not np.any(got["dgamma"]) and not np.any(got["dbeta"])
    assert got["dXQ"].shape == (2, 3, 0, 64) and got["deta"].shape == (2, 3, 0)


def test_mlp_backward_repeatable():
    x = _small(1190, 40, "bf16", B=1, H=2)
    rng = np.random.default_rng(1191)
    dO = rng.standard_normal((1, 2, 40, 64)).astype(np.float32)
    adj = _adjoints(rng, x, True)
    a, b = _run(x, 16, dO, adj, _state(x, False)), _run(x, 16, dO, adj, _state(x, False))
    for k in NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_mlp_backward_workload4_sampled_heads():
    """The TTT-MLP workload's full shape (B = 2, H = 12, L = 8192, d = 64,
    bf16 inputs: 512 chunks per sequence) in one launch, as timed; the
    oracle's autograd then runs on two of its 24 sequences, (0, 0) and (1, 7)."""
    x = gen.make_workload(4)
    rng = np.random.default_rng(1200)
    dO = rng.standard_normal((x.B, x.H, x.L, x.d)).astype(np.float32)
    adj = _adjoints(rng, x, True)
    print(f"[case] mlp backward workload 4: B={x.B} H={x.H} L={x.L}", flush=True)
    got = _run(x, 16, dO, adj, _state(x, False))
    for n, h in ((0, 0), (1, 7)):
        one = lambda a: np.ascontiguousarray(a[n:n + 1, h:h + 1])
        ref = OG.mlp_backward(one(x.XQ), one(x.XK), one(x.XV), one(x.eta), x.W1[h:h + 1], x.b1[h:h + 1],
                              x.W2[h:h + 1], x.b2[h:h + 1], x.gamma[h:h + 1], x.beta[h:h + 1], x.eps, 16,
                              one(dO), *(one(adj[k]) for k in STATE))
        sel = {k: one(v) if k not in ("dgamma", "dbeta") else v[n:n + 1, h:h + 1] for k, v in got.items()}
        _compare(sel, ref, 1, 1, f"workload 4 sequence ({n}, {h})")
