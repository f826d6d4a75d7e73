"""The entry points enqueue on the caller's stream: run each on a side
stream, with HIP events recorded on that stream around the call (the work
must fall between them), and compare with the same call on the default
stream bit for bit."""
import numpy as np
import pytest
import torch

from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu


def _on_stream(fn, stream):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        out = fn(stream)
        e1.record(stream)
    stream.synchronize()
    return out, e0.elapsed_time(e1) * 1e3  # us


def _check(fn, min_us):
    ref = fn(None)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    got, us = _on_stream(fn, s)
    print(f"[stream] {us:.1f} us between the side stream's events", flush=True)
    assert us > min_us, us
    ref = ref if isinstance(ref, (tuple, list)) else (ref,)
    got = got if isinstance(got, (tuple, list)) else (got,)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_linear_forward_on_side_stream():
    x = gen.make_workload(3, L=2048, B=2, H=32)
    dt = torch.bfloat16
    args = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta), P.dev(x.W0),
            P.dev(x.b0), P.dev(x.gamma), P.dev(x.beta)]
    _check(lambda s: ttt.ttt_linear_forward(*args, stream=s), 20.0)


def test_mlp_forward_on_side_stream():
    x = gen.make_workload(4, L=512, B=2, H=12)
    dt = torch.bfloat16
    args = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta), P.dev(x.W1),
            P.dev(x.b1), P.dev(x.W2), P.dev(x.b2), P.dev(x.gamma), P.dev(x.beta)]
    _check(lambda s: ttt.ttt_mlp_forward(*args, stream=s), 20.0)


def test_decode_steps_on_side_stream():
    rng = np.random.default_rng(77)
    dec = gen.make_decode(rng, 256, 8, 32, 64, "bf16")
    W0 = (0.3 * rng.standard_normal((8, 32, 64, 64))).astype(np.float32)
    g, be = np.ones((32, 64), np.float32), np.zeros((32, 64), np.float32)
    dt = torch.bfloat16

    def run(s):
        W, b = P.dev(W0), torch.zeros((8, 32, 64), device="cuda")
        o = ttt.ttt_decode_steps(P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt),
                                 P.dev(dec.eta), W, b, P.dev(g), P.dev(be), stream=s)
        return o, W, b
    # the state buffers are made on the current stream before the launch; the
    # side stream's events bracket the launch itself
    _check(run, 20.0)


def test_backward_on_side_stream():
    x = gen.make_workload(3, L=512, B=2, H=8)
    dt = torch.bfloat16
    dO = P.dev(np.random.default_rng(78).standard_normal((2, 8, 512, 64)).astype(np.float32))
    args = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta), P.dev(x.W0),
            P.dev(x.b0), P.dev(x.gamma), P.dev(x.beta), dO]

    def run(s):
        gr = ttt.ttt_linear_backward(*args, stream=s)
        return tuple(gr[k] for k in sorted(gr))
    _check(run, 20.0)


def test_mlp_backward_on_side_stream():
    x = gen.make_workload(4, L=256, B=2, H=4)
    dt = torch.bfloat16
    dO = P.dev(np.random.default_rng(79).standard_normal((2, 4, 256, 64)).astype(np.float32))
    args = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt), P.dev(x.eta), P.dev(x.W1),
            P.dev(x.b1), P.dev(x.W2), P.dev(x.b2), P.dev(x.gamma), P.dev(x.beta), dO]

    def run(s):
        gr = ttt.ttt_mlp_backward(*args, stream=s)
        return tuple(gr[k] for k in sorted(gr))
    _check(run, 20.0)


def test_qkv_project_on_side_stream():
    x = gen.make_proj_workload(2, L=1024)
    X = P.dev(x.X, torch.bfloat16)
    th = P.dev(x.theta, torch.bfloat16)
    _check(lambda s: ttt.ttt_qkv_project(X, th, x.H, stream=s), 5.0)


def _variant_args(kind):
    dt = torch.bfloat16
    if kind.startswith("linear"):
        x = gen.make_workload(3, L=1024, B=2, H=32)
        ins = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt)]
        st = [P.dev(x.W0), P.dev(x.b0), P.dev(x.gamma), P.dev(x.beta)]
    else:
        x = gen.make_workload(4, L=512, B=2, H=12)
        ins = [P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt)]
        st = [P.dev(x.W1), P.dev(x.b1), P.dev(x.W2), P.dev(x.b2), P.dev(x.gamma), P.dev(x.beta)]
    th = P.dev((0.3 * np.random.default_rng(78).standard_normal((x.H, x.d))).astype(np.float32))
    return x, ins, st, th, P.dev(x.eta)


def _decode_gated(ins, th, eb, st, s):
    """64 gated decode steps on 2 x 32 states (the first 64 tokens of the
    linear case as step-major inputs), each call from the same start state."""
    step = lambda a: a[:, :, :64].permute(2, 0, 1, 3).contiguous()   # [B,H,T,d] -> [T,B,H,d]
    W = st[0].unsqueeze(0).expand(2, -1, -1, -1).contiguous()
    b = st[1].unsqueeze(0).expand(2, -1, -1).contiguous()
    o = ttt.ttt_decode_steps_gated(step(ins[0]), step(ins[1]), step(ins[2]), th, eb, W, b, st[2],
                                   st[3], stream=s)
    return o, W, b


@pytest.mark.parametrize("kind", ["linear_gated", "linear_opts", "mlp_gated", "mlp_opts", "gate",
                                  "decode_gated"])
def test_variant_entry_points_on_side_stream(kind):
    """The gated and option prefills and the standalone gate: side stream
    against default stream, bit for bit (the kernels are deterministic)."""
    x, ins, st, th, eta = _variant_args("linear" if kind == "decode_gated" else kind)
    eb = 1.0 / x.d
    fn = {
        "linear_gated": lambda s: ttt.ttt_linear_forward_gated(*ins, th, eb, *st, stream=s),
        "linear_opts": lambda s: ttt.ttt_linear_forward_opts(*ins, eta, *st, "inner_product", 0.5,
                                                             stream=s),
        "mlp_gated": lambda s: ttt.ttt_mlp_forward_gated(*ins, th, eb, *st, stream=s),
        "mlp_opts": lambda s: ttt.ttt_mlp_forward_opts(*ins, eta, *st, "inner_product", 0.5,
                                                       stream=s),
        "gate": lambda s: ttt.ttt_eta_gate(ins[1], th, eb, stream=s),
        "decode_gated": lambda s: _decode_gated(ins, th, eb, st, s),
    }[kind]
    _check(fn, 1.0 if kind in ("gate", "decode_gated") else 20.0)
