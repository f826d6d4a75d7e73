"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs. Sizes range from oracle-quick cases that span several
chunks and a ragged tail up to the five full workloads."""
import numpy as np
import pytest
import torch

import oracle
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu

LIN_NAMES = ("O", "W_out", "b_out")
MLP_NAMES = ("O", "W1", "b1", "W2", "b2")


def _report(tag, err):
    print(f"[parity] {tag}: " + " ".join(f"{k}={v:.3e}" for k, v in err.items()), flush=True)


def _check_linear(x, tag, mb=None, tol=None):
    got = P.linear_gpu(x, mb=mb)
    ref = P.linear_oracle(x, mb=mb)
    err = P.errors(got, ref, x.B * x.H, LIN_NAMES)
    _report(tag, err)
    _report(tag + " elementwise (floor 1e-3 max|ref|)", P.elem_errors(got, ref, x.B * x.H, LIN_NAMES))
    tol = tol or P.TOL[x.io]
    assert max(err.values()) <= tol, err
    return got


# ---------------------------------------------------------------------------
# LN + L2 backward on its own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("rows", [1, 17, 1000])
def test_ln_l2_bwd(d, rows):
    rng = np.random.default_rng(rows * 100 + d)
    Z = (rng.standard_normal((rows, d)) * rng.uniform(0.1, 3, (rows, 1))
         + rng.standard_normal((rows, 1))).astype(np.float32)
    T = rng.standard_normal((rows, d)).astype(np.float32)
    g = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    b = (0.2 * rng.standard_normal(d)).astype(np.float32)
    G = ttt.ttt_ln_l2_bwd(P.dev(Z), P.dev(T), P.dev(g), P.dev(b), ln_eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.ln_l2_bwd(Z, T, g, b, 1e-6)
    err = np.abs(P.to_np(G) - ref).max(1) / np.abs(ref).max(1)
    assert err.max() < 1e-5, err.max()


# ---------------------------------------------------------------------------
# TTT-Linear prefill
# ---------------------------------------------------------------------------
def test_linear_workload1_fp32():
    _check_linear(gen.make_workload(1), "workload1 fp32 d16")


@pytest.mark.parametrize("mb", [16, 5, 1])
@pytest.mark.parametrize("d", [16, 64])
def test_linear_fp32_ragged(d, mb):
    x = gen.make_linear(200 + d + mb, 2, 3, 53, d, io="f32", ln_random=True, b_random=True)
    _check_linear(x, f"fp32 d{d} mb{mb} L53")


@pytest.mark.parametrize("num", [2, 3])
def test_linear_bf16_small(num):
    x = gen.make_workload(num, L=16 * 12 + 7, B=2, H=3)
    _check_linear(x, f"workload{num} small L199")


def test_linear_bf16_random_ln():
    x = gen.make_linear(301, 2, 4, 16 * 20, 64, io="bf16", ln_random=True, b_random=True)
    _check_linear(x, "bf16 random gamma/beta/b0")


@pytest.mark.parametrize("L", [1, 15, 16, 17])
def test_linear_bf16_short(L):
    x = gen.make_linear(400 + L, 1, 2, L, 64, io="bf16")
    _check_linear(x, f"bf16 L{L}")


@pytest.mark.parametrize("num", [2, 3])
def test_linear_full_workload(num):
    x = gen.make_workload(num)
    _check_linear(x, f"workload{num} full")


def test_linear_full_workload5_prefill():
    pre, _ = gen.make_workload(5, decode_steps=0)
    _check_linear(pre, "workload5 prefill L32768")


def test_linear_empty_sequence_passes_state():
    x = gen.make_linear(500, 2, 3, 0, 64, io="bf16", b_random=True)
    O, W, b = P.linear_gpu(x)
    assert O.shape == (2, 3, 0, 64)
    assert np.array_equal(W, np.broadcast_to(x.W0, W.shape))
    assert np.array_equal(b, np.broadcast_to(x.b0, b.shape))


def test_linear_in_place_resume():
    """forward(L1) with the state updated in place, then forward(L2) from it,
    matches the oracle's forward(L1 + L2)."""
    x = gen.make_linear(510, 2, 3, 160, 64, io="bf16")
    dt = torch.bfloat16
    W = P.dev(np.broadcast_to(x.W0, (2, 3, 64, 64)))
    b = P.dev(np.broadcast_to(x.b0, (2, 3, 64)))
    outs = []
    for s in (slice(0, 96), slice(96, 160)):
        O, _, _ = ttt.ttt_linear_forward(P.dev(x.XQ[:, :, s], dt), P.dev(x.XK[:, :, s], dt),
                                         P.dev(x.XV[:, :, s], dt), P.dev(x.eta[:, :, s]), W, b,
                                         P.dev(x.gamma), P.dev(x.beta), W_out=W, b_out=b)
        outs.append(P.to_np(O))
    torch.cuda.synchronize()
    ref = P.linear_oracle(x)
    err = P.errors((np.concatenate(outs, 2), P.to_np(W), P.to_np(b)), ref, 6, LIN_NAMES)
    _report("in-place resume", err)
    assert max(err.values()) <= P.TOL["bf16"]


def test_linear_prefill_rows_past_4gib():
    """One head at L = 2^25 + 32: the bf16 rows of the last two chunks start
    4 GiB into XQ, XK, XV and O, where 32-bit byte offsets would wrap. The
    single call's last two chunks of O and its final state are compared with
    the oracle run over those two chunks from the state the kernel returns
    for the first 2^25 tokens (a chain of 2^21 chunks is out of the oracle's
    reach). Inputs follow the bf16 recipe (rows N(0, 1), eta = logistic(N(0, 1))
    / d), drawn on the GPU from a seeded torch generator, W0, b0, gamma, beta
    from the generator module; O starts as NaN, so an unwritten row fails."""
    L0, tail, d = 1 << 25, 32, 64
    L = L0 + tail
    print(f"[parity] prefill past 4 GiB: B=1 H=1 L={L}", flush=True)
    rng = torch.Generator(device="cuda")
    rng.manual_seed(2525)
    shp = (1, 1, L, d)
    XQ, XK, XV = (torch.randn(shp, generator=rng, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    eta = torch.sigmoid(torch.randn((1, 1, L), generator=rng, device="cuda")) / d
    x0 = gen.make_linear(2525, 1, 1, 16, d)
    W0, b0, g, be = (P.dev(a) for a in (x0.W0, x0.b0, x0.gamma, x0.beta))
    O = torch.full(shp, float("nan"), device="cuda", dtype=torch.bfloat16)
    _, W_full, b_full = ttt.ttt_linear_forward(XQ, XK, XV, eta, W0, b0, g, be, O=O)
    h = slice(0, L0)
    _, W_mid, b_mid = ttt.ttt_linear_forward(XQ[:, :, h], XK[:, :, h], XV[:, :, h], eta[:, :, h], W0, b0, g, be)
    torch.cuda.synchronize()
    t = slice(L0, L)
    f32 = lambda a: P.to_np(a).astype(np.float32)
    two = gen.LinearInputs(1, 1, tail, d, "bf16", f32(XQ[:, :, t]), f32(XK[:, :, t]), f32(XV[:, :, t]),
                           f32(eta[:, :, t]), f32(W_mid)[0], f32(b_mid)[0], x0.gamma, x0.beta)
    got = (P.to_np(O[:, :, t]), P.to_np(W_full), P.to_np(b_full))
    del XQ, XK, XV, eta, O
    torch.cuda.empty_cache()
    ref = P.linear_oracle(two)
    err = P.errors(got, ref, 1, LIN_NAMES)
    _report("prefill L = 2^25 + 32, last two chunks", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_mlp_prefill_rows_past_4gib():
    """TTT-MLP at L = 2^25 + 32, checked as the TTT-Linear case above: the
    single call's last two chunks of O and its final W1, b1, W2, b2 against the
    oracle run over those two chunks from the state the kernel returns for
    the first 2^25 tokens."""
    L0, tail, d = 1 << 25, 32, 64
    L = L0 + tail
    print(f"[parity] MLP prefill past 4 GiB: B=1 H=1 L={L}", flush=True)
    rng = torch.Generator(device="cuda")
    rng.manual_seed(2526)
    shp = (1, 1, L, d)
    XQ, XK, XV = (torch.randn(shp, generator=rng, device="cuda", dtype=torch.bfloat16) for _ in range(3))
    eta = torch.sigmoid(torch.randn((1, 1, L), generator=rng, device="cuda")) / d
    x0 = gen.make_mlp(2526, 1, 1, 16, d)
    st = [P.dev(a) for a in (x0.W1, x0.b1, x0.W2, x0.b2, x0.gamma, x0.beta)]
    O = torch.full(shp, float("nan"), device="cuda", dtype=torch.bfloat16)
    full = ttt.ttt_mlp_forward(XQ, XK, XV, eta, *st, O=O)
    h = slice(0, L0)
    mid = ttt.ttt_mlp_forward(XQ[:, :, h], XK[:, :, h], XV[:, :, h], eta[:, :, h], *st)
    torch.cuda.synchronize()
    t = slice(L0, L)
    f32 = lambda a: P.to_np(a).astype(np.float32)
    two = gen.MLPInputs(1, 1, tail, d, "bf16", f32(XQ[:, :, t]), f32(XK[:, :, t]), f32(XV[:, :, t]),
                        f32(eta[:, :, t]), *(f32(a)[0] for a in mid[1:]), x0.gamma, x0.beta)
    got = (P.to_np(O[:, :, t]), *(P.to_np(a) for a in full[1:]))
    del XQ, XK, XV, eta, O, full, mid
    torch.cuda.empty_cache()
    ref = P.mlp_oracle(two)
    err = P.errors(got, ref, 1, MLP_NAMES)
    _report("MLP prefill L = 2^25 + 32, last two chunks", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_linear_bitwise_repeatable():
    x = gen.make_workload(3, L=16 * 40, B=2, H=4)
    a = P.linear_gpu(x)
    b = P.linear_gpu(x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# TTT-MLP prefill
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("io,mb", [("f32", 16), ("f32", 3), ("bf16", 16)])
def test_mlp_small(io, mb):
    x = gen.make_mlp(600 + mb, 2, 2, 16 * 5 + 9, 64, io=io, ln_random=True, b_random=True)
    got = P.mlp_gpu(x, mb=mb)
    ref = P.mlp_oracle(x, mb=mb)
    err = P.errors(got, ref, 4, MLP_NAMES)
    _report(f"mlp {io} mb{mb}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_mlp_full_workload4():
    x = gen.make_workload(4)
    got = P.mlp_gpu(x)
    ref = P.mlp_oracle(x)
    err = P.errors(got, ref, x.B * x.H, MLP_NAMES)
    _report("workload 4 elementwise (floor 1e-3 max|ref|)", P.elem_errors(got, ref, x.B * x.H, MLP_NAMES))
    _report("workload4 full", err)
    assert max(err.values()) <= P.TOL["bf16"], err


@pytest.mark.parametrize("L", [0, 1, 16, 17])
def test_mlp_bf16_short(L):
    """MFMA path (bf16, mb = 16) at the lengths around one chunk, random LN and biases."""
    x = gen.make_mlp(640 + L, 2, 3, L, 64, io="bf16", ln_random=True, b_random=True)
    got = P.mlp_gpu(x)
    ref = P.mlp_oracle(x)
    assert got[0].shape == (2, 3, L, 64)
    err = P.errors(got, ref, 6, MLP_NAMES)
    _report(f"mlp bf16 L{L}", err)
    if L == 0:  # the state passes through unchanged
        for g_, r_ in zip(got[1:], (x.W1, x.b1, x.W2, x.b2)):
            assert np.array_equal(g_, np.broadcast_to(r_, g_.shape))
    assert max(err.values()) <= P.TOL["bf16"], err


def test_mlp_in_place_resume():
    """forward(L1) with the per-batch state updated in place, then forward(L2)
    from it, matches the oracle's forward(L1 + L2)."""
    x = gen.make_mlp(660, 2, 2, 112, 64, io="bf16", b_random=True)
    dt = torch.bfloat16
    st = [P.dev(np.broadcast_to(a, (2,) + a.shape)) for a in (x.W1, x.b1, x.W2, x.b2)]
    outs = []
    for s_ in (slice(0, 64), slice(64, 112)):
        res = ttt.ttt_mlp_forward(P.dev(x.XQ[:, :, s_], dt), P.dev(x.XK[:, :, s_], dt),
                                  P.dev(x.XV[:, :, s_], dt), P.dev(x.eta[:, :, s_]), *st,
                                  P.dev(x.gamma), P.dev(x.beta), outs=tuple(st))
        outs.append(P.to_np(res[0]))
    torch.cuda.synchronize()
    ref = P.mlp_oracle(x)
    got = (np.concatenate(outs, 2),) + tuple(P.to_np(t) for t in st)
    err = P.errors(got, ref, 4, MLP_NAMES)
    _report("mlp in-place resume", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_mlp_bitwise_repeatable():
    x = gen.make_workload(4, L=16 * 20, B=1, H=3)
    a = P.mlp_gpu(x)
    b = P.mlp_gpu(x)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------------------
# Chunk-local parity: the oracle's state at the start of a sampled chunk is
# handed to the kernel, which runs that one chunk; its outputs are compared
# with the oracle's run of the same chunk from the same state. This checks
# the kernel at depth without the chain's accumulated rounding.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("num,chunks", [(3, (0, 1, 255, 511)), (5, (1024, 2047))])
def test_linear_chunk_local_teacher_forced(num, chunks):
    x = gen.make_workload(num, decode_steps=0) if num == 5 else gen.make_workload(num)
    if num == 5:
        x = x[0]
    B, H = x.B, x.H
    worst = 0.0
    for c in chunks:
        t0 = 16 * c
        pre = slice(0, t0)
        cur = slice(t0, t0 + 16)
        if t0 > 0:
            _, Wc, bc = oracle.linear_forward(x.XQ[:, :, pre], x.XK[:, :, pre], x.XV[:, :, pre],
                                              x.eta[:, :, pre], x.W0, x.b0, x.gamma, x.beta, x.eps)
        else:
            Wc = np.broadcast_to(x.W0, (B, H, 64, 64))
            bc = np.broadcast_to(x.b0, (B, H, 64))
        Wc = np.ascontiguousarray(Wc, np.float32)  # both sides start from the same fp32 state
        bc = np.ascontiguousarray(bc, np.float32)
        one = gen.LinearInputs(B, H, 16, 64, x.io, x.XQ[:, :, cur], x.XK[:, :, cur], x.XV[:, :, cur],
                               x.eta[:, :, cur], Wc, bc, x.gamma, x.beta)
        got = P.linear_gpu(one)
        ref = P.linear_oracle(one)
        err = P.errors(got, ref, B * H, LIN_NAMES)
        _report(f"workload{num} chunk {c} teacher-forced", err)
        worst = max(worst, max(err.values()))
    assert worst <= P.TOL["bf16"], worst


# ---------------------------------------------------------------------------
# Decode (b = 1 primal step, state in place)
# ---------------------------------------------------------------------------
def _decode_run(W0, b0, dec, gamma, beta, eps):
    dt = P.io_dtype(dec.io)
    W = P.dev(W0)
    b = P.dev(b0)
    g, be = P.dev(gamma), P.dev(beta)
    xq, xk, xv, et = (P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt), P.dev(dec.eta))
    outs = []
    for s in range(dec.steps):
        outs.append(ttt.ttt_decode_step(xq[s], xk[s], xv[s], et[s], W, b, g, be, ln_eps=eps))
    torch.cuda.synchronize()
    O = np.stack([P.to_np(o) for o in outs], 2)  # [B,H,steps,d]
    return O, P.to_np(W), P.to_np(b)


def _decode_oracle(W0, b0, dec, gamma, beta, eps):
    tr = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))  # step-major -> [B,H,steps,...]
    return oracle.linear_forward(tr(dec.XQ), tr(dec.XK), tr(dec.XV), tr(dec.eta), W0, b0,
                                 gamma, beta, eps, mb=1, w0_batched=True)


@pytest.mark.parametrize("io,d", [("f32", 16), ("f32", 64), ("bf16", 64)])
def test_decode_small(io, d):
    rng = np.random.default_rng(700 + d)
    dec = gen.make_decode(rng, 20, 3, 2, d, io)
    W0 = (0.3 * rng.standard_normal((3, 2, d, d))).astype(np.float32)
    b0 = (0.1 * rng.standard_normal((3, 2, d))).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal((2, d))).astype(np.float32)
    beta = (0.1 * rng.standard_normal((2, d))).astype(np.float32)
    got = _decode_run(W0, b0, dec, gamma, beta, 1e-6)
    ref = _decode_oracle(W0, b0, dec, gamma, beta, 1e-6)
    err = P.errors(got, ref, 6, LIN_NAMES)
    _report(f"decode {io} d{d}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_prefill_then_decode_matches_mixed_schedule():
    """Prefill (mb = 16) then decode steps equals the oracle's single run with
    chunk schedule [16]*k + [1]*n."""
    x = gen.make_linear(720, 1, 4, 64 + 24, 64, io="bf16")
    Lp = 64
    sl = slice(0, Lp)
    pre = gen.LinearInputs(1, 4, Lp, 64, "bf16", x.XQ[:, :, sl], x.XK[:, :, sl], x.XV[:, :, sl],
                           x.eta[:, :, sl], x.W0, x.b0, x.gamma, x.beta)
    _, W, b = P.linear_gpu(pre)
    mv = lambda a: np.ascontiguousarray(np.moveaxis(a[:, :, Lp:], 2, 0))
    dec = gen.DecodeInputs(24, 1, 4, 64, "bf16", mv(x.XQ), mv(x.XK), mv(x.XV), mv(x.eta))
    O, Wd, bd = _decode_run(W.astype(np.float32), b.astype(np.float32), dec, x.gamma, x.beta, x.eps)
    ref = P.linear_oracle(x, schedule=[16] * 4 + [1] * 24)
    err = P.errors((O, Wd, bd), (ref[0][:, :, Lp:], ref[1], ref[2]), 4, LIN_NAMES)
    _report("prefill+decode", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_decode_full_workload5():
    """Workload 5: prefill B=1, H=32, L=32768, then 1024 single-token steps for
    64 independent sequences, each starting from a copy of the prefill state."""
    pre, dec = gen.make_workload(5)
    _, Wp, bp = P.linear_gpu(pre)
    rW, rb = P.linear_oracle(pre)[1:]
    W0 = np.broadcast_to(Wp[0], (64,) + Wp.shape[1:]).astype(np.float32)
    b0 = np.broadcast_to(bp[0], (64,) + bp.shape[1:]).astype(np.float32)
    got = _decode_run(W0, b0, dec, pre.gamma, pre.beta, pre.eps)
    # the oracle continues from its own prefill state
    ref = _decode_oracle(np.broadcast_to(rW[0], W0.shape), np.broadcast_to(rb[0], b0.shape),
                         dec, pre.gamma, pre.beta, pre.eps)
    err = P.errors(got, ref, 64 * 32, LIN_NAMES)
    _report("workload5 decode 64x1024", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def _steps_run(W0, b0, dec, gamma, beta, eps):
    """ttt_decode_steps over all steps of `dec` in one call."""
    dt = P.io_dtype(dec.io)
    W = P.dev(W0)
    b = P.dev(b0)
    o = ttt.ttt_decode_steps(P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt),
                             P.dev(dec.eta), W, b, P.dev(gamma), P.dev(beta), ln_eps=eps)
    torch.cuda.synchronize()
    return np.ascontiguousarray(np.moveaxis(P.to_np(o), 0, 2)), P.to_np(W), P.to_np(b)


def _decode_case(seed, steps, B, H, d, io, ln):
    rng = np.random.default_rng(seed)
    dec = gen.make_decode(rng, steps, B, H, d, io)
    W0 = (0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    b0 = (0.1 * rng.standard_normal((B, H, d))).astype(np.float32)
    if ln == "ident":
        gamma, beta = np.ones((H, d), np.float32), np.zeros((H, d), np.float32)
    else:
        gamma = (1 + 0.1 * rng.standard_normal((H, d))).astype(np.float32)
        beta = (0.1 * rng.standard_normal((H, d))).astype(np.float32)
    return dec, W0, b0, gamma, beta


@pytest.mark.parametrize("io,d,ln", [("f32", 16, "random"), ("f32", 64, "random"),
                                     ("f32", 64, "ident"), ("bf16", 64, "random"),
                                     ("bf16", 64, "ident")])
def test_decode_steps_small(io, d, ln):
    """T steps in one call (state resident for d = 64) against the oracle's
    b = 1 schedule, and against T calls of the single-step entry point."""
    dec, W0, b0, gamma, beta = _decode_case(760 + d, 37, 3, 2, d, io, ln)
    got = _steps_run(W0, b0, dec, gamma, beta, 1e-6)
    ref = _decode_oracle(W0, b0, dec, gamma, beta, 1e-6)
    err = P.errors(got, ref, 6, LIN_NAMES)
    _report(f"decode_steps {io} d{d} {ln}", err)
    assert max(err.values()) <= P.TOL[io], err
    one = _decode_run(W0, b0, dec, gamma, beta, 1e-6)
    err1 = P.errors(got, one, 6, LIN_NAMES)
    _report(f"decode_steps vs single steps {io} d{d} {ln}", err1)
    assert max(err1.values()) <= P.TOL[io], err1


@pytest.mark.parametrize("steps", [0, 1, 2])
def test_decode_steps_edge(steps):
    """T = 0 leaves the state untouched; T = 1 and 2 equal the single-step path."""
    dec, W0, b0, gamma, beta = _decode_case(790 + steps, steps, 2, 3, 64, "bf16", "random")
    got = _steps_run(W0, b0, dec, gamma, beta, 1e-6)
    if steps == 0:
        assert np.array_equal(got[1], W0) and np.array_equal(got[2], b0)
        assert got[0].shape == (2, 3, 0, 64)
        return
    ref = _decode_oracle(W0, b0, dec, gamma, beta, 1e-6)
    err = P.errors(got, ref, 6, LIN_NAMES)
    _report(f"decode_steps T{steps}", err)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_decode_steps_resume_and_repeatable():
    """A repeat of the same call is bitwise identical, and two calls of T1
    and T2 steps equal one call of T1 + T2 steps. Within a call the kernel
    holds the state with its row means removed and restores them on the way
    out, so a split run differs from one call only by the rounding of that
    round trip: the state to 1e-6 relative, the bf16 outputs by at most one
    rounding step of bf16."""
    dec, W0, b0, gamma, beta = _decode_case(795, 24, 2, 4, 64, "bf16", "ident")
    full = _steps_run(W0, b0, dec, gamma, beta, 1e-6)
    again = _steps_run(W0, b0, dec, gamma, beta, 1e-6)
    for a, b in zip(full, again):
        assert np.array_equal(a, b)
    cut = lambda lo, hi: gen.DecodeInputs(hi - lo, dec.B, dec.H, dec.d, dec.io, dec.XQ[lo:hi],
                                          dec.XK[lo:hi], dec.XV[lo:hi], dec.eta[lo:hi])
    O1, W1, b1 = _steps_run(W0, b0, cut(0, 10), gamma, beta, 1e-6)
    O2, W2, b2 = _steps_run(W1, b1, cut(10, 24), gamma, beta, 1e-6)
    err = P.errors((np.concatenate([O1, O2], 2), W2, b2), full, 8, LIN_NAMES)
    _report("decode_steps split vs one call", err)
    assert err["W_out"] <= 1e-6 and err["b_out"] <= 1e-6, err
    assert err["O"] <= 2.0 ** -7, err


def test_decode_steps_full_workload5():
    """Workload 5's 1024 decode steps for 64 x 32 states in one call."""
    pre, dec = gen.make_workload(5)
    _, Wp, bp = P.linear_gpu(pre)
    rW, rb = P.linear_oracle(pre)[1:]
    W0 = np.broadcast_to(Wp[0], (64,) + Wp.shape[1:]).astype(np.float32)
    b0 = np.broadcast_to(bp[0], (64,) + bp.shape[1:]).astype(np.float32)
    got = _steps_run(W0, b0, dec, pre.gamma, pre.beta, pre.eps)
    ref = _decode_oracle(np.broadcast_to(rW[0], W0.shape), np.broadcast_to(rb[0], b0.shape),
                         dec, pre.gamma, pre.beta, pre.eps)
    err = P.errors(got, ref, 64 * 32, LIN_NAMES)
    _report("workload5 decode_steps 64x1024", err)
    assert max(err.values()) <= P.TOL["bf16"], err


@pytest.mark.parametrize("mb", [8, 13])
def test_linear_bf16_other_minibatch(mb):
    """Mini-batch sizes other than 16 (VALU path) with bf16 storage."""
    x = gen.make_linear(800 + mb, 2, 3, 16 * 6 + 3, 64, io="bf16", ln_random=True)
    _check_linear(x, f"bf16 mb{mb}", mb=mb)


# ---------------------------------------------------------------------------
# Mini-batch decode (b = mb > 1): prefill + decode calls = one prefill over
# the whole sequence with chunks aligned at its first token
# ---------------------------------------------------------------------------
def _mb_case(seed, io, d, B=2, H=3):
    return gen.make_linear(seed, B, H, 0, d, io=io, ln_random=True, b_random=True, w_std=0.3)


@pytest.mark.parametrize("io,d", [("bf16", 64), ("f32", 64), ("f32", 16), ("bf16", 16)])
@pytest.mark.parametrize("mb", [4, 16])
def test_decode_steps_mb_continues_the_prefill(io, d, mb):
    """Prefill 2 chunks, then decode 2.5 chunks in three calls that end and
    resume inside a chunk; the outputs and both states against the oracle's
    prefill over the whole sequence (its chunk-start state at the end)."""
    B, H, L0 = 2, 3, 2 * mb
    splits = [mb // 2 + 1, mb + 1, mb - 2]           # 2.5 chunks, ends mid-chunk
    T = sum(splits)
    x = gen.make_linear(700 + 3 * d + mb, B, H, L0 + T, d, io=io, ln_random=True, b_random=True,
                        w_std=0.3)
    dt = P.io_dtype(io)
    pre = dict(XQ=x.XQ[:, :, :L0], XK=x.XK[:, :, :L0], XV=x.XV[:, :, :L0], eta=x.eta[:, :, :L0])
    O0, W, b = ttt.ttt_linear_forward(*(P.dev(pre[k], dt) for k in ("XQ", "XK", "XV")),
                                      P.dev(pre["eta"]), P.dev(x.W0), P.dev(x.b0), P.dev(x.gamma),
                                      P.dev(x.beta), mb=mb, ln_eps=x.eps)
    Wc = torch.full_like(W, float("nan"))  # not read at pos = 0
    bc = torch.full_like(b, float("nan"))
    step = lambda a: np.ascontiguousarray(np.moveaxis(a, 2, 0))   # [B,H,T,...] -> [T,B,H,...]
    outs, t, pos = [], L0, 0
    for n in splits:
        sl = slice(t, t + n)
        o = ttt.ttt_decode_steps_mb(P.dev(step(x.XQ[:, :, sl]), dt), P.dev(step(x.XK[:, :, sl]), dt),
                                    P.dev(step(x.XV[:, :, sl]), dt), P.dev(step(x.eta[:, :, sl])),
                                    Wc, bc, W, b, P.dev(x.gamma), P.dev(x.beta), mb=mb, pos=pos,
                                    ln_eps=x.eps)
        outs.append(np.moveaxis(P.to_np(o), 0, 2))
        t, pos = t + n, (pos + n) % mb
    torch.cuda.synchronize()
    O_ref, W_ref, b_ref = oracle.linear_forward(x.XQ, x.XK, x.XV, x.eta, x.W0, x.b0, x.gamma,
                                                x.beta, x.eps, mb=mb)
    # chunk-start state of the last (partial) chunk: the oracle run up to its start
    Lc = L0 + T - pos
    _, Wc_ref, bc_ref = oracle.linear_forward(x.XQ[:, :, :Lc], x.XK[:, :, :Lc], x.XV[:, :, :Lc],
                                              x.eta[:, :, :Lc], x.W0, x.b0, x.gamma, x.beta,
                                              x.eps, mb=mb)
    got = (np.concatenate(outs, 2), P.to_np(W), P.to_np(b), P.to_np(Wc), P.to_np(bc))
    ref = (O_ref[:, :, L0:], W_ref, b_ref, Wc_ref, bc_ref)
    err = P.errors(got, ref, B * H, ("o", "W", "b", "W_chunk", "b_chunk"))
    _report(f"decode mb={mb} {io} d{d}", err)
    assert max(err.values()) <= P.TOL[io], err


def test_decode_steps_mb1_is_decode_steps():
    """mb = 1 ignores the chunk state and equals ttt_decode_steps bit for bit."""
    x = gen.make_linear(760, 2, 3, 9, 64, io="bf16", ln_random=True, b_random=True, w_std=0.3)
    dt = torch.bfloat16
    step = lambda a: P.dev(np.ascontiguousarray(np.moveaxis(a, 2, 0)), dt)
    args = (step(x.XQ), step(x.XK), step(x.XV),
            P.dev(np.ascontiguousarray(np.moveaxis(x.eta, 2, 0))))
    W0 = np.broadcast_to(x.W0, (2, 3, 64, 64)).copy()
    b0 = np.broadcast_to(x.b0, (2, 3, 64)).copy()
    Wa, ba, Wb, bb = P.dev(W0), P.dev(b0), P.dev(W0), P.dev(b0)
    oa = ttt.ttt_decode_steps(*args, Wa, ba, P.dev(x.gamma), P.dev(x.beta), ln_eps=x.eps)
    ob = ttt.ttt_decode_steps_mb(*args, torch.empty_like(Wb), torch.empty_like(bb), Wb, bb,
                                 P.dev(x.gamma), P.dev(x.beta), mb=1, ln_eps=x.eps)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(Wa, Wb) and torch.equal(ba, bb)


def test_decode_steps_mb_zero_steps_leaves_state():
    """T = 0 touches neither state."""
    rng = np.random.default_rng(765)
    W = P.dev(rng.standard_normal((2, 3, 64, 64)).astype(np.float32))
    b = P.dev(rng.standard_normal((2, 3, 64)).astype(np.float32))
    Wc, bc = W.clone() * 2, b.clone() * 2
    W1, b1, Wc1, bc1 = W.clone(), b.clone(), Wc.clone(), bc.clone()
    e = torch.empty((0, 2, 3, 64), device="cuda", dtype=torch.bfloat16)
    ttt.ttt_decode_steps_mb(e, e, e, torch.empty((0, 2, 3), device="cuda"), Wc, bc, W, b,
                            P.dev(np.ones((3, 64), np.float32)), P.dev(np.zeros((3, 64), np.float32)),
                            mb=16, pos=5)
    torch.cuda.synchronize()
    assert torch.equal(W, W1) and torch.equal(b, b1) and torch.equal(Wc, Wc1) and torch.equal(bc, bc1)


def test_decode_steps_mb16_full_workload5():
    """Workload 5's 1024 decode tokens on 64 x 32 states under the mini-batch
    rule with b = 16 in one call (the benchmark's launch), from per-state start
    states: outputs, final state and the last chunk's start state against the
    oracle's b = 16 recurrence over the same tokens."""
    _, dec = gen.make_workload(5)
    rng = np.random.default_rng(56)
    W0 = (0.3 * rng.standard_normal((dec.B, dec.H, dec.d, dec.d))).astype(np.float32)
    b0 = (0.1 * rng.standard_normal((dec.B, dec.H, dec.d))).astype(np.float32)
    g, be = np.ones((dec.H, dec.d), np.float32), np.zeros((dec.H, dec.d), np.float32)
    dt = P.io_dtype(dec.io)
    W, b = P.dev(W0), P.dev(b0)
    Wc, bc = torch.full_like(W, float("nan")), torch.full_like(b, float("nan"))  # unread at pos 0
    o = ttt.ttt_decode_steps_mb(P.dev(dec.XQ, dt), P.dev(dec.XK, dt), P.dev(dec.XV, dt),
                                P.dev(dec.eta), Wc, bc, W, b, P.dev(g), P.dev(be), mb=16, pos=0)
    torch.cuda.synchronize()
    tr = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))  # step-major -> [B,H,T,...]
    xs = [tr(a) for a in (dec.XQ, dec.XK, dec.XV, dec.eta)]
    O_ref, W_ref, b_ref = oracle.linear_forward(*xs, W0, b0, g, be, 1e-6, mb=16, w0_batched=True)
    Lc = dec.steps - 16  # start of the last chunk
    _, Wc_ref, bc_ref = oracle.linear_forward(*(a[:, :, :Lc] for a in xs), W0, b0, g, be, 1e-6,
                                              mb=16, w0_batched=True)
    got = (tr(P.to_np(o)), P.to_np(W), P.to_np(b), P.to_np(Wc), P.to_np(bc))
    err = P.errors(got, (O_ref, W_ref, b_ref, Wc_ref, bc_ref), dec.B * dec.H,
                   ("o", "W", "b", "W_chunk", "b_chunk"))
    _report("workload5 decode_steps_mb b=16 64x32x1024", err)
    assert max(err.values()) <= P.TOL["bf16"], err
