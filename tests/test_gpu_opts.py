"""GPU parity of ttt_linear_forward_opts and ttt_mlp_forward_opts (the
Modular-TTT options: inner loss and weight decay on the weight matrices)
through the C ABI against the fp64 oracle's linear_forward_opts /
mlp_forward_opts on the same inputs. bf16 storage with d = 64 and b = 16
runs the MFMA prefills (both layer-norm paths: general gamma/beta and
gamma = 1, beta = 0); the other shapes run the fp32 VALU prefills."""
import numpy as np
import pytest
import torch

import oracle
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu

NAMES = ("O", "W_out", "b_out")


def _run(x, loss, wd, mb):
    dt = P.io_dtype(x.io)
    O, W, b = ttt.ttt_linear_forward_opts(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt),
                                          P.dev(x.eta), P.dev(x.W0), P.dev(x.b0), P.dev(x.gamma),
                                          P.dev(x.beta), inner_loss=loss, weight_decay=wd, mb=mb,
                                          ln_eps=x.eps)
    torch.cuda.synchronize()
    return P.to_np(O), P.to_np(W), P.to_np(b)


def _ref(x, loss, wd, mb):
    return oracle.linear_forward_opts(x.XQ, x.XK, x.XV, x.eta, x.W0, x.b0, x.gamma, x.beta, x.eps,
                                      mb=mb, loss=loss, weight_decay=wd)


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.5])
@pytest.mark.parametrize("io,d,mb,L", [("f32", 16, 16, 64), ("f32", 64, 16, 16 * 5 + 3),
                                       ("bf16", 64, 16, 16 * 6 + 5), ("bf16", 64, 5, 23),
                                       ("f32", 16, 1, 9)])
def test_options(loss, wd, io, d, mb, L):
    x = gen.make_linear(600 + d + L + mb, 2, 3, L, d, io=io, ln_random=True, b_random=True,
                        w_std=0.3)
    got, ref = _run(x, loss, wd, mb), _ref(x, loss, wd, mb)
    err = P.errors(got, ref, x.B * x.H, NAMES)
    print(f"[parity] opts {loss} wd={wd} {io} d{d} mb{mb} L{L}: "
          + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.5])
def test_options_mfma_identity_layer_norm(loss, wd):
    """gamma = 1, beta = 0 takes the MFMA kernel's three-sum layer-norm path."""
    x = gen.make_linear(650, 2, 3, 16 * 9 + 7, 64, io="bf16", b_random=True, w_std=0.3)
    got, ref = _run(x, loss, wd, 16), _ref(x, loss, wd, 16)
    err = P.errors(got, ref, x.B * x.H, NAMES)
    print(f"[parity] opts mfma ident {loss} wd={wd}: "
          + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_defaults_run_the_plain_kernels():
    """TTT_LOSS_MSE with no decay is ttt_linear_forward (same kernel, same bits)."""
    x = gen.make_workload(3, L=16 * 9 + 3, B=2, H=3)
    a = _run(x, "mse", 0.0, 16)
    b = P.linear_gpu(x)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_workload3_shape_sampled_heads():
    """Workload 3's shape (B=2, H=32, L=8192, bf16) with the inner-product loss
    and weight decay 0.5; the oracle checks batch 1, heads 5 and 30."""
    full = gen.make_workload(3)
    got = _run(full, "inner_product", 0.5, 16)
    hs = [5, 30]
    sl = lambda a: np.ascontiguousarray(a[1:2, hs])
    ref = oracle.linear_forward_opts(sl(full.XQ), sl(full.XK), sl(full.XV), sl(full.eta),
                                     np.ascontiguousarray(full.W0[hs]),
                                     np.ascontiguousarray(full.b0[hs]),
                                     np.ascontiguousarray(full.gamma[hs]),
                                     np.ascontiguousarray(full.beta[hs]), full.eps, mb=16,
                                     loss="inner_product", weight_decay=0.5)
    err = P.errors(tuple(sl(g) for g in got), ref, 2, NAMES)
    print("[parity] opts workload3 shape: " + " ".join(f"{k}={v:.2e}" for k, v in err.items()),
          flush=True)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_options_empty_sequence():
    """L = 0 with both options: the final state is the initial one."""
    x = gen.make_linear(660, 2, 3, 0, 64, io="bf16", b_random=True)
    O, W, b = _run(x, "inner_product", 0.5, 16)
    assert O.shape == (2, 3, 0, 64)
    assert np.array_equal(W, np.broadcast_to(x.W0, W.shape))
    assert np.array_equal(b, np.broadcast_to(x.b0, b.shape))


# ---------------------------------------------------------------------------
# TTT-MLP with the same options (ttt_mlp_forward_opts against the oracle's
# mlp_forward_opts). bf16 with b = 16 runs the MFMA kernel, other shapes the
# fp32 VALU kernel.
# ---------------------------------------------------------------------------
MLP_NAMES = ("O", "W1_out", "b1_out", "W2_out", "b2_out")


def _mlp_run(x, loss, wd, mb):
    dt = P.io_dtype(x.io)
    out = ttt.ttt_mlp_forward_opts(P.dev(x.XQ, dt), P.dev(x.XK, dt), P.dev(x.XV, dt),
                                   P.dev(x.eta), P.dev(x.W1), P.dev(x.b1), P.dev(x.W2),
                                   P.dev(x.b2), P.dev(x.gamma), P.dev(x.beta), inner_loss=loss,
                                   weight_decay=wd, mb=mb, ln_eps=x.eps)
    torch.cuda.synchronize()
    return tuple(P.to_np(t) for t in out)


def _mlp_ref(x, loss, wd, mb):
    return oracle.mlp_forward_opts(x.XQ, x.XK, x.XV, x.eta, x.W1, x.b1, x.W2, x.b2, x.gamma,
                                   x.beta, x.eps, mb=mb, loss=loss, weight_decay=wd)


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.5])
@pytest.mark.parametrize("io,mb,L", [("bf16", 16, 16 * 5 + 9), ("f32", 16, 16 * 3 + 5),
                                     ("bf16", 5, 23), ("f32", 1, 7)])
def test_mlp_options(loss, wd, io, mb, L):
    x = gen.make_mlp(700 + mb + L, 2, 2, L, 64, io=io, ln_random=True, b_random=True)
    got, ref = _mlp_run(x, loss, wd, mb), _mlp_ref(x, loss, wd, mb)
    err = P.errors(got, ref, x.B * x.H, MLP_NAMES)
    print(f"[parity] mlp opts {loss} wd={wd} {io} mb{mb} L{L}: "
          + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= P.TOL[io], err


@pytest.mark.parametrize("loss", ["mse", "inner_product"])
@pytest.mark.parametrize("wd", [0.0, 0.5])
def test_mlp_options_mfma_identity_layer_norm(loss, wd):
    """gamma = 1, beta = 0 takes the MFMA kernel's one-round layer-norm path."""
    x = gen.make_mlp(750, 2, 3, 16 * 7 + 11, 64, io="bf16", b_random=True)
    got, ref = _mlp_run(x, loss, wd, 16), _mlp_ref(x, loss, wd, 16)
    err = P.errors(got, ref, x.B * x.H, MLP_NAMES)
    print(f"[parity] mlp opts mfma ident {loss} wd={wd}: "
          + " ".join(f"{k}={v:.2e}" for k, v in err.items()), flush=True)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_mlp_defaults_run_the_plain_kernels():
    """TTT_LOSS_MSE with no decay is ttt_mlp_forward (same kernel, same bits)."""
    x = gen.make_workload(4, L=16 * 9 + 3, B=2, H=3)
    a = _mlp_run(x, "mse", 0.0, 16)
    b = P.mlp_gpu(x)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_mlp_workload4_shape_sampled_heads():
    """Workload 4's shape (B=2, H=12, L=8192, bf16) with the inner-product loss
    and weight decay 0.5; the oracle checks batch 0, heads 2 and 11."""
    full = gen.make_workload(4)
    got = _mlp_run(full, "inner_product", 0.5, 16)
    hs = [2, 11]
    sl = lambda a: np.ascontiguousarray(a[0:1, hs])
    hp = lambda a: np.ascontiguousarray(a[hs])
    ref = oracle.mlp_forward_opts(sl(full.XQ), sl(full.XK), sl(full.XV), sl(full.eta),
                                  hp(full.W1), hp(full.b1), hp(full.W2), hp(full.b2),
                                  hp(full.gamma), hp(full.beta), full.eps, mb=16,
                                  loss="inner_product", weight_decay=0.5)
    err = P.errors(tuple(sl(g) for g in got), ref, 2, MLP_NAMES)
    print("[parity] mlp opts workload4 shape: " + " ".join(f"{k}={v:.2e}" for k, v in err.items()),
          flush=True)
    assert max(err.values()) <= P.TOL["bf16"], err


def test_mlp_options_empty_sequence():
    """L = 0 with both options: the final state is the initial one."""
    x = gen.make_mlp(760, 2, 3, 0, 64, io="bf16", b_random=True)
    got = _mlp_run(x, "inner_product", 0.5, 16)
    assert got[0].shape == (2, 3, 0, 64)
    for g_, r_ in zip(got[1:], (x.W1, x.b1, x.W2, x.b2)):
        assert np.array_equal(g_, np.broadcast_to(r_, g_.shape))


@pytest.mark.parametrize("L", [1, 15, 17])
def test_options_mfma_lengths_around_one_chunk(L):
    """Both options on the MFMA prefills (bf16, b = 16) with a single partial
    chunk, one chunk short of a full one, and one token past it."""
    x = gen.make_linear(670 + L, 2, 3, L, 64, io="bf16", ln_random=True, b_random=True, w_std=0.3)
    err = P.errors(_run(x, "inner_product", 0.5, 16), _ref(x, "inner_product", 0.5, 16), 6, NAMES)
    xm = gen.make_mlp(770 + L, 2, 3, L, 64, io="bf16", ln_random=True, b_random=True)
    err_m = P.errors(_mlp_run(xm, "inner_product", 0.5, 16), _mlp_ref(xm, "inner_product", 0.5, 16),
                     6, MLP_NAMES)
    print(f"[parity] opts L{L}: linear " + " ".join(f"{k}={v:.2e}" for k, v in err.items())
          + " | mlp " + " ".join(f"{k}={v:.2e}" for k, v in err_m.items()), flush=True)
    assert max(err.values()) <= P.TOL["bf16"], err
    assert max(err_m.values()) <= P.TOL["bf16"], err_m
