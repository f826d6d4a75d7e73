"""GPU parity of ttt_qkv_project (the input projections of the layer, lryc.cn
TTT article §2.2; views XQ, XK, XV of the damodev.csdn.net deep-dive §4.2)
against the fp64 oracle.

Bar: the kernel multiplies bf16 values exactly, sums in fp32 and rounds the
result to bf16 once, so every output is within half a bf16 ulp of the exact
sum (relative 2^-8) plus the fp32 summation error, which is below
d_model * 2^-24 * sum_k |x_k theta_k|. Each output is checked against
2^-8 |ref| + d_model * 2^-24 * sum_k |x_k theta_k|; the max relative error
per (view, b, h) slice is reported and held to the bf16 bar of 2e-2."""
import numpy as np
import pytest
import torch

import oracle
from test_sequence_layer_ttt_amd import gen, ttt
from tests import parity as P

pytestmark = pytest.mark.gpu


def _run(x):
    X = P.dev(x.X, torch.bfloat16)
    th = P.dev(x.theta, torch.bfloat16)
    out = ttt.ttt_qkv_project(X, th, x.H)
    torch.cuda.synchronize()
    return [P.to_np(o) for o in out]


def _bound(x, idx):
    """Elementwise bound at outputs idx (view, b, h, t, j)."""
    v, b, h, t, j = idx.T
    rows = x.theta[v, h * x.d + j].astype(np.float64)
    xs = x.X[b, t].astype(np.float64)
    s = np.abs(rows * xs).sum(1)
    return s * x.dm * 2.0 ** -24


@pytest.mark.parametrize("B,L,dm,H", [(1, 1, 64, 1), (2, 300, 128, 2), (1, 257, 192, 4), (3, 40, 64, 3)])
def test_proj_small_vs_oracle(B, L, dm, H):
    """Several tiles and ragged edges: tokens B L not a multiple of 256,
    features 3 H 64 not a multiple of 256, d_model = 1, 2, 3 steps of 64."""
    x = gen.make_proj(11 + B + H, B, L, dm, H, 64)
    got = _run(x)
    ref = oracle.qkv_project(x.X, x.theta, H)
    for v in range(3):
        g, r = got[v], ref[v]
        b_, h_, t_, j_ = np.meshgrid(np.arange(B), np.arange(H), np.arange(L), np.arange(64), indexing="ij")
        idx = np.stack([np.full(b_.size, v), b_.ravel(), h_.ravel(), t_.ravel(), j_.ravel()], axis=1)
        tol = 2.0 ** -8 * np.abs(r.ravel()) + _bound(x, idx)
        err = np.abs(g.ravel() - r.ravel())
        assert (err <= tol).all(), (v, float((err - tol).max()))
        assert P.max_rel(g, r, B * H) < 2e-2


@pytest.mark.parametrize("num", [2, 3])
def test_proj_full_workload_sampled(num):
    """Workload 2 (B4 L2048, model width 768) and workload 3 (B2 L8192, model
    width 2048), in the launch the benchmark times; 8192 sampled outputs
    checked one by one against the oracle's sums."""
    x = gen.make_proj_workload(num)
    got = _run(x)
    rng = np.random.default_rng(num)
    n = 8192
    idx = np.stack([rng.integers(0, 3, n), rng.integers(0, x.B, n), rng.integers(0, x.H, n),
                    rng.integers(0, x.L, n), rng.integers(0, 64, n)], axis=1)
    # always include the first and last token and feature of every view
    corners = [[v, b, h, t, j] for v in range(3) for b in (0, x.B - 1) for h in (0, x.H - 1)
               for t in (0, x.L - 1) for j in (0, 63)]
    idx = np.concatenate([idx, np.array(corners)], axis=0).astype(np.int32)
    ref = oracle.qkv_project_at(x.X, x.theta, x.H, idx)
    g = np.array([got[v][b, h, t, j] for v, b, h, t, j in idx])
    tol = 2.0 ** -8 * np.abs(ref) + _bound(x, idx)
    err = np.abs(g - ref)
    assert (err <= tol).all(), float((err - tol).max())
    assert float(err.max() / np.abs(ref).max()) < 2e-2


def test_proj_empty_is_a_no_op():
    X = torch.empty((2, 0, 64), device="cuda", dtype=torch.bfloat16)
    th = torch.zeros((3, 64, 64), device="cuda", dtype=torch.bfloat16)
    q, k, v = ttt.ttt_qkv_project(X, th, 1)
    assert q.numel() == 0 and k.numel() == 0 and v.numel() == 0


def test_proj_repeatable():
    x = gen.make_proj(5, 2, 300, 128, 2, 64)
    a = _run(x)
    b = _run(x)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
