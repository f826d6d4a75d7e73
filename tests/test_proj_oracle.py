"""Pins of the projection oracle (oracle.qkv_project): the key, value and
query views of the layer input, lryc.cn TTT article §2.2 (the outer loop
learns theta_K, theta_V, theta_Q), fed to the inner loop as XQ, XK, XV
(damodev.csdn.net deep-dive §4.2). CPU only."""
import numpy as np
import pytest

import oracle
from test_sequence_layer_ttt_amd import gen


def _views_by_matmul(X, theta, H):
    """NumPy fp64 matmul (a library primitive) per view, then the head split."""
    B, L, dm = X.shape
    d = theta.shape[1] // H
    return tuple((X.astype(np.float64) @ theta[v].astype(np.float64).T)
                 .reshape(B, L, H, d).transpose(0, 2, 1, 3) for v in range(3))


@pytest.mark.parametrize("B,L,dm,H,d", [(1, 1, 64, 1, 64), (2, 37, 128, 2, 64), (1, 19, 96, 3, 16)])
def test_matches_numpy_matmul(B, L, dm, H, d):
    x = gen.make_proj(7, B, L, dm, H, d)
    got = oracle.qkv_project(x.X, x.theta, H)
    ref = _views_by_matmul(x.X, x.theta, H)
    for g, r in zip(got, ref):
        assert g.shape == (B, H, L, d)
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_identity_projection_splits_heads():
    """theta_Q = I (d_model = H d): XQ[b,h,t,j] = X[b,t,h d + j] exactly; the
    three views use theta[0], theta[1], theta[2] in that order."""
    B, L, H, d = 2, 5, 3, 16
    dm = H * d
    rng = np.random.default_rng(1)
    X = rng.standard_normal((B, L, dm))
    theta = np.stack([np.eye(dm), 2.0 * np.eye(dm), np.eye(dm)[::-1]])
    q, k, v = oracle.qkv_project(X, theta, H)
    for h in range(H):
        np.testing.assert_array_equal(q[:, h], X[:, :, h * d:(h + 1) * d])
        np.testing.assert_array_equal(k[:, h], 2.0 * X[:, :, h * d:(h + 1) * d])
    # reversed identity: output feature n reads input feature dm - 1 - n
    Xr = X[:, :, ::-1]
    for h in range(H):
        np.testing.assert_array_equal(v[:, h], Xr[:, :, h * d:(h + 1) * d])


def test_at_agrees_with_full():
    x = gen.make_proj(3, 2, 33, 128, 2, 64)
    full = oracle.qkv_project(x.X, x.theta, 2)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.integers(0, 3, 200), rng.integers(0, 2, 200), rng.integers(0, 2, 200),
                    rng.integers(0, 33, 200), rng.integers(0, 64, 200)], axis=1)
    at = oracle.qkv_project_at(x.X, x.theta, 2, idx)
    ref = np.array([full[v][b, h, t, j] for v, b, h, t, j in idx])
    np.testing.assert_array_equal(at, ref)


def test_rejects_bad_index():
    x = gen.make_proj(3, 1, 4, 64, 1, 64)
    with pytest.raises(ValueError):
        oracle.qkv_project_at(x.X, x.theta, 1, [[3, 0, 0, 0, 0]])
    with pytest.raises(ValueError):
        oracle.qkv_project_at(x.X, x.theta, 1, [[0, 0, 0, 4, 0]])


def test_generator_shapes_and_scale():
    x = gen.make_proj_workload(3, L=64)
    assert x.X.shape == (2, 64, 2048) and x.theta.shape == (3, 2048, 2048)
    assert abs(float(x.theta.std()) - 0.02) < 1e-3
    assert np.array_equal(gen.round_bf16(x.X), x.X)
