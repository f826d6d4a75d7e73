"""fp32 emulation (NumPy, CPU) of the layer-norm statistics the kernels form,
on rows whose mean is large against their spread.

The layer norm is the one of the LN-residual output (lryc.cn TTT article,
§2.1) and of the fused LN + L2 backward (damodev.csdn.net TTT deep-dive, §4.2);
both need 1/sqrt(var + eps) per row of 64 features. Sums are emulated as the
kernels form them: float32 butterflies over the 64 features (the DPP and lane
swap reductions add pairs), every operation rounded to float32. Reference:
float64 on the same float32 inputs.

  * one pass, E[z^2] - mean(z)^2 on raw rows: loses ~(mean / spread)^2 * 2^-24
    of the variance -- the formula no kernel uses any more;
  * the bf16 MFMA prefill: the same one-pass sums, but z comes from the
    centred state W - wbar 1^T, b - bbar, so its rows have a mean near zero;
  * the resident decode: the mean first, then sums of centred values;
  * the fp32 VALU kernels: the mean, the mean of the centred values (the first
    mean's rounding error), then the variance of the corrected values.
"""
import numpy as np
import pytest

f32 = np.float32


def tree_sum(x):
    """float32 pairwise sum over the last axis (length a power of two)."""
    x = np.asarray(x, f32)
    while x.shape[-1] > 1:
        x = (x[..., 0::2] + x[..., 1::2]).astype(f32)
    return x[..., 0]


def rstd_ref(z):
    z = np.asarray(z, np.float64)
    return 1.0 / np.sqrt(z.var(-1) + 1e-6)


def rel(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - b) / np.abs(b)))


def rows(m, s, n=512, seed=0):
    rng = np.random.default_rng(seed)
    return (m + s * rng.standard_normal((n, 64))).astype(f32)


def one_pass(z):
    inv = f32(1 / 64)
    mu = (tree_sum(z) * inv).astype(f32)
    var = np.maximum((tree_sum((z * z).astype(f32)) * inv - mu * mu).astype(f32), f32(0))
    return (1 / np.sqrt(var.astype(np.float64) + 1e-6))


def two_round(z):
    inv = f32(1 / 64)
    mu = (tree_sum(z) * inv).astype(f32)
    c = (z - mu[:, None]).astype(f32)
    return 1 / np.sqrt((tree_sum((c * c).astype(f32)) * inv).astype(np.float64) + 1e-6)


def three_round(z):
    inv = f32(1 / 64)
    m1 = (tree_sum(z) * inv).astype(f32)
    c = (z - m1[:, None]).astype(f32)
    dm = (tree_sum(c) * inv).astype(f32)
    c = (c - dm[:, None]).astype(f32)
    return 1 / np.sqrt((tree_sum((c * c).astype(f32)) * inv).astype(np.float64) + 1e-6)


def test_one_pass_formula_fails_on_offset_rows():
    """Why the kernels changed: at mean 100 and spread 0.2 the raw one-pass
    variance is off by several per cent."""
    z = rows(100.0, 0.2)
    assert rel(one_pass(z), rstd_ref(z)) > 1e-2
    z = rows(0.0, 0.2)
    assert rel(one_pass(z), rstd_ref(z)) < 1e-5


@pytest.mark.parametrize("m", [10.0, 100.0])
def test_two_round_sums(m):
    """Resident decode and the MLP's row-layout layer norms."""
    z = rows(m, 0.2, seed=int(m))
    assert rel(two_round(z), rstd_ref(z)) < 1e-4


@pytest.mark.parametrize("m", [10.0, 100.0, 1000.0])
def test_three_round_sums(m):
    """fp32 VALU kernels: the corrected mean keeps 1e-6 even at mean 1000."""
    z = rows(m, 0.2, seed=int(m) + 1)
    assert rel(three_round(z), rstd_ref(z)) < 2e-6


@pytest.mark.parametrize("c", [10.0, 100.0])
def test_centred_state_one_pass(c):
    """The bf16 MFMA prefill: z = XK (W - wbar 1^T) + (b - bbar) in fp32 with
    the state's row means removed, then the one-pass sums. W0 carries row
    offsets and b0 the offset c; the reference is the variance of the exact
    rows XK W + b."""
    rng = np.random.default_rng(7)
    XK = rng.standard_normal((256, 64)).astype(f32)
    W = (0.02 * rng.standard_normal((64, 64)) + rng.standard_normal((64, 1))).astype(f32)
    b = (c + 0.02 * rng.standard_normal(64)).astype(f32)
    wbar = (tree_sum(W) * f32(1 / 64)).astype(f32)
    bbar = f32(tree_sum(b) * f32(1 / 64))
    Wc = (W - wbar[:, None]).astype(f32)
    bc = (b - bbar).astype(f32)
    zc = (XK @ Wc + bc).astype(f32)
    exact = XK.astype(np.float64) @ W.astype(np.float64) + b.astype(np.float64)
    # the raw rows' one-pass variance is useless here
    zr = (XK @ W + b).astype(f32)
    assert rel(one_pass(zr), rstd_ref(exact)) > 1e-3
    assert rel(one_pass(zc), rstd_ref(exact)) < 1e-4
