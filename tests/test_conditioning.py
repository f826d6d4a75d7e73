"""Conditioning floor of the chunk chain (CPU): how far two correct
computations of the same TTT-Linear prefill drift apart over a full-length
sequence, before any kernel is judged.

  (i)  the fp64 oracle against itself with W0 moved by one fp32 ulp;
  (ii) an emulation of the dual form (damodev.csdn.net deep-dive §4.2, with
       the LN-residual output of the lryc.cn article §2.1) in fp32 with every
       product operand rounded to bfloat16 -- the precision the bf16 kernels
       compute in -- against the fp64 oracle.

One head of workloads 2, 3 and 5 (prefill) at full length (128, 512 and 2048
chunks). The error is the per-output metric of the parity tests (max |diff| /
max |ref|), taken per chunk for O; the assertions say the chain does not
amplify rounding (late chunks no worse than early ones) and that the bf16
bar of 2e-2 is reachable by a correct computation. The per-chunk profile is
printed (run with -s to see it)."""
import numpy as np
import pytest

import oracle
from test_sequence_layer_ttt_amd import gen


def _rbf(a):
    return gen.round_bf16(np.asarray(a, np.float32))


def _ln_stats(z, eps):
    mu = z.mean(-1, keepdims=True, dtype=np.float32)
    c = (z - mu).astype(np.float32)
    sig = np.sqrt((c * c).mean(-1, keepdims=True, dtype=np.float32) + np.float32(eps)).astype(np.float32)
    return c / sig, sig


def _emulate_bf16(x, L):
    """Dual-form chunk recurrence in fp32, product operands rounded to bf16
    (XK, XQ, W, E and the token-token matrices), gamma = 1, beta = 0."""
    f32 = np.float32
    XQ, XK, XV, eta = (np.asarray(a, f32) for a in (x.XQ[0, 0, :L], x.XK[0, 0, :L], x.XV[0, 0, :L], x.eta[0, 0, :L]))
    W = np.asarray(x.W0[0], f32).copy()
    b = np.asarray(x.b0[0], f32).copy()
    eps = x.eps
    O = np.empty((L, XQ.shape[1]), f32)
    for c0 in range(0, L, 16):
        q, k, v, e = XQ[c0:c0 + 16], XK[c0:c0 + 16], XV[c0:c0 + 16], eta[c0:c0 + 16]
        Wb = _rbf(W)
        Z = (_rbf(k) @ Wb + b).astype(f32)
        xh, sig = _ln_stats(Z, eps)
        gh = (xh - (v - k)).astype(f32)
        G = ((gh - gh.mean(-1, keepdims=True) - xh * (gh * xh).mean(-1, keepdims=True)) / sig).astype(f32)
        E = (-e[:, None] * G).astype(f32)
        Eb = _rbf(E)
        T = np.tril(_rbf(_rbf(q) @ _rbf(k).T + f32(1.0)))
        Zb = (_rbf(q) @ Wb + b + T @ Eb).astype(f32)
        xb, _ = _ln_stats(Zb, eps)
        O[c0:c0 + 16] = q + xb
        W = (W + _rbf(k).T @ Eb).astype(f32)
        b = (b + E.sum(0, dtype=f32)).astype(f32)
    return O, W, b


def _oracle_head(x, L, W0=None):
    sl = lambda a: np.ascontiguousarray(a[:1, :1, :L])
    W0 = x.W0[:1] if W0 is None else W0
    return oracle.linear_forward(sl(x.XQ), sl(x.XK), sl(x.XV), sl(x.eta), W0, x.b0[:1], x.gamma[:1],
                                 x.beta[:1], x.eps, mb=16)


def _per_chunk(got, ref):
    """O error per chunk: max |diff| over the chunk / max |ref| over the sequence."""
    d = np.abs(np.asarray(got, np.float64) - ref).reshape(-1, 16, ref.shape[-1]).max((1, 2))
    return d / np.abs(ref).max()


def _rel(got, ref):
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / np.abs(ref).max())


@pytest.mark.parametrize("num", [2, 3, 5])
def test_conditioning_floor(num):
    w = gen.WORKLOADS[num]
    x = gen.make_workload(num, B=1, H=1) if num != 5 else gen.make_workload(5, B=1, H=1, decode_steps=1)[0]
    L = w.L
    O, W, b = _oracle_head(x, L)
    O = O[0, 0]
    # (i) W0 moved by one fp32 ulp (every element, upwards)
    W0p = np.nextafter(np.asarray(x.W0[:1], np.float32), np.float32(np.inf))
    Op, Wp, bp = _oracle_head(x, L, W0=W0p)
    pc = _per_chunk(Op[0, 0], O)
    e_ulp = (_rel(Op, O[None, None]), _rel(Wp, W), _rel(bp, b))
    # (ii) fp32 with bf16 product operands
    Oe, We, be = _emulate_bf16(x, L)
    pe = _per_chunk(Oe, O)
    e_bf = (_rel(Oe, O), _rel(We, W[0, 0]), _rel(be, b[0, 0]))
    q = len(pe) // 4
    print(f"\nworkload {num} (L={L}, {len(pe)} chunks)")
    print(f"  W0 + 1 ulp: O {e_ulp[0]:.2e}  W {e_ulp[1]:.2e}  b {e_ulp[2]:.2e};  O per chunk: first "
          f"{pc[0]:.1e}, quarters {[f'{pc[i * q:(i + 1) * q].max():.1e}' for i in range(4)]}")
    print(f"  bf16 operands: O {e_bf[0]:.2e}  W {e_bf[1]:.2e}  b {e_bf[2]:.2e};  O per chunk by quarter "
          f"{[f'{pe[i * q:(i + 1) * q].max():.1e}' for i in range(4)]}")
    # a one-ulp change of the initial state stays at the rounding level: no amplification
    assert max(e_ulp) < 1e-5
    assert pc[-q:].max() <= 2 * pc[:q].max() + 1e-12
    # bf16 operands: inside the bar at every depth, and the last quarter is no worse than the first
    assert max(e_bf) < 1e-2
    assert pe[-q:].max() <= 2 * pe[:q].max()
