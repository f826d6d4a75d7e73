"""Python binding of libttt.so with the C ABI's names.

Argument marshalling only: checks device / dtype / shape / contiguity of
torch tensors, then passes raw device pointers and the current HIP stream.
Every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import TTT_BF16, TTT_F32, TTTError  # noqa: F401

_IO = {torch.float32: TTT_F32, torch.bfloat16: TTT_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() or None


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def ttt_linear_forward(XQ, XK, XV, eta, W0, b0, ln_gamma, ln_beta, O=None, W_out=None,
                       b_out=None, mb: int = 16, ln_eps: float = 1e-6, stream=None):
    """TTT-Linear prefill. XQ/XK/XV/O [B,H,L,d] (fp32 or bf16); eta [B,H,L];
    W0 [H,d,d] (shared over B) or [B,H,d,d]; b0 [H,d] or [B,H,d]; gamma/beta [H,d].
    Returns (O, W_out, b_out); outputs are allocated when not given."""
    B, H, L, d = XQ.shape
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    batched = W0.dim() == 4
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(eta, "eta", (B, H, L), torch.float32)
    _need(W0, "W0", ((B,) if batched else ()) + (H, d, d), torch.float32)
    _need(b0, "b0", ((B,) if batched else ()) + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if O is None:
        O = torch.empty_like(XQ)
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=XQ.device, dtype=torch.float32)
    if b_out is None:
        b_out = torch.empty((B, H, d), device=XQ.device, dtype=torch.float32)
    _need(O, "O", (B, H, L, d), XQ.dtype)
    _need(W_out, "W_out", (B, H, d, d), torch.float32)
    _need(b_out, "b_out", (B, H, d), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_linear_forward(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV),
                                      _ptr(eta), _ptr(W0), _ptr(b0), int(batched),
                                      _ptr(ln_gamma), _ptr(ln_beta), _ptr(O), _ptr(W_out),
                                      _ptr(b_out), _stream(stream)))
    return O, W_out, b_out


def ttt_linear_forward_gated(XQ, XK, XV, theta_lr, eta_base: float, W0, b0, ln_gamma, ln_beta,
                             O=None, W_out=None, b_out=None, mb: int = 16, ln_eps: float = 1e-6,
                             stream=None):
    """TTT-Linear prefill with eta_t = eta_base * logistic(theta_lr[h] . XK_t)
    evaluated in the kernel. theta_lr [H,d] fp32; the rest as ttt_linear_forward."""
    B, H, L, d = XQ.shape
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    batched = W0.dim() == 4
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(theta_lr, "theta_lr", (H, d), torch.float32)
    _need(W0, "W0", ((B,) if batched else ()) + (H, d, d), torch.float32)
    _need(b0, "b0", ((B,) if batched else ()) + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    O = torch.empty_like(XQ) if O is None else O
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=XQ.device, dtype=torch.float32)
    if b_out is None:
        b_out = torch.empty((B, H, d), device=XQ.device, dtype=torch.float32)
    _need(O, "O", (B, H, L, d), XQ.dtype)
    _need(W_out, "W_out", (B, H, d, d), torch.float32)
    _need(b_out, "b_out", (B, H, d), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_linear_forward_gated(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK),
                                            _ptr(XV), _ptr(theta_lr), float(eta_base), _ptr(W0),
                                            _ptr(b0), int(batched), _ptr(ln_gamma),
                                            _ptr(ln_beta), _ptr(O), _ptr(W_out), _ptr(b_out),
                                            _stream(stream)))
    return O, W_out, b_out


def ttt_linear_forward_opts(XQ, XK, XV, eta, W0, b0, ln_gamma, ln_beta, inner_loss: str = "mse",
                            weight_decay: float = 0.0, O=None, W_out=None, b_out=None,
                            mb: int = 16, ln_eps: float = 1e-6, stream=None):
    """TTT-Linear prefill with the inner loss ("mse" or "inner_product") and
    weight decay on W as options; the rest as ttt_linear_forward."""
    B, H, L, d = XQ.shape
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    loss = {"mse": _lib.TTT_LOSS_MSE, "inner_product": _lib.TTT_LOSS_INNER_PRODUCT}.get(inner_loss)
    if loss is None:
        raise ValueError(f"inner_loss {inner_loss!r} is not 'mse' or 'inner_product'")
    batched = W0.dim() == 4
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(eta, "eta", (B, H, L), torch.float32)
    _need(W0, "W0", ((B,) if batched else ()) + (H, d, d), torch.float32)
    _need(b0, "b0", ((B,) if batched else ()) + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    O = torch.empty_like(XQ) if O is None else O
    if W_out is None:
        W_out = torch.empty((B, H, d, d), device=XQ.device, dtype=torch.float32)
    if b_out is None:
        b_out = torch.empty((B, H, d), device=XQ.device, dtype=torch.float32)
    _need(O, "O", (B, H, L, d), XQ.dtype)
    _need(W_out, "W_out", (B, H, d, d), torch.float32)
    _need(b_out, "b_out", (B, H, d), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_linear_forward_opts(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV),
                                           _ptr(eta), _ptr(W0), _ptr(b0), int(batched),
                                           _ptr(ln_gamma), _ptr(ln_beta), loss,
                                           float(weight_decay), _ptr(O), _ptr(W_out),
                                           _ptr(b_out), _stream(stream)))
    return O, W_out, b_out


def ttt_eta_gate(XK, theta_lr, eta_base: float, eta=None, stream=None):
    """eta [B,H,L] = eta_base * logistic(theta_lr[h] . XK[n,h,t])."""
    B, H, L, d = XK.shape
    io = _IO.get(XK.dtype)
    if io is None:
        raise TypeError(f"XK dtype {XK.dtype} not supported")
    _need(theta_lr, "theta_lr", (H, d), torch.float32)
    eta = torch.empty((B, H, L), device=XK.device, dtype=torch.float32) if eta is None else eta
    _need(eta, "eta", (B, H, L), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_eta_gate(B, H, L, d, io, _ptr(XK), _ptr(theta_lr), float(eta_base),
                                _ptr(eta), _stream(stream)))
    return eta


def ttt_qkv_project(X, theta, H: int, out=None, stream=None):
    """XQ, XK, XV [B,H,L,64] bf16 from X [B,L,d_model] bf16 and theta
    [3,H*64,d_model] bf16 (output-major): XQ[b,h,t,j] = sum_k X[b,t,k]
    theta[0][h*64+j][k], likewise XK (theta[1]) and XV (theta[2])."""
    B, L, dm = X.shape
    d = 64
    _need(X, "X", (B, L, dm), torch.bfloat16)
    _need(theta, "theta", (3, H * d, dm), torch.bfloat16)
    if out is None:
        out = tuple(torch.empty((B, H, L, d), device=X.device, dtype=torch.bfloat16) for _ in range(3))
    for o, n in zip(out, ("XQ", "XK", "XV")):
        _need(o, n, (B, H, L, d), torch.bfloat16)
    lib = _lib.load()
    _lib.check(lib.ttt_qkv_project(B, L, dm, H, d, _ptr(X), _ptr(theta), _ptr(out[0]), _ptr(out[1]),
                                   _ptr(out[2]), _stream(stream)))
    return out


def ttt_eta_gate_backward(XK, theta_lr, eta_base: float, deta, dXK, dtheta=None, stream=None):
    """Adds the gate's share to dXK [B,H,L,d] fp32 in place; returns dtheta
    [B,H,d] per sequence (sum over B for the parameter's gradient)."""
    B, H, L, d = XK.shape
    io = _IO.get(XK.dtype)
    if io is None:
        raise TypeError(f"XK dtype {XK.dtype} not supported")
    _need(theta_lr, "theta_lr", (H, d), torch.float32)
    _need(deta, "deta", (B, H, L), torch.float32)
    _need(dXK, "dXK", (B, H, L, d), torch.float32)
    dtheta = torch.empty((B, H, d), device=XK.device, dtype=torch.float32) if dtheta is None else dtheta
    _need(dtheta, "dtheta", (B, H, d), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_eta_gate_backward(B, H, L, d, io, _ptr(XK), _ptr(theta_lr), float(eta_base),
                                         _ptr(deta), _ptr(dXK), _ptr(dtheta), _stream(stream)))
    return dtheta


def ttt_linear_backward_workspace(B: int, H: int, L: int, d: int, mb: int = 16) -> int:
    """Bytes of device workspace ttt_linear_backward needs."""
    n = ctypes.c_size_t(0)
    lib = _lib.load()
    _lib.check(lib.ttt_linear_backward_workspace(B, H, L, d, mb, ctypes.byref(n)))
    return n.value


def ttt_linear_backward(XQ, XK, XV, eta, W0, b0, ln_gamma, ln_beta, dO, dW_out=None, db_out=None,
                        mb: int = 16, ln_eps: float = 1e-6, workspace=None, stream=None) -> dict:
    """Gradients of <dO,O> + <dW_out,W_L> + <db_out,b_L> through ttt_linear_forward.
    Inputs as ttt_linear_forward plus dO [B,H,L,d] fp32 and optional dW_out
    [B,H,d,d], db_out [B,H,d]. Returns per-sequence fp32 gradients dXQ, dXK,
    dXV [B,H,L,d], deta [B,H,L], dW0 [B,H,d,d], db0, dgamma, dbeta [B,H,d]."""
    B, H, L, d = XQ.shape
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    batched = W0.dim() == 4
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(eta, "eta", (B, H, L), torch.float32)
    _need(W0, "W0", ((B,) if batched else ()) + (H, d, d), torch.float32)
    _need(b0, "b0", ((B,) if batched else ()) + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    _need(dO, "dO", (B, H, L, d), torch.float32)
    if dW_out is not None:
        _need(dW_out, "dW_out", (B, H, d, d), torch.float32)
    if db_out is not None:
        _need(db_out, "db_out", (B, H, d), torch.float32)
    kw = dict(device=XQ.device, dtype=torch.float32)
    g = {"dXQ": torch.empty((B, H, L, d), **kw), "dXK": torch.empty((B, H, L, d), **kw),
         "dXV": torch.empty((B, H, L, d), **kw), "deta": torch.empty((B, H, L), **kw),
         "dW0": torch.empty((B, H, d, d), **kw), "db0": torch.empty((B, H, d), **kw),
         "dgamma": torch.empty((B, H, d), **kw), "dbeta": torch.empty((B, H, d), **kw)}
    need = ttt_linear_backward_workspace(B, H, L, d, mb)
    if workspace is None:
        workspace = torch.empty(max(need, 4), device=XQ.device, dtype=torch.uint8)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.ttt_linear_backward(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV),
                                       _ptr(eta), _ptr(W0), _ptr(b0), int(batched),
                                       _ptr(ln_gamma), _ptr(ln_beta), _ptr(dO), _ptr(dW_out),
                                       _ptr(db_out), _ptr(g["dXQ"]), _ptr(g["dXK"]),
                                       _ptr(g["dXV"]), _ptr(g["deta"]), _ptr(g["dW0"]),
                                       _ptr(g["db0"]), _ptr(g["dgamma"]), _ptr(g["dbeta"]),
                                       _ptr(workspace), nbytes, _stream(stream)))
    return g


def ttt_mlp_backward_workspace(B: int, H: int, L: int, d: int, mb: int = 16) -> int:
    """Bytes of device workspace ttt_mlp_backward needs."""
    n = ctypes.c_size_t(0)
    lib = _lib.load()
    _lib.check(lib.ttt_mlp_backward_workspace(B, H, L, d, mb, ctypes.byref(n)))
    return n.value


def ttt_mlp_backward(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta, dO, dW1_out=None,
                     db1_out=None, dW2_out=None, db2_out=None, mb: int = 16, ln_eps: float = 1e-6,
                     workspace=None, stream=None) -> dict:
    """Gradients of <dO,O> + <dW1_out,W1_L> + <db1_out,b1_L> + <dW2_out,W2_L> +
    <db2_out,b2_L> through ttt_mlp_forward. Inputs as ttt_mlp_forward plus dO
    [B,H,L,d] fp32 and the optional state adjoints. Returns per-sequence fp32
    gradients dXQ, dXK, dXV [B,H,L,d], deta [B,H,L], dW1 [B,H,d,4d], db1
    [B,H,4d], dW2 [B,H,4d,d], db2, dgamma, dbeta [B,H,d]."""
    B, H, L, d = XQ.shape
    m = 4 * d
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    batched = W1.dim() == 4
    pre = (B,) if batched else ()
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(eta, "eta", (B, H, L), torch.float32)
    _need(W1, "W1", pre + (H, d, m), torch.float32)
    _need(b1, "b1", pre + (H, m), torch.float32)
    _need(W2, "W2", pre + (H, m, d), torch.float32)
    _need(b2, "b2", pre + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    _need(dO, "dO", (B, H, L, d), torch.float32)
    for t, n, shp in ((dW1_out, "dW1_out", (B, H, d, m)), (db1_out, "db1_out", (B, H, m)),
                      (dW2_out, "dW2_out", (B, H, m, d)), (db2_out, "db2_out", (B, H, d))):
        if t is not None:
            _need(t, n, shp, torch.float32)
    kw = dict(device=XQ.device, dtype=torch.float32)
    g = {"dXQ": torch.empty((B, H, L, d), **kw), "dXK": torch.empty((B, H, L, d), **kw),
         "dXV": torch.empty((B, H, L, d), **kw), "deta": torch.empty((B, H, L), **kw),
         "dW1": torch.empty((B, H, d, m), **kw), "db1": torch.empty((B, H, m), **kw),
         "dW2": torch.empty((B, H, m, d), **kw), "db2": torch.empty((B, H, d), **kw),
         "dgamma": torch.empty((B, H, d), **kw), "dbeta": torch.empty((B, H, d), **kw)}
    need = ttt_mlp_backward_workspace(B, H, L, d, mb)
    if workspace is None:
        workspace = torch.empty(max(need, 4), device=XQ.device, dtype=torch.uint8)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.ttt_mlp_backward(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV),
                                    _ptr(eta), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), int(batched),
                                    _ptr(ln_gamma), _ptr(ln_beta), _ptr(dO), _ptr(dW1_out),
                                    _ptr(db1_out), _ptr(dW2_out), _ptr(db2_out), _ptr(g["dXQ"]),
                                    _ptr(g["dXK"]), _ptr(g["dXV"]), _ptr(g["deta"]), _ptr(g["dW1"]),
                                    _ptr(g["db1"]), _ptr(g["dW2"]), _ptr(g["db2"]),
                                    _ptr(g["dgamma"]), _ptr(g["dbeta"]), _ptr(workspace), nbytes,
                                    _stream(stream)))
    return g


def ttt_linear_backward_noalloc(XQ, XK, XV, eta, W0, b0, ln_gamma, ln_beta, dO, dW_out=None,
                                db_out=None, mb: int = 16, ln_eps: float = 1e-6,
                                grads=None, stream=None) -> dict:
    """ttt_linear_backward without a workspace: the checkpoints go to the
    library's fixed device scratch (TTT_BACKWARD_SCRATCH_BYTES per GPU), and
    the library allocates nothing. `grads` may hold preallocated outputs
    (a dict like the one returned), so the call itself allocates nothing on
    the Python side either; calls that overlap on one GPU race."""
    B, H, L, d = XQ.shape
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    batched = W0.dim() == 4
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    _need(eta, "eta", (B, H, L), torch.float32)
    _need(W0, "W0", ((B,) if batched else ()) + (H, d, d), torch.float32)
    _need(b0, "b0", ((B,) if batched else ()) + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    _need(dO, "dO", (B, H, L, d), torch.float32)
    if dW_out is not None:
        _need(dW_out, "dW_out", (B, H, d, d), torch.float32)
    if db_out is not None:
        _need(db_out, "db_out", (B, H, d), torch.float32)
    shapes = {"dXQ": (B, H, L, d), "dXK": (B, H, L, d), "dXV": (B, H, L, d), "deta": (B, H, L),
              "dW0": (B, H, d, d), "db0": (B, H, d), "dgamma": (B, H, d), "dbeta": (B, H, d)}
    if grads is None:
        grads = {k: torch.empty(v, device=XQ.device, dtype=torch.float32) for k, v in shapes.items()}
    for k, v in shapes.items():
        _need(grads[k], k, v, torch.float32)
    g = grads
    lib = _lib.load()
    _lib.check(lib.ttt_linear_backward_noalloc(
        B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV), _ptr(eta), _ptr(W0), _ptr(b0),
        int(batched), _ptr(ln_gamma), _ptr(ln_beta), _ptr(dO), _ptr(dW_out), _ptr(db_out),
        _ptr(g["dXQ"]), _ptr(g["dXK"]), _ptr(g["dXV"]), _ptr(g["deta"]), _ptr(g["dW0"]),
        _ptr(g["db0"]), _ptr(g["dgamma"]), _ptr(g["dbeta"]), _stream(stream)))
    return g


def ttt_mlp_forward(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta, O=None, outs=None,
                    mb: int = 16, ln_eps: float = 1e-6, stream=None):
    """TTT-MLP prefill (d = 64, hidden 4d). W1 [.,H,d,4d], b1 [.,H,4d],
    W2 [.,H,4d,d], b2 [.,H,d] with "." = B when per batch. Returns
    (O, W1_out, b1_out, W2_out, b2_out)."""
    return _mlp(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta, O, outs, mb, ln_eps, stream,
                None, 0.0)


def ttt_mlp_forward_gated(XQ, XK, XV, theta_lr, eta_base: float, W1, b1, W2, b2, ln_gamma,
                          ln_beta, O=None, outs=None, mb: int = 16, ln_eps: float = 1e-6,
                          stream=None):
    """TTT-MLP prefill with eta_t = eta_base * logistic(theta_lr[h] . XK_t)
    formed inside the kernel (theta_lr [H,d] fp32); the rest as ttt_mlp_forward."""
    return _mlp(XQ, XK, XV, None, W1, b1, W2, b2, ln_gamma, ln_beta, O, outs, mb, ln_eps, stream,
                None, 0.0, gate=(theta_lr, eta_base))


def ttt_mlp_forward_opts(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta,
                         inner_loss: str = "mse", weight_decay: float = 0.0, O=None, outs=None,
                         mb: int = 16, ln_eps: float = 1e-6, stream=None):
    """TTT-MLP prefill with the inner loss ("mse" or "inner_product") and
    weight decay on W1, W2 as options; the rest as ttt_mlp_forward."""
    return _mlp(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta, O, outs, mb, ln_eps, stream,
                inner_loss, weight_decay)


def _mlp(XQ, XK, XV, eta, W1, b1, W2, b2, ln_gamma, ln_beta, O, outs, mb, ln_eps, stream,
         inner_loss, weight_decay, gate=None):
    B, H, L, d = XQ.shape
    m = 4 * d
    io = _IO.get(XQ.dtype)
    if io is None:
        raise TypeError(f"XQ dtype {XQ.dtype} not supported")
    loss = None
    if inner_loss is not None:
        loss = {"mse": _lib.TTT_LOSS_MSE,
                "inner_product": _lib.TTT_LOSS_INNER_PRODUCT}.get(inner_loss)
        if loss is None:
            raise ValueError(f"inner_loss {inner_loss!r} is not 'mse' or 'inner_product'")
    batched = W1.dim() == 4
    pre = (B,) if batched else ()
    for t, n in ((XQ, "XQ"), (XK, "XK"), (XV, "XV")):
        _need(t, n, (B, H, L, d), XQ.dtype)
    if gate is None:
        _need(eta, "eta", (B, H, L), torch.float32)
    else:
        _need(gate[0], "theta_lr", (H, d), torch.float32)
    _need(W1, "W1", pre + (H, d, m), torch.float32)
    _need(b1, "b1", pre + (H, m), torch.float32)
    _need(W2, "W2", pre + (H, m, d), torch.float32)
    _need(b2, "b2", pre + (H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if O is None:
        O = torch.empty_like(XQ)
    if outs is None:
        kw = dict(device=XQ.device, dtype=torch.float32)
        outs = (torch.empty((B, H, d, m), **kw), torch.empty((B, H, m), **kw),
                torch.empty((B, H, m, d), **kw), torch.empty((B, H, d), **kw))
    _need(O, "O", (B, H, L, d), XQ.dtype)
    for t, n, s in zip(outs, ("W1_out", "b1_out", "W2_out", "b2_out"),
                       ((B, H, d, m), (B, H, m), (B, H, m, d), (B, H, d))):
        _need(t, n, s, torch.float32)
    lib = _lib.load()
    tail = (_ptr(O),) + tuple(_ptr(t) for t in outs) + (_stream(stream),)
    if gate is not None:
        _lib.check(lib.ttt_mlp_forward_gated(B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK),
                                             _ptr(XV), _ptr(gate[0]), float(gate[1]), _ptr(W1),
                                             _ptr(b1), _ptr(W2), _ptr(b2), int(batched),
                                             _ptr(ln_gamma), _ptr(ln_beta), *tail))
        return (O,) + tuple(outs)
    head = (B, H, L, d, mb, io, ln_eps, _ptr(XQ), _ptr(XK), _ptr(XV), _ptr(eta), _ptr(W1),
            _ptr(b1), _ptr(W2), _ptr(b2), int(batched), _ptr(ln_gamma), _ptr(ln_beta))
    if loss is None:
        _lib.check(lib.ttt_mlp_forward(*head, *tail))
    else:
        _lib.check(lib.ttt_mlp_forward_opts(*head, loss, float(weight_decay), *tail))
    return (O,) + tuple(outs)


def ttt_decode_step(xq, xk, xv, eta, W, b, ln_gamma, ln_beta, o=None, ln_eps: float = 1e-6,
                    stream=None):
    """One b = 1 step on B x H states, updating W [B,H,d,d] and b [B,H,d] in
    place. xq/xk/xv/o [B,H,d]; eta [B,H]. Returns o."""
    B, H, d = xq.shape
    io = _IO.get(xq.dtype)
    if io is None:
        raise TypeError(f"xq dtype {xq.dtype} not supported")
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n, (B, H, d), xq.dtype)
    _need(eta, "eta", (B, H), torch.float32)
    _need(W, "W", (B, H, d, d), torch.float32)
    _need(b, "b", (B, H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if o is None:
        o = torch.empty_like(xq)
    _need(o, "o", (B, H, d), xq.dtype)
    lib = _lib.load()
    _lib.check(lib.ttt_decode_step(B, H, d, io, ln_eps, _ptr(xq), _ptr(xk), _ptr(xv),
                                   _ptr(eta), _ptr(W), _ptr(b), _ptr(ln_gamma), _ptr(ln_beta),
                                   _ptr(o), _stream(stream)))
    return o


def ttt_decode_steps(xq, xk, xv, eta, W, b, ln_gamma, ln_beta, o=None, ln_eps: float = 1e-6,
                     stream=None):
    """T consecutive b = 1 steps on B x H states, updating W [B,H,d,d] and
    b [B,H,d] in place. xq/xk/xv/o [T,B,H,d] step-major; eta [T,B,H].
    Returns o."""
    T, B, H, d = xq.shape
    io = _IO.get(xq.dtype)
    if io is None:
        raise TypeError(f"xq dtype {xq.dtype} not supported")
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n, (T, B, H, d), xq.dtype)
    _need(eta, "eta", (T, B, H), torch.float32)
    _need(W, "W", (B, H, d, d), torch.float32)
    _need(b, "b", (B, H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if o is None:
        o = torch.empty_like(xq)
    _need(o, "o", (T, B, H, d), xq.dtype)
    lib = _lib.load()
    _lib.check(lib.ttt_decode_steps(T, B, H, d, io, ln_eps, _ptr(xq), _ptr(xk), _ptr(xv),
                                    _ptr(eta), _ptr(W), _ptr(b), _ptr(ln_gamma), _ptr(ln_beta),
                                    _ptr(o), _stream(stream)))
    return o


def ttt_decode_steps_mb(xq, xk, xv, eta, W_chunk, b_chunk, W, b, ln_gamma, ln_beta, mb: int,
                        pos: int = 0, o=None, ln_eps: float = 1e-6, stream=None):
    """T consecutive tokens under the mini-batch rule with b = mb: every token
    of a chunk takes its gradient at the chunk-start state (W_chunk, b_chunk),
    and the current state (W, b) is updated token by token; pos is the first
    step's position within its chunk. All four state tensors are updated in
    place. Shapes as ttt_decode_steps. Returns o."""
    T, B, H, d = xq.shape
    io = _IO.get(xq.dtype)
    if io is None:
        raise TypeError(f"xq dtype {xq.dtype} not supported")
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n, (T, B, H, d), xq.dtype)
    _need(eta, "eta", (T, B, H), torch.float32)
    for t, n in ((W_chunk, "W_chunk"), (W, "W")):
        _need(t, n, (B, H, d, d), torch.float32)
    for t, n in ((b_chunk, "b_chunk"), (b, "b")):
        _need(t, n, (B, H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if o is None:
        o = torch.empty_like(xq)
    _need(o, "o", (T, B, H, d), xq.dtype)
    lib = _lib.load()
    _lib.check(lib.ttt_decode_steps_mb(T, B, H, d, io, ln_eps, mb, pos, _ptr(xq), _ptr(xk),
                                       _ptr(xv), _ptr(eta), _ptr(W_chunk), _ptr(b_chunk), _ptr(W),
                                       _ptr(b), _ptr(ln_gamma), _ptr(ln_beta), _ptr(o),
                                       _stream(stream)))
    return o


def ttt_decode_steps_gated(xq, xk, xv, theta_lr, eta_base: float, W, b, ln_gamma, ln_beta,
                           mb: int = 1, pos: int = 0, W_chunk=None, b_chunk=None, o=None,
                           ln_eps: float = 1e-6, stream=None):
    """T consecutive decode tokens with eta_t = eta_base * logistic(theta_lr[h]
    . xk_t) formed in the kernel (theta_lr [H,d] fp32). mb = 1 is b = 1 decode;
    mb > 1 follows the mini-batch rule of ttt_decode_steps_mb and needs
    W_chunk, b_chunk. States are updated in place. Returns o."""
    T, B, H, d = xq.shape
    io = _IO.get(xq.dtype)
    if io is None:
        raise TypeError(f"xq dtype {xq.dtype} not supported")
    for t, n in ((xq, "xq"), (xk, "xk"), (xv, "xv")):
        _need(t, n, (T, B, H, d), xq.dtype)
    _need(theta_lr, "theta_lr", (H, d), torch.float32)
    _need(W, "W", (B, H, d, d), torch.float32)
    _need(b, "b", (B, H, d), torch.float32)
    if mb > 1:
        _need(W_chunk, "W_chunk", (B, H, d, d), torch.float32)
        _need(b_chunk, "b_chunk", (B, H, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (H, d), torch.float32)
    _need(ln_beta, "ln_beta", (H, d), torch.float32)
    if o is None:
        o = torch.empty_like(xq)
    _need(o, "o", (T, B, H, d), xq.dtype)
    lib = _lib.load()
    _lib.check(lib.ttt_decode_steps_gated(T, B, H, d, io, ln_eps, mb, pos, _ptr(xq), _ptr(xk),
                                          _ptr(xv), _ptr(theta_lr), float(eta_base),
                                          _ptr(W_chunk), _ptr(b_chunk), _ptr(W), _ptr(b),
                                          _ptr(ln_gamma), _ptr(ln_beta), _ptr(o),
                                          _stream(stream)))
    return o


def ttt_ln_l2_bwd(Z, target, ln_gamma, ln_beta, G=None, ln_eps: float = 1e-6, stream=None):
    """Row-wise fused LN + L2 backward. Z, target, G [rows,d] fp32; gamma/beta [d]."""
    rows, d = Z.shape
    _need(Z, "Z", (rows, d), torch.float32)
    _need(target, "target", (rows, d), torch.float32)
    _need(ln_gamma, "ln_gamma", (d,), torch.float32)
    _need(ln_beta, "ln_beta", (d,), torch.float32)
    if G is None:
        G = torch.empty_like(Z)
    _need(G, "G", (rows, d), torch.float32)
    lib = _lib.load()
    _lib.check(lib.ttt_ln_l2_bwd(rows, d, _ptr(Z), _ptr(target), _ptr(ln_gamma), _ptr(ln_beta),
                                 ln_eps, _ptr(G), _stream(stream)))
    return G


def ttt_version() -> int:
    return _lib.load().ttt_version()


def ttt_last_error() -> str:
    return _lib.load().ttt_last_error().decode()
