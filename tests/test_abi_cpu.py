"""libttt.so loads, exports every function include/ttt.h declares, and its host
validation rejects bad arguments before any HIP call (no GPU needed: the
pointers below are never dereferenced)."""
import ctypes

import pytest

from test_sequence_layer_ttt_amd import _lib

FAKE = 0x10000          # 16-byte aligned, never dereferenced by the host checks
FAKE2 = 0x20000000


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _lib.header_functions()
    assert set(names) >= {"ttt_linear_forward", "ttt_mlp_forward", "ttt_decode_step",
                          "ttt_decode_steps", "ttt_linear_backward",
                          "ttt_linear_backward_workspace", "ttt_ln_l2_bwd", "ttt_last_error",
                          "ttt_version", "ttt_linear_forward_gated", "ttt_eta_gate",
                          "ttt_eta_gate_backward", "ttt_linear_backward_noalloc", "ttt_qkv_project"}
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version(lib):
    assert lib.ttt_version() == 1


def _lin(lib, B=1, H=1, L=16, d=64, mb=16, io=1, ptrs=None, batched=0, W_out=None, b_out=None,
         O=None, eps=1e-6):
    # distinct non-overlapping fake buffers, 1 MiB apart
    p = ptrs or [FAKE + i * (1 << 20) for i in range(8)]
    Wo = W_out if W_out is not None else FAKE + 9 * (1 << 20)
    bo = b_out if b_out is not None else FAKE + 10 * (1 << 20)
    Oo = O if O is not None else FAKE + 11 * (1 << 20)
    return lib.ttt_linear_forward(B, H, L, d, mb, io, eps, p[0], p[1], p[2], p[3], p[4], p[5],
                                  batched, p[6], p[7], Oo, Wo, bo, None)


def test_linear_rejects_negative_sizes(lib):
    assert _lin(lib, B=-1) == _lib.TTT_E_SHAPE
    assert _lin(lib, L=-3) == _lib.TTT_E_SHAPE
    assert "negative" in lib.ttt_last_error().decode()


def test_linear_rejects_unsupported_d_and_mb(lib):
    assert _lin(lib, d=48) == _lib.TTT_E_SHAPE
    assert _lin(lib, mb=0) == _lib.TTT_E_SHAPE
    assert _lin(lib, mb=17) == _lib.TTT_E_SHAPE


def test_prefill_rejects_sequences_longer_than_max_l(lib):
    """Token and chunk indices in the kernels are 32-bit ints: L is bounded
    by TTT_MAX_L = 2^30 on every prefill entry point."""
    big = (1 << 30) + 1
    assert _lin(lib, L=big) == _lib.TTT_E_SHAPE
    assert "TTT_MAX_L" in lib.ttt_last_error().decode()
    p = [FAKE + i * (1 << 20) for i in range(16)]
    assert lib.ttt_mlp_forward(1, 1, big, 64, 16, 1, 1e-6, *p[:8], 0, p[8], p[9], p[10],
                               p[11], p[12], p[13], p[14], None) == _lib.TTT_E_SHAPE
    assert _lin(lib, L=1 << 30) != _lib.TTT_E_SHAPE or "TTT_MAX_L" not in lib.ttt_last_error().decode()


@pytest.mark.parametrize("eps", [0.0, -1e-6, 1e-40, float("inf"), float("nan")])
def test_every_entry_point_rejects_bad_eps(lib, eps):
    """The layer norms need var + eps to be a positive normal float."""
    assert _lin(lib, eps=eps) == _lib.TTT_E_SHAPE
    assert "ln_eps" in lib.ttt_last_error().decode()
    p = [FAKE + i * (1 << 20) for i in range(16)]
    assert lib.ttt_mlp_forward(1, 1, 16, 64, 16, 1, eps, *p[:8], 0, p[8], p[9], p[10], p[11],
                               p[12], p[13], p[14], None) == _lib.TTT_E_SHAPE
    assert lib.ttt_decode_step(1, 1, 64, 1, eps, *p[:9], None) == _lib.TTT_E_SHAPE
    assert lib.ttt_decode_steps(4, 1, 1, 64, 1, eps, *p[:9], None) == _lib.TTT_E_SHAPE
    assert lib.ttt_ln_l2_bwd(4, 64, FAKE, FAKE2, FAKE + 4096, FAKE + 8192, eps,
                             FAKE2 + (1 << 20), None) == _lib.TTT_E_SHAPE


def test_linear_rejects_bad_dtype(lib):
    assert _lin(lib, io=7) == _lib.TTT_E_DTYPE


def test_linear_rejects_null(lib):
    p = [FAKE + i * (1 << 20) for i in range(8)]
    p[2] = 0
    assert _lin(lib, ptrs=p) == _lib.TTT_E_NULL
    assert "XV" in lib.ttt_last_error().decode()


def test_linear_rejects_misaligned(lib):
    p = [FAKE + i * (1 << 20) for i in range(8)]
    p[0] += 4
    assert _lin(lib, ptrs=p) == _lib.TTT_E_ALIGN


def test_linear_rejects_aliasing(lib):
    p = [FAKE + i * (1 << 20) for i in range(8)]
    assert _lin(lib, ptrs=p, O=p[1] + 64) == _lib.TTT_E_ALIAS
    # W_out == W0 is only allowed with per-batch state
    assert _lin(lib, ptrs=p, W_out=p[4]) == _lib.TTT_E_ALIAS
    # partial overlap of W_out with W0 is never allowed
    assert _lin(lib, ptrs=p, batched=1, W_out=p[4] + 16) == _lib.TTT_E_ALIAS
    # W_out overlapping b_out
    assert _lin(lib, ptrs=p, W_out=FAKE2, b_out=FAKE2 + 256) == _lib.TTT_E_ALIAS


def test_linear_empty_batch_is_a_noop(lib):
    # B*H == 0: every buffer is empty, NULL pointers are fine, nothing launched
    # (per-head parameters W0, b0, gamma, beta are still [H, ...] and non-empty)
    assert lib.ttt_linear_forward(0, 4, 16, 64, 16, 1, 1e-6, None, None, None, None, FAKE,
                                  FAKE2, 0, FAKE2 + 4096, FAKE2 + 8192, None, None, None,
                                  None) == _lib.TTT_OK


def test_mlp_validation(lib):
    p = [FAKE + i * (1 << 20) for i in range(16)]

    def call(d=64, mb=16, outs=(p[11], p[12], p[13], p[14]), io=1):
        return lib.ttt_mlp_forward(1, 1, 16, d, mb, io, 1e-6, p[0], p[1], p[2], p[3], p[4], p[5],
                                   p[6], p[7], 0, p[8], p[9], p[10], *outs, None)

    assert call(d=16) == _lib.TTT_E_SHAPE
    assert call(mb=0) == _lib.TTT_E_SHAPE
    assert call(io=2) == _lib.TTT_E_DTYPE
    assert call(outs=(p[11], None, p[13], p[14])) == _lib.TTT_E_NULL
    assert call(outs=(p[4], p[12], p[13], p[14])) == _lib.TTT_E_ALIAS


def test_decode_validation(lib):
    p = [FAKE + i * (1 << 20) for i in range(10)]
    assert lib.ttt_decode_step(1, 1, 32, 1, 1e-6, *p[:9], None) == _lib.TTT_E_SHAPE
    assert lib.ttt_decode_step(1, 1, 64, 1, 1e-6, p[0], p[1], p[2], p[3], p[0], p[5], p[6],
                               p[7], p[8], None) == _lib.TTT_E_ALIAS
    assert lib.ttt_decode_step(1, 1, 64, 1, 1e-6, p[0], 0, p[2], p[3], p[4], p[5], p[6], p[7],
                               p[8], None) == _lib.TTT_E_NULL


def test_decode_steps_validation(lib):
    p = [FAKE + i * (1 << 20) for i in range(10)]
    assert lib.ttt_decode_steps(-1, 1, 1, 64, 1, 1e-6, *p[:9], None) == _lib.TTT_E_SHAPE
    assert "T = -1" in lib.ttt_last_error().decode()
    assert lib.ttt_decode_steps(3, 1, 1, 32, 1, 1e-6, *p[:9], None) == _lib.TTT_E_SHAPE
    assert lib.ttt_decode_steps(3, 1, 1, 64, 5, 1e-6, *p[:9], None) == _lib.TTT_E_DTYPE
    # W overlapping xq
    assert lib.ttt_decode_steps(3, 1, 1, 64, 1, 1e-6, p[0], p[1], p[2], p[3], p[0], p[5], p[6],
                                p[7], p[8], None) == _lib.TTT_E_ALIAS
    assert lib.ttt_decode_steps(3, 1, 1, 64, 1, 1e-6, p[0], 0, p[2], p[3], p[4], p[5], p[6], p[7],
                                p[8], None) == _lib.TTT_E_NULL
    # misaligned xk (bf16 needs 2-byte alignment)
    assert lib.ttt_decode_steps(3, 1, 1, 64, 1, 1e-6, p[0], p[1] + 1, p[2], p[3], p[4], p[5], p[6],
                                p[7], p[8], None) == _lib.TTT_E_ALIGN
    # no steps, or no states: nothing to do, no HIP call
    assert lib.ttt_decode_steps(0, 2, 3, 64, 1, 1e-6, *p[:9], None) == _lib.TTT_OK
    assert lib.ttt_decode_steps(5, 0, 3, 64, 1, 1e-6, *p[:9], None) == _lib.TTT_OK


def _bwd(lib, B=2, H=3, L=40, d=64, mb=16, io=1, eps=1e-6, ws_bytes=None, ptrs=None, ws=None):
    p = ptrs or [FAKE + i * (1 << 24) for i in range(20)]
    need = ctypes.c_size_t(0)
    lib.ttt_linear_backward_workspace(max(B, 0), max(H, 0), max(L, 0), 64, 16, ctypes.byref(need))
    nb = need.value if ws_bytes is None else ws_bytes
    return lib.ttt_linear_backward(B, H, L, d, mb, io, eps, p[0], p[1], p[2], p[3], p[4], p[5], 0,
                                   p[6], p[7], p[8], None, None, p[9], p[10], p[11], p[12], p[13],
                                   p[14], p[15], p[16], ws if ws is not None else p[17], nb, None)


def _dmb(lib, T=3, mb=4, pos=0, d=64, Wc=FAKE + 6 * (1 << 20), bc=FAKE + 7 * (1 << 20),
         W=FAKE + 8 * (1 << 20)):
    p = [FAKE + i * (1 << 20) for i in range(6)]
    return lib.ttt_decode_steps_mb(T, 2, 3, d, 1, 1e-6, mb, pos, p[0], p[1], p[2], p[3], Wc, bc, W,
                                   FAKE + 9 * (1 << 20), p[4], p[5], FAKE + 10 * (1 << 20), None)


def test_decode_steps_mb_validation(lib):
    assert _dmb(lib, mb=0) == _lib.TTT_E_SHAPE
    assert _dmb(lib, mb=17) == _lib.TTT_E_SHAPE
    assert _dmb(lib, pos=4) == _lib.TTT_E_SHAPE and "pos" in lib.ttt_last_error().decode()
    assert _dmb(lib, pos=-1) == _lib.TTT_E_SHAPE
    assert _dmb(lib, T=-1) == _lib.TTT_E_SHAPE
    assert _dmb(lib, d=32) == _lib.TTT_E_SHAPE
    assert _dmb(lib, Wc=0) == _lib.TTT_E_NULL and "W_chunk" in lib.ttt_last_error().decode()
    assert _dmb(lib, bc=0) == _lib.TTT_E_NULL
    assert _dmb(lib, Wc=FAKE + 8 * (1 << 20)) == _lib.TTT_E_ALIAS   # W_chunk is W
    assert _dmb(lib, Wc=FAKE) == _lib.TTT_E_ALIAS                   # W_chunk over xq
    assert _dmb(lib, mb=1, pos=0, Wc=0, bc=0, T=0) == _lib.TTT_OK  # mb = 1 ignores them
    assert _dmb(lib, T=0, pos=3) == _lib.TTT_OK


def test_linear_backward_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.ttt_linear_backward_workspace(2, 3, 40, 64, 16, ctypes.byref(n)) == _lib.TTT_OK
    # ceil(40 / 16) = 3 chunks, each a start state (W, b) and a record (five [16 x d] row
    # tensors, two values per row, two per feature)
    assert n.value == 2 * 3 * 3 * (64 * 64 + 64 + 5 * 16 * 64 + 2 * 16 + 2 * 64) * 4
    assert lib.ttt_linear_backward_workspace(1, 1, 16, 16, 16, ctypes.byref(n)) == _lib.TTT_OK
    assert n.value == (16 * 16 + 16 + 5 * 16 * 16 + 2 * 16 + 2 * 16) * 4
    assert lib.ttt_linear_backward_workspace(2, 3, 0, 16, 4, ctypes.byref(n)) == _lib.TTT_OK
    assert n.value == 0
    assert lib.ttt_linear_backward_workspace(2, 3, 40, 48, 16, ctypes.byref(n)) == _lib.TTT_E_SHAPE
    assert lib.ttt_linear_backward_workspace(2, 3, 40, 64, 16, None) == _lib.TTT_E_NULL


def test_linear_backward_validation(lib):
    assert _bwd(lib, ws_bytes=1024) == _lib.TTT_E_SHAPE
    assert "workspace" in lib.ttt_last_error().decode()
    assert _bwd(lib, d=32) == _lib.TTT_E_SHAPE
    assert _bwd(lib, mb=0) == _lib.TTT_E_SHAPE
    assert _bwd(lib, io=3) == _lib.TTT_E_DTYPE
    assert _bwd(lib, eps=0.0) == _lib.TTT_E_SHAPE
    p = [FAKE + i * (1 << 24) for i in range(20)]
    q = list(p); q[9] = p[0]  # dXQ on XQ
    assert _bwd(lib, ptrs=q) == _lib.TTT_E_ALIAS
    q = list(p); q[12] = p[13]  # deta on dW0
    assert _bwd(lib, ptrs=q) == _lib.TTT_E_ALIAS
    assert _bwd(lib, ws=p[11]) == _lib.TTT_E_ALIAS  # workspace on dXV
    q = list(p); q[8] = 0  # dO
    assert _bwd(lib, ptrs=q) == _lib.TTT_E_NULL
    assert _bwd(lib, B=0) == _lib.TTT_OK  # nothing to do, no HIP call


def _gated(lib, B=1, H=1, L=16, d=64, mb=16, io=1, theta=None, eta_base=1 / 64, eps=1e-6,
           O=None):
    p = [FAKE + i * (1 << 20) for i in range(8)]
    th = theta if theta is not None else p[3]
    Oo = O if O is not None else FAKE + 11 * (1 << 20)
    return lib.ttt_linear_forward_gated(B, H, L, d, mb, io, eps, p[0], p[1], p[2], th, eta_base,
                                        p[4], p[5], 0, p[6], p[7], Oo, FAKE + 9 * (1 << 20),
                                        FAKE + 10 * (1 << 20), None)


def test_linear_forward_gated_validation(lib):
    assert _gated(lib, B=-1) == _lib.TTT_E_SHAPE
    assert _gated(lib, d=32) == _lib.TTT_E_SHAPE
    assert _gated(lib, eps=0.0) == _lib.TTT_E_SHAPE
    for bad in (float("inf"), float("nan")):
        assert _gated(lib, eta_base=bad) == _lib.TTT_E_SHAPE
        assert "eta_base" in lib.ttt_last_error().decode()
    assert _gated(lib, theta=0) == _lib.TTT_E_NULL
    assert "theta_lr" in lib.ttt_last_error().decode()
    assert _gated(lib, theta=FAKE + 3 * (1 << 20) + 4) == _lib.TTT_E_ALIGN
    assert _gated(lib, O=FAKE + 3 * (1 << 20)) == _lib.TTT_E_ALIAS  # O over theta_lr
    assert _gated(lib, B=0) == _lib.TTT_OK


def _opts(lib, loss=0, wd=0.0, B=1, d=64):
    p = [FAKE + i * (1 << 20) for i in range(8)]
    return lib.ttt_linear_forward_opts(B, 1, 16, d, 16, 1, 1e-6, p[0], p[1], p[2], p[3], p[4],
                                       p[5], 0, p[6], p[7], loss, wd, FAKE + 11 * (1 << 20),
                                       FAKE + 9 * (1 << 20), FAKE + 10 * (1 << 20), None)


def test_linear_forward_opts_validation(lib):
    assert _opts(lib, loss=2) == _lib.TTT_E_SHAPE
    assert "inner_loss" in lib.ttt_last_error().decode()
    assert _opts(lib, loss=-1) == _lib.TTT_E_SHAPE
    for bad in (-0.1, float("inf"), float("nan")):
        assert _opts(lib, wd=bad) == _lib.TTT_E_SHAPE
        assert "weight_decay" in lib.ttt_last_error().decode()
    assert _opts(lib, d=32) == _lib.TTT_E_SHAPE
    assert _opts(lib, loss=1, wd=0.5, B=0) == _lib.TTT_OK


def _mlp_opts(lib, loss=0, wd=0.0, B=1, d=64):
    p = [FAKE + i * (1 << 20) for i in range(15)]
    return lib.ttt_mlp_forward_opts(B, 1, 16, d, 16, 1, 1e-6, *p[:8], 0, p[8], p[9], loss, wd,
                                    *p[10:15], None)


def test_mlp_forward_opts_validation(lib):
    assert _mlp_opts(lib, loss=2) == _lib.TTT_E_SHAPE
    assert "inner_loss" in lib.ttt_last_error().decode()
    assert _mlp_opts(lib, loss=-1) == _lib.TTT_E_SHAPE
    for bad in (-0.1, float("inf"), float("nan")):
        assert _mlp_opts(lib, wd=bad) == _lib.TTT_E_SHAPE
        assert "weight_decay" in lib.ttt_last_error().decode()
    assert _mlp_opts(lib, d=32) == _lib.TTT_E_SHAPE
    assert _mlp_opts(lib, loss=1, wd=0.5, B=0) == _lib.TTT_OK


def _mlp_gated(lib, eta_base=0.5, theta=FAKE + 3 * (1 << 20), B=1, O=FAKE + 10 * (1 << 20)):
    p = [FAKE + i * (1 << 20) for i in range(15)]
    return lib.ttt_mlp_forward_gated(B, 1, 16, 64, 16, 1, 1e-6, p[0], p[1], p[2], theta, eta_base,
                                     *p[4:8], 0, p[8], p[9], O, *p[11:15], None)


def test_mlp_forward_gated_validation(lib):
    for bad in (float("nan"), float("inf")):
        assert _mlp_gated(lib, eta_base=bad) == _lib.TTT_E_SHAPE
        assert "eta_base" in lib.ttt_last_error().decode()
    assert _mlp_gated(lib, theta=0) == _lib.TTT_E_NULL
    assert "theta_lr" in lib.ttt_last_error().decode()
    assert _mlp_gated(lib, theta=FAKE + 3 * (1 << 20) + 4) == _lib.TTT_E_ALIGN
    assert _mlp_gated(lib, O=FAKE + 3 * (1 << 20)) == _lib.TTT_E_ALIAS  # O over theta_lr
    assert _mlp_gated(lib, B=0) == _lib.TTT_OK


def _dec_gated(lib, eta_base=0.5, theta=FAKE + 3 * (1 << 20), mb=1, T=4, d=64,
               o=FAKE + 8 * (1 << 20)):
    p = [FAKE + i * (1 << 20) for i in range(12)]
    return lib.ttt_decode_steps_gated(T, 2, 3, d, 1, 1e-6, mb, 0, p[0], p[1], p[2], theta, eta_base,
                                      p[4], p[5], p[6], p[7], p[9], p[10], o, None)


def test_decode_steps_gated_validation(lib):
    for bad in (float("nan"), float("-inf")):
        assert _dec_gated(lib, eta_base=bad) == _lib.TTT_E_SHAPE
        assert "eta_base" in lib.ttt_last_error().decode()
    assert _dec_gated(lib, theta=0) == _lib.TTT_E_NULL
    assert "theta_lr" in lib.ttt_last_error().decode()
    assert _dec_gated(lib, theta=FAKE + 3 * (1 << 20) + 2) == _lib.TTT_E_ALIGN
    assert _dec_gated(lib, o=FAKE + 3 * (1 << 20)) == _lib.TTT_E_ALIAS  # o over theta_lr
    assert _dec_gated(lib, d=32) == _lib.TTT_E_SHAPE
    assert _dec_gated(lib, T=-1) == _lib.TTT_E_SHAPE
    assert _dec_gated(lib, T=0) == _lib.TTT_OK  # returns before any launch


def _gate(lib, B=2, H=3, L=40, d=64, io=1, xk=FAKE, th=FAKE + (1 << 20), eta_base=0.5,
          eta=FAKE + 2 * (1 << 20)):
    return lib.ttt_eta_gate(B, H, L, d, io, xk, th, eta_base, eta, None)


def _gate_bwd(lib, B=2, H=3, L=40, d=64, io=1, deta=FAKE + 2 * (1 << 20),
              dxk=FAKE + 3 * (1 << 20), dth=FAKE + 4 * (1 << 20), eta_base=0.5):
    return lib.ttt_eta_gate_backward(B, H, L, d, io, FAKE, FAKE + (1 << 20), eta_base, deta, dxk,
                                     dth, None)


def test_eta_gate_validation(lib):
    assert _gate(lib, L=-1) == _lib.TTT_E_SHAPE
    assert _gate(lib, d=48) == _lib.TTT_E_SHAPE
    assert _gate(lib, io=2) == _lib.TTT_E_DTYPE
    assert _gate(lib, eta_base=float("nan")) == _lib.TTT_E_SHAPE
    assert _gate(lib, xk=0) == _lib.TTT_E_NULL
    assert _gate(lib, eta=0) == _lib.TTT_E_NULL
    assert _gate(lib, xk=FAKE + 8) == _lib.TTT_E_ALIGN
    assert _gate(lib, eta=FAKE + 64) == _lib.TTT_E_ALIAS
    assert _gate(lib, B=0) == _lib.TTT_OK and _gate(lib, L=0) == _lib.TTT_OK
    assert _gate_bwd(lib, d=8) == _lib.TTT_E_SHAPE
    assert _gate_bwd(lib, deta=0) == _lib.TTT_E_NULL
    assert _gate_bwd(lib, dth=0) == _lib.TTT_E_NULL
    assert _gate_bwd(lib, dxk=FAKE + 3 * (1 << 20) + 4) == _lib.TTT_E_ALIGN
    assert _gate_bwd(lib, dxk=FAKE) == _lib.TTT_E_ALIAS          # dXK over XK
    assert _gate_bwd(lib, dth=FAKE + 3 * (1 << 20) + 256) == _lib.TTT_E_ALIAS
    assert _gate_bwd(lib, B=0) == _lib.TTT_OK


def test_ln_bwd_validation(lib):
    assert lib.ttt_ln_l2_bwd(4, 48, FAKE, FAKE2, FAKE + 4096, FAKE + 8192, 1e-6,
                             FAKE2 + (1 << 20), None) == _lib.TTT_E_SHAPE
    assert lib.ttt_ln_l2_bwd(-1, 64, FAKE, FAKE2, FAKE + 4096, FAKE + 8192, 1e-6,
                             FAKE2 + (1 << 20), None) == _lib.TTT_E_SHAPE
    assert lib.ttt_ln_l2_bwd(4, 64, FAKE, FAKE2, FAKE + 4096, FAKE + 8192, 1e-6, FAKE,
                             None) == _lib.TTT_E_ALIAS
    assert lib.ttt_ln_l2_bwd(0, 64, None, None, FAKE, FAKE + 4096, 1e-6, None, None) == _lib.TTT_OK


def test_binding_rejects_cpu_tensors():
    import torch
    from test_sequence_layer_ttt_amd import ttt
    x = torch.zeros(1, 1, 16, 64)
    with pytest.raises(ValueError):
        ttt.ttt_linear_forward(x, x, x, torch.zeros(1, 1, 16), torch.zeros(1, 64, 64),
                               torch.zeros(1, 64), torch.ones(1, 64), torch.zeros(1, 64))


def test_backward_noalloc_rejects_inputs_beyond_its_scratch(lib):
    """The no-allocation backward refuses, before any HIP call, inputs whose
    checkpoints and chunk records exceed its fixed 64 MiB scratch (1777 d = 64 chunks)."""
    p = [FAKE + i * (1 << 24) for i in range(24)]

    def call(B, H, L):
        return lib.ttt_linear_backward_noalloc(B, H, L, 64, 16, 1, 1e-6, *p[:6], 0, *p[6:19], None)
    assert call(1, 1, 16 * 1778) == _lib.TTT_E_SHAPE
    msg = lib.ttt_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg
    assert call(1, 1, -1) == _lib.TTT_E_SHAPE


def _proj(lib, B=1, L=16, dm=64, H=1, d=64, ptrs=None):
    p = ptrs or [FAKE + i * (1 << 24) for i in range(5)]
    return lib.ttt_qkv_project(B, L, dm, H, d, *[ctypes.c_void_p(x) for x in p], None)


def test_qkv_project_rejects_bad_arguments(lib):
    TTT_E_NULL, TTT_E_SHAPE, TTT_E_ALIGN, TTT_E_ALIAS = -1, -2, -4, -5
    assert _proj(lib, d=32) == TTT_E_SHAPE
    assert _proj(lib, dm=96) == TTT_E_SHAPE
    assert _proj(lib, dm=0) == TTT_E_SHAPE
    assert _proj(lib, B=-1) == TTT_E_SHAPE
    assert _proj(lib, B=1 << 16, L=1 << 16) == TTT_E_SHAPE          # B*L > INT_MAX
    p = [FAKE + i * (1 << 24) for i in range(5)]
    assert _proj(lib, ptrs=[0] + p[1:]) == TTT_E_NULL
    assert _proj(lib, ptrs=p[:2] + [p[2] + 8] + p[3:]) == TTT_E_ALIGN
    assert _proj(lib, ptrs=p[:2] + [p[0]] + p[3:]) == TTT_E_ALIAS   # XQ over X
    assert _proj(lib, ptrs=p[:3] + [p[2]] + p[4:]) == TTT_E_ALIAS   # XK over XQ
    assert _proj(lib, ptrs=p[:4] + [p[3]]) == TTT_E_ALIAS           # XV over XK
    # nothing to write: no pointer is needed and nothing is launched
    assert _proj(lib, L=0, ptrs=[0, 0, 0, 0, 0]) == 0


def _mbwd(lib, B=2, H=3, L=40, d=64, mb=16, io=1, eps=1e-6, ws_bytes=None, ptrs=None, ws=None,
          adj=(None, None, None, None)):
    p = ptrs or [FAKE + i * (1 << 24) for i in range(24)]
    need = ctypes.c_size_t(0)
    lib.ttt_mlp_backward_workspace(max(B, 0), max(H, 0), max(L, 0), 64, 16, ctypes.byref(need))
    nb = need.value if ws_bytes is None else ws_bytes
    return lib.ttt_mlp_backward(B, H, L, d, mb, io, eps, *p[:8], 0, p[8], p[9], p[10], *adj,
                                *p[11:21], ws if ws is not None else p[21], nb, None)


def test_mlp_backward_workspace_size(lib):
    n = ctypes.c_size_t(0)
    assert lib.ttt_mlp_backward_workspace(2, 3, 40, 64, 16, ctypes.byref(n)) == _lib.TTT_OK
    # ceil(40 / 16) = 3 chunk-start states plus two adjoint states, each W1, b1, W2, b2,
    # and 3 chunk records: eight [16 x 256] hidden tensors, five [16 x 64] row tensors,
    # two values per row and two per feature
    state = 2 * 64 * 256 + 256 + 64
    record = 8 * 16 * 256 + 5 * 16 * 64 + 2 * 16 + 2 * 64
    assert n.value == 2 * 3 * ((3 + 2) * state + 3 * record) * 4
    assert lib.ttt_mlp_backward_workspace(1, 1, 0, 64, 16, ctypes.byref(n)) == _lib.TTT_OK
    assert n.value == 2 * 132352
    assert lib.ttt_mlp_backward_workspace(2, 3, 40, 16, 16, ctypes.byref(n)) == _lib.TTT_E_SHAPE
    assert lib.ttt_mlp_backward_workspace(2, 3, 40, 64, 17, ctypes.byref(n)) == _lib.TTT_E_SHAPE
    assert lib.ttt_mlp_backward_workspace(2, 3, 40, 64, 16, None) == _lib.TTT_E_NULL
    # one pre-pass workgroup per chunk: B*H*ceil(L/mb) must fit a launch grid
    assert lib.ttt_mlp_backward_workspace(64, 64, 1 << 20, 64, 1, ctypes.byref(n)) == _lib.TTT_E_SHAPE


def test_mlp_backward_validation(lib):
    assert _mbwd(lib, ws_bytes=4096) == _lib.TTT_E_SHAPE
    assert "workspace" in lib.ttt_last_error().decode()
    assert _mbwd(lib, d=16) == _lib.TTT_E_SHAPE
    assert _mbwd(lib, mb=0) == _lib.TTT_E_SHAPE
    assert _mbwd(lib, io=3) == _lib.TTT_E_DTYPE
    assert _mbwd(lib, eps=0.0) == _lib.TTT_E_SHAPE
    assert _mbwd(lib, L=-1) == _lib.TTT_E_SHAPE
    p = [FAKE + i * (1 << 24) for i in range(24)]
    q = list(p); q[11] = p[0]  # dXQ on XQ
    assert _mbwd(lib, ptrs=q) == _lib.TTT_E_ALIAS
    q = list(p); q[15] = p[17]  # dW1 on dW2
    assert _mbwd(lib, ptrs=q) == _lib.TTT_E_ALIAS
    assert _mbwd(lib, ws=p[13]) == _lib.TTT_E_ALIAS  # workspace on dXV
    assert _mbwd(lib, adj=(p[15], None, None, None)) == _lib.TTT_E_ALIAS  # dW1_out is dW1
    q = list(p); q[10] = 0  # dO
    assert _mbwd(lib, ptrs=q) == _lib.TTT_E_NULL
    q = list(p); q[20] = 0  # dbeta
    assert _mbwd(lib, ptrs=q) == _lib.TTT_E_NULL
    q = list(p); q[4] = p[4] + 2  # W1_0 misaligned
    assert _mbwd(lib, ptrs=q) == _lib.TTT_E_ALIGN
    assert _mbwd(lib, B=0) == _lib.TTT_OK  # nothing to do, no HIP call
