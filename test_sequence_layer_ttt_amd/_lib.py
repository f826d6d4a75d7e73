"""Loader for libttt.so (the HIP / gfx950 library). There is no fallback:
if the library is not built, every entry point raises."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libttt.so")
HEADER = os.path.join(ROOT, "include", "ttt.h")

TTT_OK = 0
TTT_LOSS_MSE = 0
TTT_LOSS_INNER_PRODUCT = 1
TTT_E_NULL = -1
TTT_E_SHAPE = -2
TTT_E_DTYPE = -3
TTT_E_ALIGN = -4
TTT_E_ALIAS = -5
TTT_E_HIP = -6
TTT_F32 = 0
TTT_BF16 = 1

_lib = None

_P = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


class TTTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libttt error {code}: {msg}")
        self.code = code


def load():
    """Load libttt.so and declare the argument types of every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python test_sequence_layer_ttt_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ttt_linear_forward.argtypes = [_i] * 6 + [_f] + [_P] * 6 + [_i] + [_P] * 5 + [_P]
    lib.ttt_linear_forward_gated.argtypes = ([_i] * 6 + [_f] + [_P] * 4 + [_f] + [_P] * 2 + [_i]
                                            + [_P] * 5 + [_P])
    lib.ttt_linear_forward_opts.argtypes = ([_i] * 6 + [_f] + [_P] * 6 + [_i] + [_P] * 2
                                            + [_i, _f] + [_P] * 3 + [_P])
    lib.ttt_eta_gate.argtypes = [_i] * 5 + [_P, _P, _f, _P, _P]
    lib.ttt_qkv_project.argtypes = [_i] * 5 + [_P] * 5 + [_P]
    lib.ttt_eta_gate_backward.argtypes = [_i] * 5 + [_P, _P, _f, _P, _P, _P, _P]
    lib.ttt_mlp_forward.argtypes = [_i] * 6 + [_f] + [_P] * 8 + [_i] + [_P] * 7 + [_P]
    lib.ttt_mlp_forward_opts.argtypes = ([_i] * 6 + [_f] + [_P] * 8 + [_i] + [_P] * 2
                                         + [_i, _f] + [_P] * 5 + [_P])
    lib.ttt_mlp_forward_gated.argtypes = ([_i] * 6 + [_f] + [_P] * 4 + [_f] + [_P] * 4 + [_i]
                                          + [_P] * 2 + [_P] * 5 + [_P])
    lib.ttt_decode_step.argtypes = [_i] * 4 + [_f] + [_P] * 9 + [_P]
    lib.ttt_decode_steps.argtypes = [_i] * 5 + [_f] + [_P] * 9 + [_P]
    lib.ttt_decode_steps_mb.argtypes = [_i] * 5 + [_f] + [_i] * 2 + [_P] * 11 + [_P]
    lib.ttt_decode_steps_gated.argtypes = ([_i] * 5 + [_f] + [_i] * 2 + [_P] * 4 + [_f] + [_P] * 7
                                           + [_P])
    lib.ttt_linear_backward.argtypes = ([_i] * 6 + [_f] + [_P] * 6 + [_i] + [_P] * 14
                                        + [ctypes.c_size_t, _P])
    lib.ttt_linear_backward_noalloc.argtypes = ([_i] * 6 + [_f] + [_P] * 6 + [_i] + [_P] * 13
                                                + [_P])
    lib.ttt_linear_backward_workspace.argtypes = [_i] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_mlp_backward.argtypes = ([_i] * 6 + [_f] + [_P] * 8 + [_i] + [_P] * 18
                                     + [ctypes.c_size_t, _P])
    lib.ttt_mlp_backward_workspace.argtypes = [_i] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
    lib.ttt_ln_l2_bwd.argtypes = [_i, _i, _P, _P, _P, _P, _f, _P, _P]
    for name in ("ttt_linear_forward", "ttt_mlp_forward", "ttt_decode_step", "ttt_decode_steps",
                 "ttt_linear_backward", "ttt_linear_backward_workspace", "ttt_ln_l2_bwd",
                 "ttt_linear_backward_noalloc", "ttt_mlp_backward", "ttt_mlp_backward_workspace",
                 "ttt_linear_forward_gated", "ttt_eta_gate", "ttt_eta_gate_backward", "ttt_qkv_project",
                 "ttt_linear_forward_opts", "ttt_decode_steps_mb", "ttt_mlp_forward_opts",
                 "ttt_mlp_forward_gated", "ttt_decode_steps_gated",
                 "ttt_version"):
        getattr(lib, name).restype = _i
    lib.ttt_last_error.restype = ctypes.c_char_p
    lib.ttt_last_error.argtypes = []
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != TTT_OK:
        raise TTTError(code, load().ttt_last_error().decode())


def header_functions() -> list:
    """Names of the functions declared in include/ttt.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ttt_\w+)\s*\(", txt, re.M)))
