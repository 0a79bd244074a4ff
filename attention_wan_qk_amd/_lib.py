"""ctypes loader for libwanattn.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

# The binding only ever loads the in-tree build next to this file.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwanattn.so")

WAN_SUCCESS = 0
WAN_ERROR_INVALID_VALUE = 1
WAN_ERROR_NOT_SUPPORTED = 2
WAN_ERROR_LAUNCH = 3

WAN_NORM = 1
WAN_ROPE = 2
WAN_NORM_PER_HEAD = 4

# Exported symbol -> (restype, argtypes); mirrors include/wanattn.h.
_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_U = ctypes.c_uint
SIGNATURES = {
    "wan_status_string": (ctypes.c_char_p, [_I]),
    "wan_version": (_I, []),
    "wan_qk_norm_rope3d": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _L, _L, _F, _F, _U, _P]),
    "wan_self_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _L,
                               _F, _P]),
    "wan_self_attn_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "wan_self_attn_fwd_ws": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _L,
                                  _F, _P, ctypes.c_size_t, _P]),
    "wan_self_attn_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L, _L, _L, _L,
                                       _F, _P]),
    "wan_cross_attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _L, _L, _L, _F,
                                _P]),
    "wan_chunk_causal_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _L, _L, _L, _L, _F, _P]),
    "wan_adaln_modulate_gate": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _L, _L, _F,
                                     _P]),
    "wan_linear_fwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _L, _L, _L, _P]),
    "wan_quantize_qkv_8bit": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L,
                                   _L, _L, _P]),
    "wan_self_attn_fwd_8bit": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _L,
                                    _F, _P]),
}

_lib = None


class WanError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        name = {1: "WAN_ERROR_INVALID_VALUE", 2: "WAN_ERROR_NOT_SUPPORTED",
                3: "WAN_ERROR_LAUNCH"}.get(status, f"status {status}")
        super().__init__(f"{call} failed: {name}")


def lib() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m attention_wan_qk_amd.build` "
                "(there is no fallback implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def check(call: str, status: int) -> None:
    if status != WAN_SUCCESS:
        raise WanError(call, status)
