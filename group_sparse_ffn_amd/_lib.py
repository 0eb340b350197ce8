"""ctypes declarations for libwide.so (the C ABI in include/wide.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwide.so")

# Mirrors of the header's enums and macros.
WIDE_OK = 0
WIDE_ERR_NULL = 1
WIDE_ERR_SHAPE = 2
WIDE_ERR_DTYPE = 3
WIDE_ERR_ALIGN = 4
WIDE_ERR_WORKSPACE = 5
WIDE_ERR_UNSUPPORTED = 6
WIDE_ERR_HIP = 7

WIDE_F32 = 0
WIDE_BF16 = 1

WIDE_TOKEN_TILE = 256
WIDE_DECODE_T_LIMIT = 16
WIDE_FLAG_FORCE_PREFILL = 0x1
WIDE_FLAG_FORCE_DECODE = 0x2
WIDE_NOALLOC_SCRATCH_BYTES = 96 << 20

WIDE_ACT_IDENTITY = 0
WIDE_ACT_RELU = 1
WIDE_ACT_SILU = 2
WIDE_ATTN_ZERO_INACTIVE = 1

WIDE_STAGE_REORDER = 0
WIDE_STAGE_GATE_UP = 1
WIDE_STAGE_DOWN = 2
WIDE_STAGE_DECODE_GATE_UP = 3
WIDE_STAGE_DECODE_DOWN = 4

# Every symbol the header declares, with (restype, argtypes).
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_sz = ctypes.c_size_t
_FFN_ARGS = [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _p, _p, _sz, _u32, _p]
_GEMM_ARGS = [_p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int, _p, _p, _sz, _p]
SIGNATURES = {
    "wide_reorder_masks": (ctypes.c_int, [_p, _i32, _i32, _i32, _p, _p, _p, _p]),
    "wide_ffn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, ctypes.c_int]),
    "wide_ffn_workspace_size_for": (_sz, [_i32, _i32, _i32, _i32, ctypes.c_int, _i32]),
    "wide_ffn_forward": (ctypes.c_int, _FFN_ARGS),
    "wide_ffn_stage": (ctypes.c_int, [ctypes.c_int] + _FFN_ARGS),
    "wide_ffn_forward_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                                ctypes.c_int, _p, _p, _u32, _p]),
    "wide_decode_weights_size": (_sz, [_i32, _i32]),
    "wide_decode_prepare_weights": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _p, _sz, _p]),
    "wide_ffn_decode_prepared": (ctypes.c_int, [_p, _p, _p, _p, _p, _sz, _p, _i32, _i32, _i32,
                                                _i32, _p, _p, _p, _sz, _p]),
    "wide_gemm_workspace_size": (_sz, [_i32, _i32]),
    "wide_gemm_mn": (ctypes.c_int, _GEMM_ARGS),
    "wide_gemm_k": (ctypes.c_int, _GEMM_ARGS),
    "wide_router_workspace_size": (_sz, [_i32, _i32]),
    "wide_router_forward": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                           ctypes.c_int, _p, _p, _p, _sz, _p]),
    "wide_router_reorder_workspace_size": (_sz, [_i32, _i32]),
    "wide_router_reorder": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                           ctypes.c_int, _i32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "wide_attention_workspace_size": (_sz, [_i32, _i32, _i32]),
    "wide_attention_prefill": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                              _p, ctypes.c_uint32, _p, _sz, _p]),
    "wide_attention_decode_workspace_size": (_sz, [_i32, _i32, _i32]),
    "wide_attention_decode": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, ctypes.c_int,
                                             _p, ctypes.c_uint32, _p, _sz, _p]),
    "wide_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "wide_last_error": (ctypes.c_char_p, []),
    "wide_decode_max_t": (_i32, []),
}

_lib = None


class WideError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m group_sparse_ffn_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != WIDE_OK:
        lib = load()
        detail = lib.wide_last_error().decode()
        raise WideError(status, f"{lib.wide_status_string(status).decode()}: {detail}")
