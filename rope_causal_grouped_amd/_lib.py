"""ctypes loader for libgqa.so: the C-ABI declared in include/gqa.h.

The library must have been built (``python -m rope_causal_grouped_amd.build``);
there is no fallback of any kind when it is missing.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")

GQA_F32, GQA_BF16 = 0, 1
GQA_OK = 0
GQA_ERR_INVALID_ARG = -1
GQA_ERR_UNSUPPORTED = -2
GQA_ERR_WORKSPACE = -3
GQA_ERR_HIP = -4

# (name, restype, argtypes) for every exported function of include/gqa.h
_P, _I, _I64, _D, _F, _SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                            ctypes.c_double, ctypes.c_float, ctypes.c_size_t)
SIGNATURES = {
    "gqa_rope_apply": (_I, [_P, _I, _I64, _I64, _I, _I, _I64, _D, _P]),
    "gqa_prefill_workspace_size": (_SZ, [_I, _I64, _I64, _I, _I]),
    "gqa_prefill": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I64, _I, _I, _I, _D, _F, _I,
                         _P, _P, _I64, _P, _SZ, _P]),
    "gqa_decode_workspace_size": (_SZ, [_I64, _I, _I, _I, _I64]),
    "gqa_decode": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I, _I, _I, _I64, _I64, _I64, _D, _F,
                        _P, _SZ, _P]),
    "gqa_decode_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I, _I, _I, _I64, _I64, _I64, _D,
                                _F, _P]),
    "gqa_prefill_chunk_workspace_size": (_SZ, [_I, _I64, _I64, _I, _I]),
    "gqa_prefill_chunk": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I64, _I, _I, _I, _P, _P, _I64,
                               _D, _F, _I, _P, _P, _I64, _P, _SZ, _P]),
    "gqa_decode_ragged": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I, _I, _I, _I64, _P, _P, _I64,
                               _D, _F, _I, _P, _SZ, _P]),
    "gqa_decode_append": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I64, _I, _I, _I, _I64, _P,
                               _I64, _D, _F, _P, _SZ, _P]),
    "gqa_qkv_epilogue": (_I, [_P, _P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _P, _I64,
                              _D, _P]),
    "gqa_decode_paged_workspace_size": (_SZ, [_I64, _I, _I, _I, _I64]),
    "gqa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I64, _I, _I, _I, _I, _I64, _P,
                              _I64, _P, _P, _I64, _D, _F, _I, _P, _SZ, _P]),
    "gqa_set_rope_yarn": (_I, [_D, _D, _D, _D]),
    "gqa_last_error": (ctypes.c_char_p, []),
    "gqa_version": (ctypes.c_char_p, []),
    "gqa_timing_enable": (_I, [_I]),
    "gqa_timing_read": (_I, [_I, ctypes.POINTER(_D), ctypes.POINTER(_I64)]),
    "gqa_stream_read": (_I, [_P, _SZ, _P, _P]),
}

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gqa status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgqa.so once and attach the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m rope_causal_grouped_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int) -> None:
    if status != GQA_OK:
        raise GQAError(status, lib().gqa_last_error().decode())
