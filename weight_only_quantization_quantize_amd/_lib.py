"""ctypes binding of libwoq (the C ABI declared in include/woq.h).

Argument marshalling only: every step of quantization and matmul runs in the
HIP kernels of libwoq.so.  The library is loaded on first use; if it has not
been built the call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("WOQ_LIBRARY", os.path.join(HERE, "libwoq.so"))

WOQ_OK = 0
WOQ_ERR_INVALID_ARGUMENT = 1
WOQ_ERR_UNSUPPORTED = 2
WOQ_ERR_HIP = 3
WOQ_ERR_INTERNAL = 4
WOQ_F16 = 0
WOQ_BF16 = 1
WOQ_LAYOUT_V2 = 2

_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class QMatrix(ctypes.Structure):
    """woq_qmatrix: one matrix of woq_quantize_pack_many."""
    _fields_ = [("W", _vp), ("act_scale", _vp), ("packed", _vp), ("scales", _vp), ("zeros", _vp), ("N", _i64),
                ("K", _i64)]


# name -> (restype, argtypes); mirrors include/woq.h
SIGNATURES = {
    "woq_layout_version": (_i32, []),
    "woq_packed_bytes": (_sz, [_i64, _i64, _i32]),
    "woq_scales_bytes": (_sz, [_i64, _i64, _i32]),
    "woq_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "woq_quantize_pack": (_i32, [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "woq_quantize_pack_many": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp]),
    "woq_w4a16_gemv": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "woq_w4a16_gemm": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _sz,
                              _vp]),
    "woq_dequantize": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp]),
    "woq_awq_search_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
    "woq_awq_search": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "woq_awq_search_noalloc_max_bytes": (_sz, []),
    "woq_awq_search_noalloc": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "woq_gptq_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "woq_gptq_quantize_pack": (_i32, [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_double, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "woq_probe_stream_read": (_i32, [_vp, _sz, _i32, _i32, _i32, _vp, _i32, _vp]),
    "woq_probe_empty": (_i32, [_i32, _i32, _vp]),
    "woq_probe_mfma_rate": (_i32, [_vp, _i32, _i32, _vp, _i32, _vp]),
    "woq_probe_mfma_valu": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "woq_probe_gemv_timeline_words": (_sz, [_i64]),
    "woq_probe_gemv_timeline": (_i32, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "woq_status_string": (ctypes.c_char_p, [_i32]),
    "woq_last_error": (ctypes.c_char_p, []),
}

_lib = None
_lock = threading.Lock()


class WoqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load libwoq.so once and attach the signatures of include/woq.h."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"libwoq.so is not built ({LIB_PATH}); run "
                    "`python -m weight_only_quantization_quantize_amd.build` (or __graft_entry__.build())"
                )
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check(status: int, what: str) -> None:
    if status != WOQ_OK:
        lib = load()
        name = lib.woq_status_string(status).decode()
        detail = lib.woq_last_error().decode()
        raise WoqError(status, f"{what} failed: {name}: {detail}")


def call(name: str, *args) -> int:
    """Call an entry point by name and return its raw result."""
    return getattr(load(), name)(*args)
