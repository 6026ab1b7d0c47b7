"""ctypes binding of libkda.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_HIP = -3
KDA_ERR_WORKSPACE = -4
KDA_F32 = 0
KDA_BF16 = 1

# every symbol include/kda.h declares
EXPORTS = ("kda_fwd", "kda_error_string", "kda_version")


class FwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
        ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("chunk", ctypes.c_int),
        ("io_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
        ("scale", ctypes.c_float), ("flags", ctypes.c_int),
    ]


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lock = threading.Lock()
_lib = None


def lib():
    """Load libkda.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is missing: build it with `python -m linear_recurrent_attention_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            L.kda_fwd.restype = ctypes.c_int
            L.kda_fwd.argtypes = [ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 9
            L.kda_error_string.restype = ctypes.c_char_p
            L.kda_error_string.argtypes = [ctypes.c_int]
            L.kda_version.restype = ctypes.c_int
            L.kda_version.argtypes = []
            _lib = L
    return _lib


def check(code: int):
    if code != KDA_OK:
        raise KdaError(code, lib().kda_error_string(code).decode())


def fwd_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, stream) -> int:
    """Call kda_fwd with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_fwd(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, stream)
