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
KDA_ERR_SCRATCH_LIMIT = -5
KDA_CP_NOALLOC_SCRATCH_BYTES = 32 << 20  # the fixed per-device scratch of kda_fwd_cp_noalloc
KDA_F32 = 0
KDA_BF16 = 1
KDA_FWD_PRECISE = 1  # kda_fwd_desc.flags
KDA_DECODE_SPECULATIVE = 1  # kda_layer_desc.flags for kda_layer_decode
KDA_VALIDATE = 2

# every symbol include/kda.h declares
EXPORTS = ("kda_fwd_workspace_size", "kda_fwd", "kda_fwd_ckpt", "kda_decode", "kda_fwd_cp_workspace_size", "kda_fwd_cp",
           "kda_fwd_cp_noalloc",
           "kda_bwd_workspace_size", "kda_bwd", "kda_layer_workspace_size", "kda_layer_fwd",
           "kda_layer_decode_workspace_size", "kda_layer_decode_cache_bytes", "kda_layer_decode", "kda_layer_decode_commit",
           "kda_error_string", "kda_version")


class FwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
        ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("chunk", ctypes.c_int),
        ("io_dtype", ctypes.c_int), ("o_dtype", ctypes.c_int),
        ("scale", ctypes.c_float), ("flags", ctypes.c_int),
    ]


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("d_model", ctypes.c_int), ("H", ctypes.c_int),
        ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("rank", ctypes.c_int), ("conv", ctypes.c_int),
        ("scale", ctypes.c_float), ("flags", ctypes.c_int),
    ]


LAYER_WEIGHT_FIELDS = ("Wq", "Wk", "Wv", "Wg", "Wo", "Wbeta", "Wdown", "Wup", "conv_q", "conv_k", "b_alpha", "A",
                       "rms_w")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_FIELDS]


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
            L.kda_fwd.argtypes = [ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p]
            L.kda_fwd_workspace_size.restype = ctypes.c_size_t
            L.kda_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc)]
            L.kda_fwd_cp_workspace_size.restype = ctypes.c_size_t
            L.kda_fwd_cp_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), ctypes.c_int]
            L.kda_fwd_cp.restype = ctypes.c_int
            L.kda_fwd_cp.argtypes = ([ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 8 + [ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p])
            L.kda_fwd_cp_noalloc.restype = ctypes.c_int
            L.kda_fwd_cp_noalloc.argtypes = ([ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 8 + [ctypes.c_int,
                                             ctypes.c_void_p])
            L.kda_bwd_workspace_size.restype = ctypes.c_size_t
            L.kda_bwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc)]
            L.kda_bwd.restype = ctypes.c_int
            L.kda_bwd.argtypes = ([ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 15 + [ctypes.c_size_t, ctypes.c_void_p])
            L.kda_decode.restype = ctypes.c_int
            L.kda_decode.argtypes = [ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 9
            L.kda_fwd_ckpt.restype = ctypes.c_int
            L.kda_fwd_ckpt.argtypes = ([ctypes.POINTER(FwdDesc)] + [ctypes.c_void_p] * 9 + [ctypes.c_int] +
                                       [ctypes.c_void_p])
            L.kda_layer_workspace_size.restype = ctypes.c_size_t
            L.kda_layer_workspace_size.argtypes = [ctypes.POINTER(LayerDesc)]
            L.kda_layer_fwd.restype = ctypes.c_int
            L.kda_layer_fwd.argtypes = ([ctypes.POINTER(LayerDesc), ctypes.c_void_p, ctypes.POINTER(LayerWeights)] +
                                        [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p])
            for n in ("kda_layer_decode_workspace_size", "kda_layer_decode_cache_bytes"):
                getattr(L, n).restype = ctypes.c_size_t
                getattr(L, n).argtypes = [ctypes.POINTER(LayerDesc)]
            L.kda_layer_decode.restype = ctypes.c_int
            L.kda_layer_decode.argtypes = ([ctypes.POINTER(LayerDesc), ctypes.c_void_p, ctypes.POINTER(LayerWeights)] +
                                           [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p])
            L.kda_layer_decode_commit.restype = ctypes.c_int
            L.kda_layer_decode_commit.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            L.kda_error_string.restype = ctypes.c_char_p
            L.kda_error_string.argtypes = [ctypes.c_int]
            L.kda_version.restype = ctypes.c_int
            L.kda_version.argtypes = []
            _lib = L
    return _lib


def check(code: int):
    if code != KDA_OK:
        raise KdaError(code, lib().kda_error_string(code).decode())


def layer_workspace_size(desc: LayerDesc) -> int:
    return lib().kda_layer_workspace_size(ctypes.byref(desc))


def layer_fwd_raw(desc: LayerDesc, x, weights: LayerWeights, S0, conv_in, y, S_T, conv_out, ws, ws_bytes,
                  stream) -> int:
    """Call kda_layer_fwd with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_layer_fwd(ctypes.byref(desc), x, ctypes.byref(weights), S0, conv_in, y, S_T, conv_out, ws,
                               ws_bytes, stream)


def layer_decode_workspace_size(desc: LayerDesc) -> int:
    return lib().kda_layer_decode_workspace_size(ctypes.byref(desc))


def layer_decode_cache_bytes(desc: LayerDesc) -> int:
    return lib().kda_layer_decode_cache_bytes(ctypes.byref(desc))


def layer_decode_raw(desc: LayerDesc, x, weights: LayerWeights, S, conv_state, y, cache, ws, ws_bytes, stream) -> int:
    """Call kda_layer_decode with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_layer_decode(ctypes.byref(desc), x, ctypes.byref(weights), S, conv_state, y, cache, ws, ws_bytes,
                                  stream)


def layer_decode_commit_raw(desc: LayerDesc, cache, n_accept, S, conv_state, stream) -> int:
    """Call kda_layer_decode_commit with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_layer_decode_commit(ctypes.byref(desc), cache, n_accept, S, conv_state, stream)


def fwd_workspace_size(desc: FwdDesc) -> int:
    return lib().kda_fwd_workspace_size(ctypes.byref(desc))


def fwd_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, stream, ws=0, ws_bytes=0) -> int:
    """Call kda_fwd with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_fwd(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, ws, ws_bytes, stream)


def fwd_ckpt_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, S_ckpt, every, stream) -> int:
    """Call kda_fwd_ckpt with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_fwd_ckpt(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, S_ckpt, every, stream)


def decode_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, stream) -> int:
    """Call kda_decode with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_decode(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, stream)


def cp_workspace_size(desc: FwdDesc, nseg: int) -> int:
    return lib().kda_fwd_cp_workspace_size(ctypes.byref(desc), nseg)


def fwd_cp_noalloc_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, nseg, stream) -> int:
    """Call kda_fwd_cp_noalloc with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_fwd_cp_noalloc(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, nseg, stream)


def fwd_cp_raw(desc: FwdDesc, q, k, v, g, beta, S0, o, S_T, nseg, ws, ws_bytes, stream) -> int:
    """Call kda_fwd_cp with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_fwd_cp(ctypes.byref(desc), q, k, v, g, beta, S0, o, S_T, nseg, ws, ws_bytes, stream)


def bwd_workspace_size(desc: FwdDesc) -> int:
    return lib().kda_bwd_workspace_size(ctypes.byref(desc))


def bwd_raw(desc: FwdDesc, q, k, v, g, beta, S0, dO, dST, dq, dk, dv, dg, dbeta, dS0, ws, ws_bytes, stream) -> int:
    """Call kda_bwd with integer device addresses (0 = NULL); returns the status code."""
    return lib().kda_bwd(ctypes.byref(desc), q, k, v, g, beta, S0, dO, dST, dq, dk, dv, dg, dbeta, dS0, ws, ws_bytes,
                         stream)
