"""Kimi Delta Attention forward on MI355X (gfx950).

The compute runs in libkda.so (hand-written HIP kernels behind a C ABI, see include/kda.h).
This module only marshals torch tensors (device memory and the current stream) into that ABI.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import KdaError  # noqa: F401

__all__ = ["kda_fwd", "KdaError"]

_DT = {torch.float32: _lib.KDA_F32, torch.bfloat16: _lib.KDA_BF16}


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def kda_fwd(q, k, v, g, beta, S0=None, scale: float = 1.0, o_dtype=None, want_state: bool = True,
            out=None, state_out=None, chunk: int = 0):
    """Gated delta rule forward.  Shapes: q, k, g [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H];
    S0 [B,H,Dk,Dv] float32 or None.  q, k, v float32 or bfloat16; g, beta float32.

    Returns (o [B,T,H,Dv], S_T [B,H,Dk,Dv] float32 or None).
    """
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for t in (q, k, v, g, beta):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous GPU tensors")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype: float32 or bfloat16")
    if g.dtype != torch.float32 or beta.dtype != torch.float32:
        raise ValueError("g and beta must be float32")
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    if S0 is not None and (S0.dtype != torch.float32 or S0.shape != (B, H, Dk, Dv) or not S0.is_contiguous()):
        raise ValueError("S0 must be a contiguous float32 [B,H,Dk,Dv] tensor")
    o_dtype = q.dtype if o_dtype is None else o_dtype
    o = out if out is not None else torch.empty((B, T, H, Dv), dtype=o_dtype, device=q.device)
    ST = None
    if want_state:
        ST = state_out if state_out is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                 device=q.device)
    desc = _lib.FwdDesc(B, T, H, Dk, Dv, chunk, _DT[q.dtype], _DT[o_dtype], float(scale), 0)
    code = _lib.fwd_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                        _stream(q.device))
    _lib.check(code)
    return o, ST
