"""Kimi Delta Attention forward on MI355X (gfx950).

The compute runs in libkda.so (hand-written HIP kernels behind a C ABI, see include/kda.h).
This module only marshals torch tensors (device memory and the current stream) into that ABI.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import KdaError  # noqa: F401

__all__ = ["kda_fwd", "kda_fwd_ckpt", "kda_fwd_cp", "kda_fwd_cp_noalloc", "kda_layer_decode", "kda_layer_decode_commit", "kda_bwd", "kda_decode", "kda_layer_fwd", "KdaError"]

_DT = {torch.float32: _lib.KDA_F32, torch.bfloat16: _lib.KDA_BF16}


def _ptr(t):
    return 0 if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, out, state_out, chunk, precise, scale, validate=False,
              want_output=True):
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
    o = None
    if want_output:
        o = out if out is not None else torch.empty((B, T, H, Dv), dtype=o_dtype, device=q.device)
    ST = None
    if want_state:
        ST = state_out if state_out is not None else torch.empty((B, H, Dk, Dv), dtype=torch.float32,
                                                                 device=q.device)
    desc = _lib.FwdDesc(B, T, H, Dk, Dv, chunk, _DT[q.dtype], _DT[o_dtype], float(scale),
                        (_lib.KDA_FWD_PRECISE if precise else 0) | (_lib.KDA_VALIDATE if validate else 0))
    return desc, o, ST


def kda_fwd(q, k, v, g, beta, S0=None, scale: float = 1.0, o_dtype=None, want_state: bool = True,
            out=None, state_out=None, chunk: int = 0, precise: bool = False, validate: bool = False,
            workspace=None, want_output: bool = True):
    """Gated delta rule forward.  Shapes: q, k, g [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H];
    S0 [B,H,Dk,Dv] float32 or None.  q, k, v float32 or bfloat16; g, beta float32.
    precise: split-bf16 key Gram matrix and state update on the bf16 path (KDA_FWD_PRECISE).
    validate: check g in [-5, 0] and finite inputs first (KDA_VALIDATE; synchronises the stream and
    raises KdaError with KDA_ERR_INVALID_ARG on a finding).
    want_output=False (bf16 inputs): the state alone, on the leaner state-only kernel.

    Returns (o [B,T,H,Dv] or None, S_T [B,H,Dk,Dv] float32 or None).
    """
    desc, o, ST = _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, out, state_out, chunk, precise, scale,
                            validate, want_output)
    need = _lib.fwd_workspace_size(desc)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = _lib.fwd_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                        _stream(q.device), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())
    _lib.check(code)
    return o, ST


def kda_fwd_ckpt(q, k, v, g, beta, every: int, S0=None, scale: float = 1.0, o_dtype=None,
                 want_state: bool = True, chunk: int = 0, precise: bool = False, want_output: bool = True):
    """kda_fwd that also returns state checkpoints: S_ckpt [B,H,T//every,Dk,Dv] float32, entry m being
    the state after tokens [0, (m+1)*every) (the S0 that resumes the sequence there).
    want_output=False (bf16 inputs): the states alone (filling a prefix cache).

    Returns (o or None, S_T, S_ckpt)."""
    desc, o, ST = _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, None, None, chunk, precise, scale,
                            want_output=want_output)
    B, T, H, Dk = q.shape
    n = T // every if every > 0 else 0
    ck = torch.empty((B, H, n, Dk, v.shape[-1]), dtype=torch.float32, device=q.device)
    code = _lib.fwd_ckpt_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                             _ptr(ck) if n > 0 else 0, int(every), _stream(q.device))
    _lib.check(code)
    return o, ST, ck


def kda_fwd_cp(q, k, v, g, beta, S0=None, nseg: int = 0, scale: float = 1.0, o_dtype=None,
               want_state: bool = True, out=None, state_out=None, precise: bool = False, workspace=None):
    """kda_fwd with in-device context parallelism (kda_fwd_cp): each sequence is split into nseg
    segments (0 = automatic) that run side by side.  bf16 q/k/v only.  Returns (o, S_T)."""
    desc, o, ST = _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, out, state_out, 0, precise, scale)
    need = _lib.cp_workspace_size(desc, int(nseg))
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    code = _lib.fwd_cp_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                           int(nseg), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                           _stream(q.device))
    _lib.check(code)
    return o, ST


def kda_fwd_cp_noalloc(q, k, v, g, beta, S0=None, nseg: int = 0, scale: float = 1.0, o_dtype=None,
                       want_state: bool = True, out=None, state_out=None, precise: bool = False):
    """kda_fwd_cp without a workspace (kda_fwd_cp_noalloc): the library's fixed per-device scratch
    array holds the segment states, so the C call allocates nothing (pass out/state_out to allocate
    nothing here either).  Calls that overlap in time on one device race on that array.
    Raises KdaError with KDA_ERR_SCRATCH_LIMIT if the plan needs more than the array holds."""
    desc, o, ST = _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, out, state_out, 0, precise, scale)
    code = _lib.fwd_cp_noalloc_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o),
                                   _ptr(ST), int(nseg), _stream(q.device))
    _lib.check(code)
    return o, ST


def kda_bwd(q, k, v, g, beta, dO=None, dS_T=None, S0=None, scale: float = 1.0, workspace=None):
    """Gradients of kda_fwd (kda_bwd) for dL/do = dO (o's dtype, or None) and dL/dS_T = dS_T
    (float32, or None).  Returns dict(dq, dk, dv, dg, dbeta, dS0) of float32 tensors."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    o_dtype = q.dtype if dO is None else dO.dtype
    if dO is not None and (dO.shape != (B, T, H, Dv) or not dO.is_contiguous() or not dO.is_cuda):
        raise ValueError("dO must be a contiguous GPU [B,T,H,Dv] tensor")
    if dS_T is not None and (dS_T.dtype != torch.float32 or dS_T.shape != (B, H, Dk, Dv) or not dS_T.is_contiguous()):
        raise ValueError("dS_T must be a contiguous float32 [B,H,Dk,Dv] tensor")
    desc, _, _ = _fwd_args(q, k, v, g, beta, S0, o_dtype, False, q, None, 0, False, scale)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, Dk), **f32), "dk": torch.empty((B, T, H, Dk), **f32),
           "dv": torch.empty((B, T, H, Dv), **f32), "dg": torch.empty((B, T, H, Dk), **f32),
           "dbeta": torch.empty((B, T, H), **f32), "dS0": torch.empty((B, H, Dk, Dv), **f32)}
    need = _lib.bwd_workspace_size(desc)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = _lib.bwd_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(dO), _ptr(dS_T),
                        *[out[n].data_ptr() for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0")], ws.data_ptr(),
                        ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(code)
    return out


def kda_decode(q, k, v, g, beta, S0=None, scale: float = 1.0, o_dtype=None, want_state: bool = True,
               out=None, state_out=None):
    """Token-by-token step (kda_decode): the same result as kda_fwd for a few tokens per call.
    state_out may be S0 itself (in-place update).  Returns (o, S_T)."""
    desc, o, ST = _fwd_args(q, k, v, g, beta, S0, o_dtype, want_state, out, state_out, 0, False, scale)
    code = _lib.decode_raw(desc, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                           _stream(q.device))
    _lib.check(code)
    return o, ST


def kda_layer_fwd(x, weights: dict, S0=None, conv_state=None, scale: float = 1.0, want_state: bool = True,
                  workspace=None):
    """Fused KDA layer.  x [B,T,d_model] bf16; weights: dict with the kda_layer_weights fields
    (bf16 matrices [in, out]; float32 conv taps [H*Dk, 4], b_alpha [H*Dk], A [H], rms_w [Dv]).
    Returns (y [B,T,d_model] bf16, S_T [B,H,Dk,Dv] float32 or None, conv_state [B,3,2*H*Dk] float32)."""
    B, T, dm = x.shape
    H = weights["A"].shape[0]
    HD = weights["Wq"].shape[1]
    Dk = HD // H
    Dv = weights["Wv"].shape[1] // H
    R = weights["Wdown"].shape[1]
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 GPU tensor")
    for n in _lib.LAYER_WEIGHT_FIELDS:
        t = weights[n]
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"weight {n} must be a contiguous GPU tensor")
    desc = _lib.LayerDesc(B, T, dm, H, Dk, Dv, R, 4, float(scale), 0)
    need = _lib.layer_workspace_size(desc)
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=x.device)
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=x.device)
    ST = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=x.device) if want_state else None
    cs = torch.empty((B, 3, 2 * HD), dtype=torch.float32, device=x.device)
    W = _lib.LayerWeights(*[weights[n].data_ptr() for n in _lib.LAYER_WEIGHT_FIELDS])
    code = _lib.layer_fwd_raw(desc, x.data_ptr(), W, _ptr(S0), _ptr(conv_state), y.data_ptr(), _ptr(ST),
                              cs.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(code)
    return y, ST, cs


def _layer_desc(weights: dict, B: int, T: int, dm: int, scale: float, flags: int):
    H = weights["A"].shape[0]
    HD = weights["Wq"].shape[1]
    return _lib.LayerDesc(B, T, dm, H, HD // H, weights["Wv"].shape[1] // H, weights["Wdown"].shape[1], 4,
                          float(scale), flags)


def kda_layer_decode(x, weights: dict, S, conv_state=None, scale: float = 1.0, speculative: bool = False,
                     cache=None, workspace=None):
    """Layer decode step (kda_layer_decode) over x [B,T,d_model] bf16 (B*T <= 16): S [B,H,Dk,Dv] float32 and
    conv_state [B,3,2*H*Dk] float32 are updated in place unless speculative.  Returns (y, cache), cache a
    float32 tensor of the tokens' projection-input entries (allocated when speculative and not given)."""
    B, T, dm = x.shape
    desc = _layer_desc(weights, B, T, dm, scale, _lib.KDA_DECODE_SPECULATIVE if speculative else 0)
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 GPU tensor")
    if S.dtype != torch.float32 or not S.is_contiguous():
        raise ValueError("S must be a contiguous float32 tensor")
    if cache is None and speculative:
        cache = torch.empty(_lib.layer_decode_cache_bytes(desc) // 4, dtype=torch.float32, device=x.device)
    need = _lib.layer_decode_workspace_size(desc)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    y = torch.empty((B, T, dm), dtype=torch.bfloat16, device=x.device)
    W = _lib.LayerWeights(*[weights[n].data_ptr() for n in _lib.LAYER_WEIGHT_FIELDS])
    code = _lib.layer_decode_raw(desc, x.data_ptr(), W, S.data_ptr(), _ptr(conv_state), y.data_ptr(), _ptr(cache),
                                 ws.data_ptr(), ws.numel(), _stream(x.device))
    _lib.check(code)
    return y, cache


def kda_layer_decode_commit(cache, n_accept: int, S, conv_state, weights: dict, B: int, T: int, d_model: int):
    """Accept the first n_accept of the T draft tokens of a speculative kda_layer_decode call
    (kda_layer_decode_commit): S and conv_state advance in place over their cache entries."""
    desc = _layer_desc(weights, B, T, d_model, 1.0, 0)
    code = _lib.layer_decode_commit_raw(desc, _ptr(cache), int(n_accept), S.data_ptr(), _ptr(conv_state),
                                        _stream(S.device))
    _lib.check(code)
