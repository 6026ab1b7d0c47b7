"""Loader for the C recurrence oracle plus a plain numpy version of it.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_recurrence.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (float64, OpenMP).  -O3 vectorises the element-wise loops over
    value columns only (no reductions are reordered, and baseline x86-64 has no fused multiply-add),
    so the results are bit-for-bit those of an unoptimised build's arithmetic order."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
            f = lib.kda_oracle_recurrence
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 6 + [ctypes.c_double] + [ctypes.c_void_p] * 2 + [
                ctypes.c_int]
            fb = lib.kda_oracle_backward
            fb.restype = ctypes.c_int
            fb.argtypes = ([ctypes.c_int] * 6 + [ctypes.c_void_p] * 6 + [ctypes.c_double] + [ctypes.c_void_p] * 8 +
                           [ctypes.c_int])
            _lib = lib
    return _lib


def _threads(n):
    if n:
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def recurrence(q, k, v, g, beta, S0=None, scale: float = 1.0, want_o: bool = True, threads: int | None = None):
    """float64 gated delta rule over [B,T,H,*] inputs (float32 or float64 arrays).

    Returns (o [B,T,H,Dv] float64 or None, S_T [B,H,Dk,Dv] float64).
    """
    lib = _load()
    f64 = q.dtype == np.float64
    dt = np.float64 if f64 else np.float32
    q, k, v, g, beta = (np.ascontiguousarray(a, dtype=dt) for a in (q, k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    assert q.shape == k.shape == g.shape and v.shape[:3] == (B, T, H) and beta.shape == (B, T, H)
    S0p = None
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert S0.shape == (B, H, Dk, Dv)
        S0p = S0.ctypes.data
    o = np.empty((B, T, H, Dv), np.float64) if want_o else None
    ST = np.empty((B, H, Dk, Dv), np.float64)
    rc = lib.kda_oracle_recurrence(B, T, H, Dk, Dv, int(f64), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                   g.ctypes.data, beta.ctypes.data, S0p, float(scale),
                                   o.ctypes.data if want_o else None, ST.ctypes.data, _threads(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_recurrence failed ({rc})")
    return o, ST


def backward(q, k, v, g, beta, S0=None, dO=None, dST=None, scale: float = 1.0, threads: int | None = None):
    """float64 gradients of the gated delta rule (reverse-mode through the token steps), for output
    gradients dO [B,T,H,Dv] and dST [B,H,Dk,Dv] (None = zero).

    Returns dict(dq, dk, dg [B,T,H,Dk], dv [B,T,H,Dv], dbeta [B,T,H], dS0 [B,H,Dk,Dv]), float64.
    """
    lib = _load()
    f64 = q.dtype == np.float64
    dt = np.float64 if f64 else np.float32
    q, k, v, g, beta = (np.ascontiguousarray(a, dtype=dt) for a in (q, k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    assert q.shape == k.shape == g.shape and v.shape[:3] == (B, T, H) and beta.shape == (B, T, H)
    arrs = {}
    for name, a, shp in (("S0", S0, (B, H, Dk, Dv)), ("dO", dO, (B, T, H, Dv)), ("dST", dST, (B, H, Dk, Dv))):
        if a is not None:
            a = np.ascontiguousarray(a, dtype=np.float64)
            assert a.shape == shp, name
        arrs[name] = a
    out = {"dq": np.empty((B, T, H, Dk)), "dk": np.empty((B, T, H, Dk)), "dv": np.empty((B, T, H, Dv)),
           "dg": np.empty((B, T, H, Dk)), "dbeta": np.empty((B, T, H)), "dS0": np.empty((B, H, Dk, Dv))}
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    rc = lib.kda_oracle_backward(B, T, H, Dk, Dv, int(f64), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                 g.ctypes.data, beta.ctypes.data, ptr(arrs["S0"]), float(scale), ptr(arrs["dO"]),
                                 ptr(arrs["dST"]), out["dq"].ctypes.data, out["dk"].ctypes.data,
                                 out["dv"].ctypes.data, out["dg"].ctypes.data, out["dbeta"].ctypes.data,
                                 out["dS0"].ctypes.data, _threads(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed ({rc})")
    return out


def recurrence_np(q, k, v, g, beta, S0=None, scale: float = 1.0):
    """The same recurrence in numpy with explicit matrices, for small inputs.

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T (scale q_t),
    alpha_t = exp(g_t): the form of paper Eq. 1 as described in section 2.2 of the explainer page
    "Kimi K3：开放前沿智能", with the readout of its section 2.4.
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    I = np.eye(Dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], np.float64)
            for t in range(T):
                kt = k[b, t, h][:, None]
                E = I - beta[b, t, h] * (kt @ kt.T)
                S = E @ np.diag(np.exp(g[b, t, h])) @ S + beta[b, t, h] * kt @ v[b, t, h][None, :]
                o[b, t, h] = S.T @ (scale * q[b, t, h])
            ST[b, h] = S
    return o, ST


def decay_gate(z, A, g_min: float = -5.0):
    """Lower-bounded channel decay: log alpha = g_min * sigmoid(exp(A) * z).

    The scaled-sigmoid map of paper Eq. 5 (section 3.2 of the explainer page "Kimi K3：开放前沿智能"):
    g_min = -5 is fixed and A is a per-head learnable log-scale, so the factor on z is exp(A).
    z: [..., H, Dk]; A: [H].  float64.
    """
    z = np.asarray(z, np.float64)
    A = np.asarray(A, np.float64)
    return g_min / (1.0 + np.exp(-np.exp(A)[:, None] * z))
