"""Seeded generators for the five KDA forward workloads.

Every array is drawn in float64 from numpy's PCG64 and then rounded once to
the dtype the kernel receives.  Both the GPU path and the CPU oracle consume
the *rounded* values (bf16 values are carried as float32 arrays, which hold
them exactly), so rounding of the inputs is never a source of disagreement.

Draws are made per (block of tokens, head), each from its own
``SeedSequence([seed, workload, 1, block, head])`` stream, in the order q, k,
v, beta logit, z, so a block can be regenerated on its own (the
million-token workload is streamed this way) and the pieces can be drawn on
several threads.  Per-head parameters come from the stream
``[seed, workload, 0]``.

Input recipe (the reading of the workload descriptions):
  * q, k: N(0,1) per element, then scaled to unit L2 norm per (token, head);
  * v: N(0,1);
  * beta: sigmoid of an N(0,1) logit;
  * g (= log alpha, per channel): -5 * sigmoid(exp(A_h) * z), z ~ N(0, var_z);
  * S0: N(0, var_S0) or absent (zero state);
  * "N(0, s)" in the workload text is read with s as the variance.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

G_MIN = -5.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    io: str            # "f32" or "bf16": dtype of q, k, v and o
    var_z: float       # variance of the decay logit z
    A_uniform: bool    # per-head A ~ U(-1, 1) (else A = 0)
    var_S0: float      # 0 => no initial state
    block: int = 4096  # tokens per generator block
    chunk: int = 64


WORKLOADS = {
    0: Workload("kda_fwd_f32_B1_H2_T256_D64", 1, 2, 256, 64, 64, "f32", 1.0, False, 0.0, block=256),
    1: Workload("kda_fwd_bf16_B1_H16_T4096_D128", 1, 16, 4096, 128, 128, "bf16", 1.0, True, 0.1),
    2: Workload("kda_fwd_bf16_B4_H32_T16384_D128", 4, 32, 16384, 128, 128, "bf16", 2.0, False, 0.0),
    3: Workload("kda_fwd_bf16_B1_H16_T1048576_D128", 1, 16, 1 << 20, 128, 128, "bf16", 1.0, True, 0.1,
                block=1 << 16),
}

# decode: one new token for each of B sequences, after a prefill (S0 stands for the prefill's state)
DECODE = dict(name="kda_decode_bf16_B128_H32_T1_D128", B=128, H=32, T=1, D=128, var_S0=0.1)

LAYER = dict(name="kda_layer_fwd_bf16_B2_T8192_d2048_H16_D128", B=2, T=8192, d=2048, H=16, Dk=128, Dv=128,
             rank=128, conv=4)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    # finite values stay below 2^32 after the rounding increment (|x| <= 0x7F7FFFFF + 0x8000 with sign)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """bf16-rounded values carried in a float32 array (exact)."""
    b = bf16_bits(x).astype(np.uint32)
    b <<= 16
    return b.view(np.float32)


def _io_round(x: np.ndarray, io: str) -> np.ndarray:
    return bf16_round(x) if io == "bf16" else x.astype(np.float32)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *[int(k) for k in key]])))


def head_params(wid: int, seed: int = 0, H: int | None = None):
    """Per-head decay scale A [H] (float64) and initial state S0 [B,H,Dk,Dv] (float32 or None)."""
    w = WORKLOADS[wid]
    H = w.H if H is None else H
    rng = _rng(seed, wid, 0)
    A = rng.uniform(-1.0, 1.0, size=H) if w.A_uniform else np.zeros(H)
    S0 = None
    if w.var_S0 > 0:
        S0 = (rng.standard_normal((w.B, H, w.Dk, w.Dv)) * np.sqrt(w.var_S0)).astype(np.float32)
    return A, S0


def _unit(wid: int, j: int, h: int, seed: int, A_h: float, need_q: bool):
    """Draws of token block j, head h: dict of float32 arrays shaped [B, block, *]."""
    w = WORKLOADS[wid]
    TB = min(w.block, w.T)
    rng = _rng(seed, wid, 1, j, h)
    shp_k = (w.B, TB, w.Dk)
    q_raw = rng.standard_normal(shp_k)
    k_raw = rng.standard_normal(shp_k)
    v = rng.standard_normal((w.B, TB, w.Dv))
    beta_logit = rng.standard_normal((w.B, TB))
    z = rng.standard_normal(shp_k)
    out = {}
    if need_q:
        out["q"] = _io_round(q_raw / np.linalg.norm(q_raw, axis=-1, keepdims=True), w.io)
    del q_raw
    out["k"] = _io_round(k_raw / np.linalg.norm(k_raw, axis=-1, keepdims=True), w.io)
    out["v"] = _io_round(v, w.io)
    out["beta"] = _sigmoid(beta_logit).astype(np.float32)
    z *= np.sqrt(w.var_z) * np.exp(A_h)
    out["g"] = (G_MIN * _sigmoid(z)).astype(np.float32)
    return out


def _pool(threads: int | None):
    return _cf.ThreadPoolExecutor(max_workers=threads or min(16, os.cpu_count() or 1))


def core_inputs_block(wid: int, j: int, seed: int = 0, A: np.ndarray | None = None, need_q: bool = True,
                      threads: int | None = None):
    """Inputs for token block j of workload wid: dict of float32 arrays shaped [B, block, H, *].
    Heads are drawn on up to `threads` threads (each head has its own stream)."""
    w = WORKLOADS[wid]
    if A is None:
        A, _ = head_params(wid, seed)
    TB = min(w.block, w.T)
    out = {"k": np.empty((w.B, TB, w.H, w.Dk), np.float32), "v": np.empty((w.B, TB, w.H, w.Dv), np.float32),
           "g": np.empty((w.B, TB, w.H, w.Dk), np.float32), "beta": np.empty((w.B, TB, w.H), np.float32)}
    if need_q:
        out["q"] = np.empty((w.B, TB, w.H, w.Dk), np.float32)

    def fill(h):
        for name, arr in _unit(wid, j, h, seed, float(A[h]), need_q).items():
            out[name][:, :, h] = arr

    with _pool(threads) as ex:
        list(ex.map(fill, range(w.H)))
    return out


def core_inputs(wid: int, seed: int = 0, T: int | None = None, threads: int | None = None):
    """All inputs of workload wid (optionally only its first T tokens).

    Returns dict(q, k, v, g, beta: float32 [B,T,H,*]; S0: float32 [B,H,Dk,Dv] or None; A: float64 [H]).
    """
    w = WORKLOADS[wid]
    T = w.T if T is None else T
    A, S0 = head_params(wid, seed)
    TB = min(w.block, w.T)
    nblk = (T + TB - 1) // TB
    out = {
        "q": np.empty((w.B, T, w.H, w.Dk), np.float32),
        "k": np.empty((w.B, T, w.H, w.Dk), np.float32),
        "v": np.empty((w.B, T, w.H, w.Dv), np.float32),
        "g": np.empty((w.B, T, w.H, w.Dk), np.float32),
        "beta": np.empty((w.B, T, w.H), np.float32),
    }

    def fill(jh):
        j, h = divmod(jh, w.H)
        t0, t1 = j * TB, min(T, (j + 1) * TB)
        for name, arr in _unit(wid, j, h, seed, float(A[h]), True).items():
            out[name][:, t0:t1, h] = arr[:, : t1 - t0]

    with _pool(threads) as ex:
        list(ex.map(fill, range(nblk * w.H)))
    out["S0"] = S0
    out["A"] = A
    return out


def window_start(T: int, window: int, seed: int = 0, chunk: int = 64) -> int:
    """Start of the checked window: chunk * U{0, ..., (T - window) / chunk}, drawn from the seed."""
    rng = _rng(seed, 3, 2)
    return chunk * int(rng.integers(0, (T - window) // chunk + 1))


def layer_inputs(seed: int = 0, B: int | None = None, T: int | None = None, d: int | None = None,
                 H: int | None = None, D: int | None = None, rank: int | None = None):
    """Input x and random-init weights of the fused KDA layer (bf16 values in float32 arrays).

    Weights ~ N(0, 1/fan_in); conv taps ~ N(0, 1/4); alpha bias 0; A = 0; RMSNorm weight 1.
    Matrices are stored [in, out] so that a projection is x @ W.
    """
    L = LAYER
    B = L["B"] if B is None else B
    T = L["T"] if T is None else T
    d = L["d"] if d is None else d
    H = L["H"] if H is None else H
    D = L["Dk"] if D is None else D
    R = L["rank"] if rank is None else rank
    HD = H * D
    rng = _rng(seed, 4, 0)

    def w(fan_in, shape):
        return bf16_round(rng.standard_normal(shape) / np.sqrt(fan_in))

    x = bf16_round(rng.standard_normal((B, T, d)))
    p = {
        "Wq": w(d, (d, HD)), "Wk": w(d, (d, HD)), "Wv": w(d, (d, HD)), "Wg": w(d, (d, HD)),
        "Wo": w(HD, (HD, d)), "Wbeta": w(d, (d, H)), "Wdown": w(d, (d, R)), "Wup": w(R, (R, HD)),
        "conv_q": (rng.standard_normal((HD, L["conv"])) * 0.5).astype(np.float32),
        "conv_k": (rng.standard_normal((HD, L["conv"])) * 0.5).astype(np.float32),
        "b_alpha": np.zeros(HD, np.float32), "A": np.zeros(H, np.float32), "rms_w": np.ones(D, np.float32),
    }
    return x, p


def decode_inputs(seed: int = 0, B: int | None = None, H: int | None = None, D: int | None = None,
                  T: int | None = None):
    """Inputs of the decode workload: the workload-1 distributions (A ~ U(-1,1) per head, z ~ N(0,1),
    bf16 q/k/v) for T new tokens per sequence, and S0 ~ N(0, 0.1) float32.
    Returns (dict(q, k, v, g, beta) of float32 arrays [B,T,H,*], S0 [B,H,D,D])."""
    w = DECODE
    B = w["B"] if B is None else B
    H = w["H"] if H is None else H
    D = w["D"] if D is None else D
    T = w["T"] if T is None else T
    rng = _rng(seed, 5, 0)
    A = rng.uniform(-1.0, 1.0, size=H)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    v = rng.standard_normal((B, T, H, D))
    beta_logit = rng.standard_normal((B, T, H))
    z = rng.standard_normal((B, T, H, D)) * np.exp(A)[None, None, :, None]
    S0 = (rng.standard_normal((B, H, D, D)) * np.sqrt(w["var_S0"])).astype(np.float32)
    d = {"q": bf16_round(q / np.linalg.norm(q, axis=-1, keepdims=True)),
         "k": bf16_round(k / np.linalg.norm(k, axis=-1, keepdims=True)),
         "v": bf16_round(v), "beta": _sigmoid(beta_logit).astype(np.float32),
         "g": (G_MIN * _sigmoid(z)).astype(np.float32)}
    return d, S0
