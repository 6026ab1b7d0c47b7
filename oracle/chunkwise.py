"""float64 chunkwise-parallel form of the KDA forward pass (numpy) -- TEST INFRASTRUCTURE ONLY.

An independent algorithm for the same result as the token recurrence: the
sequence is cut into chunks of C tokens; inside a chunk all tokens are handled
at once with dense lower-triangular matrices, and only the d_k x d_v state is
passed from chunk to chunk (section 2.5 of the explainer page
"Kimi K3：开放前沿智能", paper Eq. 4: an inter-chunk term Gamma*Q*S plus an
intra-chunk term A*V_hat with a causal lower-triangular mask).

Per chunk, with incoming state S and r, s indexing tokens of the chunk:
  b_r     = sum_{j<=r} g_j                  cumulative log-decay per key channel
  Gamma_r = exp(b_r)
  Qg = Q*Gamma, Kg = K*Gamma, Kinv = K/Gamma, Kbar_s = k_s*exp(b_last - b_s)
  L  = strictly-lower part of Kg Kinv^T     (L_rs = sum_c k_rc k_sc Gamma_rc/Gamma_sc)
  A  = lower part (with diagonal) of Qg Kinv^T
  T  = (I + Diag(beta) L)^{-1} Diag(beta)   (the triangular "UT" inverse)
  U  = T (V - Kg S)                          ("V_hat" of Eq. 4)
  O  = Qg S + A U                            (inter term + intra term)
  S <- Diag(Gamma_last) S + Kbar^T U
Kinv can reach exp(5 * C) and stays finite in float64 for C up to 128 with g >= -5.
The triangular system is solved with numpy's dense solver (a library primitive).

Parity status: pinned (agrees with the recurrence; C = 1 reduces to it).
"""
from __future__ import annotations

import numpy as np


def chunkwise(q, k, v, g, beta, S0=None, scale: float = 1.0, C: int = 64):
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    o = np.zeros((B, T, H, Dv))
    ST = np.zeros((B, H, Dk, Dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], np.float64)
            for c0 in range(0, T, C):
                c1 = min(T, c0 + C)
                n = c1 - c0
                Q = scale * q[b, c0:c1, h]
                K = k[b, c0:c1, h]
                V = v[b, c0:c1, h]
                bet = beta[b, c0:c1, h]
                bc = np.cumsum(g[b, c0:c1, h], axis=0)
                Gam = np.exp(bc)
                Qg, Kg, Kinv = Q * Gam, K * Gam, K / Gam
                Kbar = K * np.exp(bc[-1][None, :] - bc)
                L = np.tril(Kg @ Kinv.T, -1)
                A = np.tril(Qg @ Kinv.T, 0)
                Tm = np.linalg.solve(np.eye(n) + bet[:, None] * L, np.diag(bet))
                U = Tm @ (V - Kg @ S)
                o[b, c0:c1, h] = Qg @ S + A @ U
                S = Gam[-1][:, None] * S + Kbar.T @ U
            ST[b, h] = S
    return o, ST
