"""float64 chunkwise form of the KDA backward pass (numpy) -- TEST INFRASTRUCTURE ONLY.

An independent algorithm for the same gradients as ``oracle.backward`` (reverse mode through the
token recurrence): reverse mode through the chunkwise forward of ``oracle.chunkwise`` (section 2.5
of the explainer page "Kimi K3：开放前沿智能", paper Eq. 4).  The pages give no backward formulas;
these are the chain rule applied to each line of the chunkwise forward, in reverse order.

Per chunk, with the forward quantities (Q already scaled)
  Qg = Q*Gamma, Kg = K*Gamma, Kh = K/Gamma, Kb = K*exp(b_last - b), gam = Gamma_last,
  L = tril(Kg Kh^T, -1), A = tril(Qg Kh^T), N = (I + Diag(beta) L)^{-1}, Tm = N Diag(beta),
  X = V - Kg S, U = Tm X, O = Qg S + A U, S' = Diag(gam) S + Kb^T U,
and dS = dL/dS' (from the following chunks), dO = dL/dO of the chunk:
  dS_in  = Diag(gam) dS + Qg^T dO - Kg^T dX           (to the previous chunk)
  dU     = Kb dS + A^T dO;      dKb = U dS^T;          dgam = rowsum(dS * S)
  dQg    = dO S^T + dA Kh;      dA  = tril(dO U^T)
  dTm    = dU X^T;              dX  = Tm^T dU;         dV = dX;   dKg = -dX S^T + dL Kh
  dbeta  = colsum(N * dTm) + rowsum(dM * L),  dM = -N^T (dTm Diag(beta)) N^T
  dL     = tril(Diag(beta) dM, -1);  dKh = dL^T Kg + dA^T Qg
  dK     = dKg*Gamma + dKh/Gamma + dKb*exp(b_last - b);  dQ = dQg*Gamma
  db     = dQg*Qg + dKg*Kg - dKh*Kh - dKb*Kb,  plus sum_t dKb*Kb + dgam*gam at the chunk's last row
  dg     = reverse cumulative sum of db within the chunk.

Parity status: pinned (agrees with ``oracle.backward``, which agrees with finite differences of the
forward oracle).
"""
from __future__ import annotations

import numpy as np


def chunkwise_backward(q, k, v, g, beta, S0=None, dO=None, dST=None, scale: float = 1.0, C: int = 16):
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    out = {"dq": np.zeros((B, T, H, Dk)), "dk": np.zeros((B, T, H, Dk)), "dv": np.zeros((B, T, H, Dv)),
           "dg": np.zeros((B, T, H, Dk)), "dbeta": np.zeros((B, T, H)), "dS0": np.zeros((B, H, Dk, Dv))}
    starts = list(range(0, T, C))
    for b in range(B):
        for h in range(H):
            # forward sweep: the state entering each chunk
            S = np.zeros((Dk, Dv)) if S0 is None else np.array(S0[b, h], np.float64)
            Sin = []
            for c0 in starts:
                c1 = min(T, c0 + C)
                Sin.append(S.copy())
                f = _chunk(q, k, v, g, beta, b, h, c0, c1, scale, S)
                S = f["gam"][:, None] * S + f["Kb"].T @ f["U"]
            dS = np.zeros((Dk, Dv)) if dST is None else np.array(dST[b, h], np.float64)
            for ci in range(len(starts) - 1, -1, -1):
                c0 = starts[ci]
                c1 = min(T, c0 + C)
                S = Sin[ci]
                f = _chunk(q, k, v, g, beta, b, h, c0, c1, scale, S)
                dOc = np.zeros((c1 - c0, Dv)) if dO is None else np.asarray(dO[b, c0:c1, h], np.float64)
                Qg, Kg, Kh, Kb, Gam, gam = f["Qg"], f["Kg"], f["Kh"], f["Kb"], f["Gam"], f["gam"]
                L, A, N, Tm, X, U, bet = f["L"], f["A"], f["N"], f["Tm"], f["X"], f["U"], f["bet"]
                # S' = Diag(gam) S + Kb^T U
                dS_in = gam[:, None] * dS
                dgam = (dS * S).sum(1)
                dKb = U @ dS.T
                dU = Kb @ dS
                # O = Qg S + A U
                dQg = dOc @ S.T
                dS_in += Qg.T @ dOc
                dA = np.tril(dOc @ U.T)
                dU += A.T @ dOc
                # U = Tm X
                dTm = dU @ X.T
                dX = Tm.T @ dU
                # X = V - Kg S
                dV = dX
                dKg = -dX @ S.T
                dS_in -= Kg.T @ dX
                # Tm = N Diag(beta),  N = M^{-1},  M = I + Diag(beta) L
                dN = dTm * bet[None, :]
                dbet = (N * dTm).sum(0)
                dM = -N.T @ dN @ N.T
                dbet += (dM * L).sum(1)
                dL = np.tril(bet[:, None] * dM, -1)
                # L = tril(Kg Kh^T, -1),  A = tril(Qg Kh^T)
                dKg += dL @ Kh
                dKh = dL.T @ Kg + dA.T @ Qg
                dQg += dA @ Kh
                # the decay-scaled factors back to q, k and the cumulative decay b
                Eb = np.exp(f["bc"][-1][None, :] - f["bc"])
                dK = dKg * Gam + dKh / Gam + dKb * Eb
                dbc = dQg * Qg + dKg * Kg - dKh * Kh - dKb * Kb
                dbc[-1] += (dKb * Kb).sum(0) + dgam * gam
                dg = np.cumsum(dbc[::-1], axis=0)[::-1]
                out["dq"][b, c0:c1, h] = scale * dQg * Gam
                out["dk"][b, c0:c1, h] = dK
                out["dv"][b, c0:c1, h] = dV
                out["dg"][b, c0:c1, h] = dg
                out["dbeta"][b, c0:c1, h] = dbet
                dS = dS_in
            out["dS0"][b, h] = dS
    return out


def _chunk(q, k, v, g, beta, b, h, c0, c1, scale, S):
    """The chunkwise forward quantities of tokens [c0, c1) of sequence (b, h) from state S."""
    n = c1 - c0
    Q = scale * q[b, c0:c1, h]
    K = k[b, c0:c1, h]
    V = v[b, c0:c1, h]
    bet = beta[b, c0:c1, h]
    bc = np.cumsum(g[b, c0:c1, h], axis=0)
    Gam = np.exp(bc)
    Qg, Kg, Kh = Q * Gam, K * Gam, K / Gam
    Kb = K * np.exp(bc[-1][None, :] - bc)
    L = np.tril(Kg @ Kh.T, -1)
    A = np.tril(Qg @ Kh.T, 0)
    N = np.linalg.inv(np.eye(n) + bet[:, None] * L)
    Tm = N * bet[None, :]
    X = V - Kg @ S
    U = Tm @ X
    return dict(bet=bet, bc=bc, Gam=Gam, gam=Gam[-1], Qg=Qg, Kg=Kg, Kh=Kh, Kb=Kb, L=L, A=A, N=N, Tm=Tm, X=X,
                U=U)
