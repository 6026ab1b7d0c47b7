"""float64 forward of one KDA layer (numpy + the C recurrence) -- TEST INFRASTRUCTURE ONLY.

Steps, as the explainer page "Kimi K3：开放前沿智能" describes the layer:
  * q, k, v projections of x; q and k then go through a causal depthwise short
    convolution, the Swish (SiLU) activation and L2 normalisation per head
    (section 2.4, paper Eq. 2); v is the plain projection;
  * the channel-wise decay logit comes from a low-rank projection plus bias,
    z = W_up W_down x + b_alpha (section 2.3, Eq. 2), mapped to
    log alpha = -5 * sigmoid(exp(A) z) (section 3.2, Eq. 5);
  * beta = sigmoid(x W_beta) (not on the page; the plainest reading);
  * the gated delta rule (section 2.2, Eq. 1) with readout S_t^T q_t (section 2.4);
  * per-head RMSNorm of the output, then a full-rank, data-dependent sigmoid
    gate sigmoid(x W_g) with W_g of size d x d (section 3.3, Eq. 6);
  * output projection W_o.
Readings where the page is silent: short-conv kernel 4 with no bias and a zero
initial window; L2 as x / sqrt(sum x^2 + eps); RMSNorm as
x / sqrt(mean x^2 + eps) * w; eps = 1e-6 for both; scale on q = 1.

Matrices are [in, out] (a projection is x @ W).  Conv taps are [channels, 4]
with tap 3 on the current token and tap 0 on the token three steps back.
The conv window state is [B, 3, 2*H*Dk] (q channels, then k channels; oldest
token first).

Parity status: pinned.  The composition against a hand-worked example
(tests/golden/kda_layer_hand_example.json: T=4, two heads, nonzero conv taps,
A and b_alpha nonzero, evaluated element by element at 40 digits), each piece
against a library routine or a closed form, the recurrence as pinned in the
package.
"""
from __future__ import annotations

import numpy as np

from .core import recurrence, decay_gate

EPS = 1e-6


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def l2norm(x, eps=EPS):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def rmsnorm(x, w, eps=EPS):
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def short_conv(x, w, state=None):
    """Causal depthwise convolution: y_t[c] = sum_j w[c, j] * x_{t-3+j}[c].

    x: [B, T, Ch]; w: [Ch, K]; state: [B, K-1, Ch] of earlier tokens (zeros if None).
    Returns (y [B, T, Ch], new state = the last K-1 input tokens).
    """
    B, T, Ch = x.shape
    K = w.shape[1]
    if state is None:
        state = np.zeros((B, K - 1, Ch))
    xp = np.concatenate([np.asarray(state, np.float64), x], axis=1)
    y = np.zeros((B, T, Ch))
    for j in range(K):
        y += w[:, j][None, None, :] * xp[:, j: j + T, :]
    return y, xp[:, T:, :]


def forward(x, p, S0=None, conv_state=None, scale: float = 1.0, threads=None, return_parts=False, eps: float = EPS):
    """Layer forward.  x: [B, T, d]; p: dict of weights (see synth.layer_inputs).

    Returns (y [B, T, d], S_T [B, H, Dk, Dv], conv_state_out [B, 3, 2*H*Dk]) in float64.
    """
    x = np.asarray(x, np.float64)
    B, T, d = x.shape
    H = p["A"].shape[0]
    HD = p["Wq"].shape[1]
    Dk = HD // H
    Dv = p["Wv"].shape[1] // H
    P = {n: np.asarray(a, np.float64) for n, a in p.items()}
    x2 = x.reshape(B * T, d)
    qp = (x2 @ P["Wq"]).reshape(B, T, HD)
    kp = (x2 @ P["Wk"]).reshape(B, T, HD)
    v = (x2 @ P["Wv"]).reshape(B, T, H, Dv)
    gl = (x2 @ P["Wg"]).reshape(B, T, H * Dv)
    beta = sigmoid(x2 @ P["Wbeta"]).reshape(B, T, H)
    z = ((x2 @ P["Wdown"]) @ P["Wup"] + P["b_alpha"]).reshape(B, T, H, Dk)
    g = decay_gate(z, P["A"])

    cs_q = cs_k = None
    if conv_state is not None:
        conv_state = np.asarray(conv_state, np.float64)
        cs_q, cs_k = conv_state[:, :, :HD], conv_state[:, :, HD:]
    qc, ns_q = short_conv(qp, P["conv_q"], cs_q)
    kc, ns_k = short_conv(kp, P["conv_k"], cs_k)
    q = l2norm(silu(qc).reshape(B, T, H, Dk), eps)
    k = l2norm(silu(kc).reshape(B, T, H, Dk), eps)

    o, ST = recurrence(q, k, v, g, beta, S0=S0, scale=scale, threads=threads)
    on = rmsnorm(o, P["rms_w"], eps).reshape(B, T, H * Dv)
    y = ((on * sigmoid(gl)).reshape(B * T, H * Dv) @ P["Wo"]).reshape(B, T, d)
    cs_out = np.concatenate([ns_q, ns_k], axis=2)
    if return_parts:
        return y, ST, cs_out, dict(q=q, k=k, v=v, g=g, beta=beta, o=o, gate=gl)
    return y, ST, cs_out
