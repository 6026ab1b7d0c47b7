"""Pins of the backward oracle (oracle.backward) against facts that do not come from it:
finite differences of the forward oracle, reverse-mode automatic differentiation of a plain
float64 torch transcription of the recurrence's definition, closed forms, and the chunkwise
backward (an independent algorithm) agreeing with it.  Each test names the mistake it catches."""
import numpy as np
import pytest

import oracle
from test_oracle_pins import rand_inputs

NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}


def loss_weights(rng, q, v, S0):
    B, T, H, _ = q.shape
    return rng.standard_normal((B, T, H, v.shape[-1])), rng.standard_normal(S0.shape)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    """Every gradient against central differences of L = <o, R_o> + <S_T, R_S> on a tiny problem
    with a non-unit scale and an initial state: catches any wrong term, sign, transpose or index."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=1, T=6, H=1, Dk=3, Dv=2, unit_k=False, gmin=-2.0)
    Ro, Rs = loss_weights(rng, q, v, S0)
    scale = 0.7
    args = dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)

    def loss(**a):
        o, S = oracle.recurrence(a["q"], a["k"], a["v"], a["g"], a["beta"], S0=a["S0"], scale=scale)
        return float((o * Ro).sum() + (S * Rs).sum())

    grad = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, scale=scale)
    h = 1e-6
    for n, a in args.items():
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            fd[idx] = (loss(**{**args, n: ap}) - loss(**{**args, n: am})) / (2 * h)
        np.testing.assert_allclose(grad[NAMES[n]], fd, rtol=1e-6, atol=1e-8, err_msg=n)


def test_backward_matches_torch_autograd_of_the_definition():
    """Reverse-mode autodiff (a library routine) of the recurrence written from its definition in
    float64 torch: catches a backward that is self-consistent but differentiates another function."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=9, H=2, Dk=5, Dv=4)
    Ro, Rs = loss_weights(rng, q, v, S0)
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0).items()}
    B, T, H, Dk = q.shape
    loss = 0.0
    for b in range(B):
        for hh in range(H):
            S = t["S0"][b, hh]
            for s in range(T):
                kk, qq, vv = t["k"][b, s, hh], t["q"][b, s, hh], t["v"][b, s, hh]
                bb = t["beta"][b, s, hh]
                Sd = torch.exp(t["g"][b, s, hh])[:, None] * S                       # decay
                S = Sd - bb * torch.outer(kk, kk) @ Sd + bb * torch.outer(kk, vv)   # erase, write
                o = S.T @ qq                                                         # read after
                loss = loss + (o * torch.tensor(Ro[b, s, hh])).sum()
            loss = loss + (S * torch.tensor(Rs[b, hh])).sum()
    loss.backward()
    grad = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs)
    for n in NAMES:
        np.testing.assert_allclose(grad[NAMES[n]], t[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)


def test_no_decay_no_write_closed_form():
    """beta = 0 and g = 0 leave S = S0 throughout, so o_t = S0^T q_t: dq_t = S0 dO_t,
    dS0 = sum_t q_t dO_t^T + dS_T, dv = 0, dk = 0 (catches gradient leaking through a zero write),
    dbeta_t = (S0^T k_t ... ) and dg_t = rowsum(dS_t * S0) (checked against their closed forms)."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=1, T=7, H=1, Dk=4, Dv=3)
    g[:] = 0.0
    beta[:] = 0.0
    Ro, Rs = loss_weights(rng, q, v, S0)
    grad = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs)
    S = S0[0, 0]
    np.testing.assert_allclose(grad["dq"][0, :, 0], Ro[0, :, 0] @ S.T, atol=1e-12)
    np.testing.assert_allclose(grad["dS0"][0, 0], q[0, :, 0].T @ Ro[0, :, 0] + Rs[0, 0], atol=1e-12)
    assert np.abs(grad["dv"]).max() == 0 and np.abs(grad["dk"]).max() == 0
    # dL/dS after token t: dS_T + sum_{s>=t} q_s dO_s^T; beta's gradient: (dS^T k) . (v - S^T k)
    for t_ in range(7):
        dSt = Rs[0, 0] + q[0, t_:, 0].T @ Ro[0, t_:, 0]
        du = dSt.T @ k[0, t_, 0]
        np.testing.assert_allclose(grad["dbeta"][0, t_, 0], du @ (v[0, t_, 0] - S.T @ k[0, t_, 0]), atol=1e-12)
        np.testing.assert_allclose(grad["dg"][0, t_, 0], (dSt * S).sum(1), atol=1e-12)


@pytest.mark.parametrize("C,T", [(1, 13), (16, 45), (32, 70), (32, 32)])
def test_chunkwise_backward_matches_token_backward(C, T):
    """The chunkwise backward (reverse mode through the chunkwise forward, the algorithm the GPU
    backward implements) against the token backward, including ragged last chunks."""
    rng = np.random.default_rng(5 + C)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=T, H=2, Dk=8, Dv=6)
    Ro, Rs = loss_weights(rng, q, v, S0)
    a = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, scale=0.9)
    c = oracle.chunkwise_backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, scale=0.9, C=C)
    for n in a:
        np.testing.assert_allclose(c[n], a[n], rtol=1e-9, atol=1e-10 * np.abs(a[n]).max(), err_msg=n)


def test_backward_blocks_and_threads_do_not_change_the_result():
    """T across several 64-token rebuild blocks, several sequences on several threads: the same bits
    as one thread (catches a block-boundary or per-thread buffer mistake)."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=150, H=3, Dk=8, Dv=8)
    Ro, Rs = loss_weights(rng, q, v, S0)
    a = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, threads=1)
    b = oracle.backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, threads=4)
    c = oracle.chunkwise_backward(q, k, v, g, beta, S0=S0, dO=Ro, dST=Rs, C=16)
    for n in a:
        assert np.array_equal(a[n], b[n]), n
        np.testing.assert_allclose(c[n], a[n], rtol=1e-9, atol=1e-10 * np.abs(a[n]).max(), err_msg=n)
