"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the mistake it would catch.  Sources: the recurrence and its
parts as described on the explainer page "Kimi K3：开放前沿智能" (sections 2.2-2.5,
3.2, 3.3); the rest is mathematics (closed forms, invariants, textbook
reductions, hand-worked examples under tests/golden/).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import layer as L

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B=1, T=20, H=2, Dk=6, Dv=5, unit_k=True, s0=True, gmin=-5.0):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = gmin * rng.uniform(0, 1, (B, T, H, Dk))
    beta = rng.uniform(0, 1, (B, T, H))
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


# -- the C recurrence against a hand-worked example and the explicit matrix form ---------------------

def test_hand_worked_example():
    """Two tokens worked in exact fractions: catches order of decay/erase/write and read-before-update."""
    ex = json.load(open(os.path.join(GOLD, "kda_hand_example_D2_T2.json")))
    tok = ex["tokens"]
    q = np.array([[t["q"] for t in tok]], np.float64)[:, :, None, :]
    k = np.array([[t["k"] for t in tok]], np.float64)[:, :, None, :]
    v = np.array([[t["v"] for t in tok]], np.float64)[:, :, None, :]
    g = np.log(np.array([[t["alpha"] for t in tok]], np.float64))[:, :, None, :]
    beta = np.array([[t["beta"] for t in tok]], np.float64)[:, :, None]
    S0 = np.array(ex["S0"], np.float64)[None, None]
    for fn in (oracle.recurrence, oracle.recurrence_np, oracle.chunkwise):
        o, ST = fn(q, k, v, g, beta, S0=S0)
        np.testing.assert_allclose(o[0, :, 0], ex["o"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ST[0, 0], ex["S_T"], rtol=0, atol=1e-13)


def test_c_recurrence_matches_matrix_form():
    """C rank-1 updates vs explicit (I - b k k^T) Diag(a) S + b k v^T with dense matrices; Dk != Dv."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=17, H=3, Dk=7, Dv=4, unit_k=False)
    o1, S1 = oracle.recurrence(q, k, v, g, beta, S0=S0, scale=0.7)
    o2, S2 = oracle.recurrence_np(q, k, v, g, beta, S0=S0, scale=0.7)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-12)


def test_float32_inputs_are_upcast_exactly():
    rng = np.random.default_rng(2)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=9)
    args32 = [a.astype(np.float32) for a in (q, k, v, g, beta)]
    o1, S1 = oracle.recurrence(*args32, S0=S0)
    o2, S2 = oracle.recurrence(*[a.astype(np.float64) for a in args32], S0=S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


# -- chunkwise form: an independent algorithm --------------------------------------------------------

@pytest.mark.parametrize("C", [1, 2, 4, 16, 64])
def test_chunkwise_matches_recurrence(C):
    """Chunk algebra (cumsum, Gram, triangular inverse, inter/intra split, state hand-off) vs the recurrence.
    T = 150 leaves a ragged last chunk for C in {4, 16, 64}; g reaches the -5 bound."""
    rng = np.random.default_rng(10 + C)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=150, H=2, Dk=8, Dv=6)
    o1, S1 = oracle.recurrence(q, k, v, g, beta, S0=S0, scale=0.5)
    o2, S2 = oracle.chunkwise(q, k, v, g, beta, S0=S0, scale=0.5, C=C)
    np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(S2, S1, rtol=1e-9, atol=1e-10)


def test_chunkwise_d128_hard_decay():
    """Full head width, decay pinned at the -5 bound for half of the channels (largest 1/Gamma)."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=130, H=1, Dk=128, Dv=128)
    g[..., ::2] = -5.0
    o1, S1 = oracle.recurrence(q, k, v, g, beta, S0=S0)
    o2, S2 = oracle.chunkwise(q, k, v, g, beta, S0=S0, C=64)
    np.testing.assert_allclose(o2, o1, rtol=1e-8, atol=1e-9)
    np.testing.assert_allclose(S2, S1, rtol=1e-8, atol=1e-9)


# -- closed forms ---------------------------------------------------------------------------------------

def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(alpha_t) S_{t-1}, so S_T = Diag(exp(sum g)) S0 and o_t = S0^T (exp(b_t) * q_t).
    Catches a wrong decay direction (rows vs columns) or a wrong cumulative index."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=12, Dk=5, Dv=3)
    beta[:] = 0
    o, ST = oracle.recurrence(q, k, v, g, beta, S0=S0)
    b = np.cumsum(g, axis=1)
    want_o = np.einsum("bhij,bthi->bthj", S0, np.exp(b) * q)
    want_S = np.exp(b[:, -1])[..., None] * S0
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST, want_S, rtol=1e-12, atol=1e-13)


def test_unit_key_full_write_reads_back_value():
    """beta = 1 and |k| = 1 give S_t^T k_t = v_t for ANY decay, because (I - k k^T) k = 0.
    With q = k the readout must therefore return v exactly.  Catches decay-after-erase and read-before-write."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=25, Dk=6, Dv=4)
    beta[:] = 1.0
    o, _ = oracle.recurrence(k, k, v, g, beta, S0=S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)


def test_one_step_identity_general_beta():
    """S_t^T k_t = (1 - b|k|^2) S_{t-1}^T (alpha*k) + b|k|^2 v_t for any beta and key length."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=8, Dk=5, Dv=3, unit_k=False)
    t = 7
    _, Sprev = oracle.recurrence(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0=S0)
    o, _ = oracle.recurrence(k[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1], beta[:, t:t + 1],
                             S0=Sprev)
    kk = np.sum(k[:, t] ** 2, axis=-1)  # [B,H]
    bk = beta[:, t] * kk
    ak = np.exp(g[:, t]) * k[:, t]
    want = (1 - bk)[..., None] * np.einsum("bhij,bhi->bhj", Sprev, ak) + bk[..., None] * v[:, t]
    np.testing.assert_allclose(o[:, 0], want, rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    """T = 1: o = S0^T (alpha*q) + beta (q.k) (v - S0^T(alpha*k)); S_1 = Diag(alpha) S0 + beta k (v - S0^T(alpha*k))^T.
    (With S0 != 0 the second half of o is needed; a form without it would be off.)"""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, S0 = rand_inputs(rng, B=2, T=1, H=3, Dk=6, Dv=4, unit_k=False)
    o, ST = oracle.recurrence(q, k, v, g, beta, S0=S0)
    a = np.exp(g[:, 0])
    r = v[:, 0] - np.einsum("bhij,bhi->bhj", S0, a * k[:, 0])
    qk = np.sum(q[:, 0] * k[:, 0], axis=-1)
    want_o = np.einsum("bhij,bhi->bhj", S0, a * q[:, 0]) + (beta[:, 0] * qk)[..., None] * r
    want_S = a[..., None] * S0 + beta[:, 0][..., None, None] * k[:, 0][..., :, None] * r[..., None, :]
    np.testing.assert_allclose(o[:, 0], want_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ST, want_S, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_reduce_to_causal_linear_attention():
    """alpha = 1, beta = 1, S0 = 0 and orthonormal keys: the erase term never fires, o = tril(Q K^T) V."""
    rng = np.random.default_rng(8)
    T, D, Dv = 10, 12, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = Qm[:, :T].T[None, :, None, :]
    q = rng.standard_normal((1, T, 1, D))
    v = rng.standard_normal((1, T, 1, Dv))
    g = np.zeros((1, T, 1, D))
    beta = np.ones((1, T, 1))
    o, _ = oracle.recurrence(q, k, v, g, beta)
    want = np.tril(q[0, :, 0] @ k[0, :, 0].T) @ v[0, :, 0]
    np.testing.assert_allclose(o[0, :, 0], want, rtol=1e-12, atol=1e-12)
    o2, _ = oracle.chunkwise(q, k, v, g, beta, C=4)
    np.testing.assert_allclose(o2[0, :, 0], want, rtol=1e-12, atol=1e-12)


def test_ungated_delta_rule_textbook_step():
    """alpha = 1: one step is the plain delta rule S <- S + beta k (v - S^T k)^T (Widrow-Hoff on a linear map)."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=1, Dk=4, Dv=3, unit_k=False)
    g[:] = 0
    _, ST = oracle.recurrence(q, k, v, g, beta, S0=S0)
    pred = np.einsum("bhij,bhi->bhj", S0, k[:, 0])
    want = S0 + beta[:, 0][..., None, None] * k[:, 0][..., :, None] * (v[:, 0] - pred)[..., None, :]
    np.testing.assert_allclose(ST, want, rtol=1e-12, atol=1e-13)


# -- invariants --------------------------------------------------------------------------------------------

def test_linear_in_values_and_state():
    """(o, S_T) is jointly linear in (V, S0) for fixed (k, beta, g).  Catches any term not proportional to V or S0."""
    rng = np.random.default_rng(11)
    q, k, v1, g, beta, S01 = rand_inputs(rng, T=30)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    a, b = 0.7, -1.3
    o1, T1 = oracle.recurrence(q, k, v1, g, beta, S0=S01)
    o2, T2 = oracle.recurrence(q, k, v2, g, beta, S0=S02)
    o3, T3 = oracle.recurrence(q, k, a * v1 + b * v2, g, beta, S0=a * S01 + b * S02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(T3, a * T1 + b * T2, rtol=1e-11, atol=1e-12)


def test_state_map_is_product_of_transitions():
    """S_T(S0) - S_T(0) = M S0 with M = prod_t (I - beta_t k_t k_t^T) Diag(alpha_t), newest factor on the left."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=15, H=1, Dk=5, Dv=3)
    _, Sa = oracle.recurrence(q, k, v, g, beta, S0=S0)
    _, Sb = oracle.recurrence(q, k, v, g, beta, S0=None)
    M = np.eye(5)
    for t in range(15):
        kt = k[0, t, 0][:, None]
        M = (np.eye(5) - beta[0, t, 0] * kt @ kt.T) @ np.diag(np.exp(g[0, t, 0])) @ M
    np.testing.assert_allclose(Sa[0, 0] - Sb[0, 0], M @ S0[0, 0], rtol=1e-11, atol=1e-12)


def test_segment_split_is_exact():
    """Running [0, T1) then [T1, T) from the carried state equals one pass (bitwise in the token recurrence,
    to rounding in the chunkwise form with a split off the chunk grid)."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=40)
    o, ST = oracle.recurrence(q, k, v, g, beta, S0=S0)
    t1 = 23
    oa, Sa = oracle.recurrence(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], S0=S0)
    ob, Sb = oracle.recurrence(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], S0=Sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o) and np.array_equal(Sb, ST)
    oc, Sc = oracle.chunkwise(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], S0=Sa, C=8)
    np.testing.assert_allclose(oc, ob, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(Sc, ST, rtol=1e-10, atol=1e-11)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = rand_inputs(rng, T=0)
    o, ST = oracle.recurrence(q, k, v, g, beta, S0=S0)
    assert o.shape[1] == 0 and np.array_equal(ST, S0)
    _, ST0 = oracle.recurrence(q, k, v, g, beta, S0=None)
    assert not ST0.any()


# -- gate map and layer pieces ---------------------------------------------------------------------------

def test_decay_gate_hand_values():
    ex = json.load(open(os.path.join(GOLD, "decay_gate_hand_values.json")))
    for c in ex["cases"]:
        got = oracle.decay_gate(np.array([[c["z"]]]), np.array([c["A"]]))
        np.testing.assert_allclose(got[0, 0], c["g"], rtol=1e-14)


def test_decay_gate_bounds():
    """log alpha stays inside the open interval (-5, 0): alpha in (e^-5, 1)."""
    z = np.linspace(-8, 8, 1001)[:, None, None].repeat(3, 1)
    g = oracle.decay_gate(z, np.array([-1.0, 0.0, 1.0]))
    assert np.all(g < 0) and np.all(g > -5)
    assert np.all(np.diff(g, axis=0) <= 0)  # larger logit => faster decay


def test_short_conv_matches_numpy_convolve():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((2, 11, 3))
    w = rng.standard_normal((3, 4))
    st = rng.standard_normal((2, 3, 3))
    y, ns = L.short_conv(x, w, st)
    for b in range(2):
        for c in range(3):
            xp = np.concatenate([st[b, :, c], x[b, :, c]])
            np.testing.assert_allclose(y[b, :, c], np.convolve(xp, w[c, ::-1], mode="valid"), rtol=1e-13)
    np.testing.assert_array_equal(ns, x[:, -3:, :])


def test_norms_and_activation_closed_forms():
    np.testing.assert_allclose(L.l2norm(np.array([3.0, 4.0]), eps=0), [0.6, 0.8], rtol=1e-15)
    np.testing.assert_allclose(L.rmsnorm(np.array([2.0, -2.0, 2.0, -2.0]), np.array([1.0, 2.0, 3.0, 4.0]), eps=0),
                               [1.0, -2.0, 3.0, -4.0], rtol=1e-15)
    np.testing.assert_allclose(L.silu(np.array([0.0, np.log(3.0)])), [0.0, np.log(3.0) * 0.75], rtol=1e-15)


def _small_layer(seed=0, T=24):
    import synth
    return synth.layer_inputs(seed=seed, B=2, T=T, d=32, H=2, D=16, rank=8)


def test_layer_is_causal():
    """Changing a future token leaves earlier outputs and nothing else unchanged."""
    x, p = _small_layer()
    y1, _, _ = L.forward(x, p)
    x2 = x.copy()
    x2[:, 15] += 1.0
    y2, _, _ = L.forward(x2, p)
    np.testing.assert_array_equal(y1[:, :15], y2[:, :15])
    assert np.abs(y1[:, 15:] - y2[:, 15:]).max() > 1e-3


def test_layer_segment_carry():
    """Two segments with (S, conv window) carried equal one pass: pins the conv state and S0/S_T plumbing."""
    x, p = _small_layer(T=30)
    y, ST, cs = L.forward(x, p)
    ya, Sa, ca = L.forward(x[:, :13], p)
    yb, Sb, cb = L.forward(x[:, 13:], p, S0=Sa, conv_state=ca)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sb, ST, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(cb, cs)


def test_layer_rmsnorm_removes_value_scale():
    """Scaling W_v by c > 0 scales o by c (linearity with S0 = 0); the head RMSNorm removes it (eps = 0)."""
    x, p = _small_layer()
    y1, _, _ = L.forward(x, p, eps=0.0)
    p2 = dict(p)
    p2["Wv"] = p["Wv"] * 8.0
    y2, _, _ = L.forward(x, p2, eps=0.0)
    np.testing.assert_allclose(y2, y1, rtol=1e-10, atol=1e-12)


def test_layer_zero_gate_weight_halves():
    """W_g = 0 gives gate sigmoid(0) = 1/2, so y = rmsnorm(o) @ W_o / 2: doubling W_o with W_g = 0 doubles y."""
    x, p = _small_layer()
    p0 = dict(p)
    p0["Wg"] = np.zeros_like(p["Wg"])
    y0, _, _ = L.forward(x, p0)
    _, _, _, parts = L.forward(x, p0, return_parts=True)
    o = parts["o"]
    on = o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + L.EPS)
    want = 0.5 * on.reshape(2, 24, -1) @ p["Wo"].astype(np.float64)
    np.testing.assert_allclose(y0, want, rtol=1e-12, atol=1e-12)


# -- the layer's composition against a hand-worked example ------------------------------------------------

def _hand_layer():
    ex = json.load(open(os.path.join(GOLD, "kda_layer_hand_example.json")))
    inp = {n: np.array(a, np.float64) for n, a in ex["inputs"].items()}
    x = inp.pop("x")[None]
    return ex, x, inp


def test_layer_hand_worked_example():
    """oracle.layer.forward against a T=4, H=2 layer worked element by element at 40 digits: pins the order
    conv -> SiLU -> per-head L2, z = W_up W_down x + b_alpha -> -5 sigmoid(e^A z), beta = sigmoid(x W_beta),
    and RMSNorm * sigmoid(x W_g) @ W_o (sections 2.3, 2.4, 3.2, 3.3 of the explainer page)."""
    ex, x, p = _hand_layer()
    y, ST, _, parts = L.forward(x, p, return_parts=True)
    w = ex["working"]
    np.testing.assert_allclose(parts["q"][0].reshape(4, -1), w["q"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(parts["k"][0].reshape(4, -1), w["k"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(parts["g"][0].reshape(4, -1), w["g"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(parts["beta"][0], w["beta"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(parts["o"][0].reshape(4, -1), w["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[0], ex["y"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(ST[0], ex["S_T"], rtol=0, atol=1e-13)


def _planted(monkeypatch, mistake):
    """Run the layer oracle with one plausible mistake planted in it (on the CPU) and return y."""
    ex, x, p = _hand_layer()
    if mistake == "silu_after_l2":
        real_l2 = L.l2norm
        monkeypatch.setattr(L, "silu", lambda u: u)
        monkeypatch.setattr(L, "l2norm", lambda u, eps=L.EPS: (lambda n: n * L.sigmoid(n))(real_l2(u, eps)))
    elif mistake == "l2_over_all_heads":
        real_l2 = L.l2norm
        monkeypatch.setattr(L, "l2norm", lambda u, eps=L.EPS: real_l2(u.reshape(*u.shape[:-2], -1), eps).reshape(u.shape))
    elif mistake == "bias_outside_gate_scale":  # -5 sigmoid(e^A (W_up W_down x) + b) instead of e^A (... + b)
        b = p["b_alpha"].reshape(2, 2)
        p = dict(p, b_alpha=np.zeros_like(p["b_alpha"]))
        monkeypatch.setattr(L, "decay_gate", lambda z, A: -5.0 / (1.0 + np.exp(-(np.exp(A)[:, None] * z + b))))
    elif mistake == "beta_without_sigmoid":
        real_sig = L.sigmoid
        calls = []
        def sig(u):  # the first sigmoid forward() takes is beta's
            calls.append(1)
            return u if len(calls) == 1 else real_sig(u)
        monkeypatch.setattr(L, "sigmoid", sig)
    elif mistake == "gate_before_rmsnorm":
        real_rms = L.rmsnorm
        monkeypatch.setattr(L, "rmsnorm", lambda u, w, eps=L.EPS: u * w)
    y, _, _ = L.forward(x, p)
    return ex, y


@pytest.mark.parametrize("mistake", ["silu_after_l2", "l2_over_all_heads", "bias_outside_gate_scale",
                                     "beta_without_sigmoid", "gate_before_rmsnorm"])
def test_layer_hand_example_rejects_planted_mistakes(monkeypatch, mistake):
    """Each plausible misreading of the layer, planted in the oracle, moves y off the hand-worked values."""
    ex, y = _planted(monkeypatch, mistake)
    assert np.abs(y[0] - np.array(ex["y"])).max() > 1e-3
