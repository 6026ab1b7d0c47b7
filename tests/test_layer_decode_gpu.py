"""GPU parity of the layer decode step with its projection-input cache (kda_layer_decode and
kda_layer_decode_commit through the C ABI) against the float64 layer oracle run over the accepted
tokens: plain decode steps, and speculative drafts rolled back to an accepted prefix."""
import numpy as np
import pytest
import torch

import synth
from _metrics import TOL_BF16, rel_max, rel_max_bf16_out
from oracle import layer as L

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_W = ("Wq", "Wk", "Wv", "Wg", "Wo", "Wbeta", "Wdown", "Wup")
TOL_F32 = 1e-4  # state and window: float32 arithmetic on exact inputs


def setup(seed, B=2, T=4, d=256, H=2, R=32):
    x, p = synth.layer_inputs(seed=seed, B=B, T=T, d=d, H=H, D=128, rank=R)
    rng = np.random.default_rng(seed)
    p["A"] = rng.uniform(-1, 1, H).astype(np.float32)
    p["b_alpha"] = (rng.standard_normal(H * 128) * 0.5).astype(np.float32)
    p["rms_w"] = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    S0 = (rng.standard_normal((B, H, 128, 128)) * 0.3).astype(np.float32)
    cs0 = rng.standard_normal((B, 3, 2 * H * 128)).astype(np.float32)
    W = {}
    for n, a in p.items():
        t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        W[n] = t.to(torch.bfloat16) if n in BF16_W else t.float()
    return x, p, W, S0, cs0


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def decode(x, W, S, cs, speculative=False):
    import linear_recurrent_attention_amd as kda
    y, cache = kda.kda_layer_decode(torch.from_numpy(x).to(DEV).to(torch.bfloat16), W, S, cs, speculative=speculative)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), cache


@pytest.mark.parametrize("B,T", [(1, 1), (2, 3), (4, 4)])
def test_decode_steps_match_oracle(B, T):
    """Plain decode (state and window updated in place) over B*T rows, 1 to 16."""
    x, p, W, S0, cs0 = setup(10 + T, B=B, T=T)
    y_ref, S_ref, cs_ref = L.forward(x, p, S0=S0, conv_state=cs0)
    S, cs = dev(S0), dev(cs0)
    y, _ = decode(x, W, S, cs)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_F32
    np.testing.assert_allclose(cs.cpu().numpy(), cs_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("B,T,d,H,R", [(4, 4, 260, 3, 20), (16, 1, 2048, 16, 128)])
def test_decode_projection_shapes(B, T, d, H, R):
    """Projection shapes: d_model and rank not multiples of 8 and three heads (element-wise weight and x
    loads, partial column blocks, a 4-column last block of the output projection); and 16 sequences of
    one token at d_model 2048, 16 heads, rank 128."""
    x, p, W, S0, cs0 = setup(50 + d, B=B, T=T, d=d, H=H, R=R)
    y_ref, S_ref, cs_ref = L.forward(x, p, S0=S0, conv_state=cs0)
    S, cs = dev(S0), dev(cs0)
    y, _ = decode(x, W, S, cs)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_F32
    np.testing.assert_allclose(cs.cpu().numpy(), cs_ref, rtol=1e-5, atol=1e-5)


def test_speculative_drafts_and_rollback():
    """Four drafts per sequence checked speculatively (state and window untouched, each draft's output as if
    the earlier drafts were accepted); two accepted from the cache; then one more token decoded from there."""
    import linear_recurrent_attention_amd as kda
    B, T, acc = 2, 4, 2
    x, p, W, S0, cs0 = setup(21, B=B, T=T)
    S, cs = dev(S0), dev(cs0)
    y, cache = decode(x, W, S, cs, speculative=True)
    assert torch.equal(S, dev(S0)) and torch.equal(cs, dev(cs0))           # nothing committed
    y_all, _, _ = L.forward(x, p, S0=S0, conv_state=cs0)
    assert rel_max_bf16_out(y, y_all) <= TOL_BF16
    kda.kda_layer_decode_commit(cache, acc, S, cs, W, B, T, x.shape[2])
    torch.cuda.synchronize()
    _, S_ref, cs_ref = L.forward(x[:, :acc], p, S0=S0, conv_state=cs0)
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_F32
    np.testing.assert_allclose(cs.cpu().numpy(), cs_ref, rtol=1e-5, atol=1e-5)
    # the next token continues from the accepted prefix, not from the rejected drafts
    xn, _ = synth.layer_inputs(seed=22, B=B, T=1, d=x.shape[2], H=2, D=128, rank=32)
    yn, _ = decode(xn, W, S, cs)
    y_seq, S_seq, cs_seq = L.forward(np.concatenate([x[:, :acc], xn], axis=1), p, S0=S0, conv_state=cs0)
    assert rel_max_bf16_out(yn, y_seq[:, acc:]) <= TOL_BF16
    assert rel_max(S.cpu().numpy(), S_seq) <= TOL_F32
    np.testing.assert_allclose(cs.cpu().numpy(), cs_seq, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("acc", [0, 1, 4])
def test_commit_counts(acc):
    """Accepting none leaves state and window as they were; accepting one moves the window by one row
    (the window keeps two rows of the old one); accepting all equals the plain decode of the drafts."""
    import linear_recurrent_attention_amd as kda
    B, T = 2, 4
    x, p, W, S0, cs0 = setup(31 + acc, B=B, T=T)
    S, cs = dev(S0), dev(cs0)
    _, cache = decode(x, W, S, cs, speculative=True)
    kda.kda_layer_decode_commit(cache, acc, S, cs, W, B, T, x.shape[2])
    torch.cuda.synchronize()
    if acc == 0:
        assert torch.equal(S, dev(S0)) and torch.equal(cs, dev(cs0))
        return
    _, S_ref, cs_ref = L.forward(x[:, :acc], p, S0=S0, conv_state=cs0)
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_F32
    np.testing.assert_allclose(cs.cpu().numpy(), cs_ref, rtol=1e-5, atol=1e-5)


def test_cache_entries_are_the_projection_outputs():
    """The cache holds each token's k, v, g, beta and pre-convolution q, k rows: compared with the oracle's
    intermediate values for the same tokens."""
    B, T, H = 2, 3, 2
    x, p, W, S0, cs0 = setup(41, B=B, T=T)
    S, cs = dev(S0), dev(cs0)
    _, cache = decode(x, W, S, cs, speculative=True)
    c = cache.cpu().numpy().astype(np.float64)
    N, HD = B * T, H * 128
    k, v, g = c[:N * HD].reshape(B, T, H, 128), c[N * HD:2 * N * HD].reshape(B, T, H, 128), c[2 * N * HD:3 * N * HD]
    beta = c[3 * N * HD:3 * N * HD + N * H].reshape(B, T, H)
    qpre = c[3 * N * HD + N * H:4 * N * HD + N * H].reshape(B, T, HD)
    _, _, _, parts = L.forward(x, p, S0=S0, conv_state=cs0, return_parts=True)
    xw = x.astype(np.float64).reshape(B * T, -1)
    assert rel_max(k, parts["k"]) <= TOL_F32
    assert rel_max(v, parts["v"]) <= TOL_F32
    assert rel_max(g.reshape(B, T, H, 128), parts["g"]) <= TOL_F32
    assert rel_max(beta, parts["beta"]) <= TOL_F32
    assert rel_max(qpre, (xw @ p["Wq"].astype(np.float64)).reshape(B, T, HD)) <= TOL_F32
