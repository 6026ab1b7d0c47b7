"""GPU parity of the fused KDA layer (kda_layer_fwd through the C ABI) against the float64 layer oracle."""
import numpy as np
import pytest
import torch

import synth
from _metrics import TOL_BF16, rel_max, rel_max_bf16_out
from oracle import layer as L

pytestmark = pytest.mark.gpu
DEV = "cuda"

BF16_W = ("Wq", "Wk", "Wv", "Wg", "Wo", "Wbeta", "Wdown", "Wup")


def to_dev(x, p):
    xt = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    W = {}
    for n, a in p.items():
        t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
        W[n] = t.to(torch.bfloat16) if n in BF16_W else t.float()
    return xt, W


def run(x, p, S0=None, cs=None):
    import linear_recurrent_attention_amd as kda
    xt, W = to_dev(x, p)
    S0t = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, np.float32)).to(DEV)
    cst = None if cs is None else torch.from_numpy(np.ascontiguousarray(cs, np.float32)).to(DEV)
    y, ST, cso = kda.kda_layer_fwd(xt, W, S0=S0t, conv_state=cst)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), ST.cpu().numpy(), cso.cpu().numpy()


def small(seed, B=2, T=70, d=256, H=2, R=32):
    x, p = synth.layer_inputs(seed=seed, B=B, T=T, d=d, H=H, D=128, rank=R)
    rng = np.random.default_rng(seed)
    p["A"] = rng.uniform(-1, 1, H).astype(np.float32)          # exercise the per-head scale
    p["b_alpha"] = (rng.standard_normal(H * 128) * 0.5).astype(np.float32)
    p["rms_w"] = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    return x, p


def test_layer_small_ragged():
    """Two batches, 70 tokens (ragged last chunk), nonzero A, b_alpha and RMSNorm weight."""
    x, p = small(1)
    y_ref, S_ref, cs_ref = L.forward(x, p)
    y, ST, cs = run(x, p)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)


def test_layer_state_and_window_carry():
    """A second segment started from the first segment's state and conv window matches the oracle's
    continuation (which pins the window semantics on the CPU)."""
    x, p = small(2, T=96)
    rng = np.random.default_rng(5)
    S0 = (rng.standard_normal((2, 2, 128, 128)) * 0.3).astype(np.float32)
    cs0 = rng.standard_normal((2, 3, 2 * 256)).astype(np.float32)
    y_ref, S_ref, cs_ref = L.forward(x, p, S0=S0, conv_state=cs0)
    y, ST, cs = run(x, p, S0=S0, cs=cs0)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)


def test_layer_short_sequence_window():
    """T = 2 < 3: the outgoing window mixes the incoming window and the new rows."""
    x, p = small(3, B=1, T=2)
    cs0 = np.random.default_rng(6).standard_normal((1, 3, 2 * 256)).astype(np.float32)
    y_ref, S_ref, cs_ref = L.forward(x, p, conv_state=cs0)
    y, ST, cs = run(x, p, cs=cs0)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)


def test_layer_workload4_full():
    """B=2, T=8192, d_model=2048, H=16, D=128, rank 128, weights N(0, 1/fan_in): full size."""
    x, p = synth.layer_inputs(seed=0)
    y, ST, _ = run(x, p)
    y_ref, S_ref, _ = L.forward(x, p)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16


def test_layer_long_ragged_with_state_and_window():
    """T = 1100 (35 chunks, the last one ragged; 35 prologue blocks), with S0 and an incoming
    convolution window."""
    x, p = small(7, B=2, T=1100)
    rng = np.random.default_rng(8)
    S0 = (rng.standard_normal((2, 2, 128, 128)) * 0.3).astype(np.float32)
    cs0 = rng.standard_normal((2, 3, 2 * 256)).astype(np.float32)
    y_ref, S_ref, cs_ref = L.forward(x, p, S0=S0, conv_state=cs0)
    y, ST, cs = run(x, p, S0=S0, cs=cs0)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("B,T,H", [
    (2, 512, 3),   # two 256-row tiles per sequence; three heads: one tile holds q head 2 and k head 0
    (1, 256, 2),   # every tile starts a sequence
])
def test_layer_fused_qk_epilogue(B, T, H):
    """T a multiple of 256: the short convolution, SiLU and L2 of q and k run in the input projection's
    epilogue, and the rows at tile edges are finished from the raw rows kept beside it (with the
    incoming window at a sequence start)."""
    x, p = small(11, B=B, T=T, H=H)
    rng = np.random.default_rng(12)
    S0 = (rng.standard_normal((B, H, 128, 128)) * 0.3).astype(np.float32)
    cs0 = rng.standard_normal((B, 3, 2 * H * 128)).astype(np.float32)
    y_ref, S_ref, cs_ref = L.forward(x, p, S0=S0, conv_state=cs0)
    y, ST, cs = run(x, p, S0=S0, cs=cs0)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)


def test_layer_gemm_tail_pieces_partial_rows():
    """B=2, T=4100, d=256, H=4: the input projection has 33 x 9 = 297 tiles, so its last 41 run as
    64-row pieces, and the last row tile holds 8 rows (T is not a multiple of 256: prologue path)."""
    x, p = small(13, B=2, T=4100, d=256, H=4, R=32)
    rng = np.random.default_rng(14)
    cs0 = rng.standard_normal((2, 3, 2 * 4 * 128)).astype(np.float32)
    y_ref, S_ref, cs_ref = L.forward(x, p, conv_state=cs0)
    y, ST, cs = run(x, p, cs=cs0)
    assert rel_max_bf16_out(y, y_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    np.testing.assert_allclose(cs, cs_ref, rtol=1e-5, atol=1e-5)
