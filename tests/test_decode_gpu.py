"""GPU parity of kda_decode (token-by-token step) against the float64 oracle, plus its agreement with
the chunkwise forward when decoding continues a prefill."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _metrics import TOL_BF16, TOL_F32, rel_max, rel_max_bf16_out
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


def dev_state(S0):
    return None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(DEV)


@pytest.mark.parametrize("io,D,B,T,H", [("bf16", 128, 3, 1, 5), ("bf16", 64, 2, 3, 4), ("f32", 64, 2, 7, 3),
                                        ("f32", 128, 1, 2, 6)])
def test_decode_matches_oracle(io, D, B, T, H):
    d, S0 = rand_small(21, B, T, H, D=D, io=io)
    t = to_dev(d, io)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, scale=0.75)
    # float32 output: the arithmetic is float32 on exactly widened inputs
    o32, ST = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=dev_state(S0), scale=0.75,
                                o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert rel_max(o32.cpu().numpy(), o_ref) <= TOL_F32
    assert rel_max(ST.cpu().numpy(), S_ref) <= TOL_F32
    if io == "bf16":
        o16, _ = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=dev_state(S0), scale=0.75)
        torch.cuda.synchronize()
        assert o16.dtype == torch.bfloat16
        assert rel_max_bf16_out(o16.float().cpu().numpy(), o_ref) <= TOL_BF16


def test_decode_in_place_equals_out_of_place():
    d, S0 = rand_small(22, 2, 1, 4)
    t = to_dev(d, "bf16")
    o1, S1 = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=dev_state(S0))
    S = dev_state(S0)
    o2, S2 = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S, state_out=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S)


def test_zero_initial_state_and_empty_call():
    d, _ = rand_small(23, 1, 2, 2, s0=False)
    t = to_dev(d, "bf16")
    o, ST = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert rel_max(o.cpu().numpy(), o_ref) <= TOL_F32 and rel_max(ST.cpu().numpy(), S_ref) <= TOL_F32
    # T = 0: the state passes through
    e = {n: x[:, :0].contiguous() for n, x in t.items()}
    S0 = torch.randn(1, 2, 128, 128, device=DEV)
    _, S1 = _kda().kda_decode(e["q"], e["k"], e["v"], e["g"], e["beta"], S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S1, S0)


def test_prefill_then_decode_continues_the_sequence():
    """kda_fwd over a 300-token prompt, then 20 single-token kda_decode steps in place: o and the
    final state match the oracle over all 320 tokens."""
    B, H, T0, T1 = 2, 3, 300, 20
    d, S0 = rand_small(24, B, T0 + T1, H)
    t = to_dev(d, "bf16")
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    o_pre, S = _kda().kda_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], S0=dev_state(S0),
                              o_dtype=torch.float32)
    outs = []
    for i in range(T0, T0 + T1):
        step = {n: x[:, i:i + 1].contiguous() for n, x in t.items()}
        o, _ = _kda().kda_decode(step["q"], step["k"], step["v"], step["g"], step["beta"], S0=S, state_out=S,
                                 o_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    assert rel_max(o_pre.cpu().numpy(), o_ref[:, :T0]) <= TOL_BF16
    assert rel_max(torch.cat(outs, 1).cpu().numpy(), o_ref[:, T0:]) <= TOL_BF16
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_BF16


def test_decode_workload_sampled_heads():
    """The decode workload (B=128 sequences, H=32, D=128, one token, bf16 I/O, a nonzero incoming
    state): the full launch, checked on sampled (batch, head) pairs against the oracle."""
    B, H, D = 128, 32, 128
    d, S0 = synth.decode_inputs(seed=0, B=B, H=H, D=D)
    t = to_dev(d, "bf16")
    o, ST = _kda().kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=dev_state(S0), o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, ST = o.cpu().numpy(), ST.cpu().numpy()
    rng = np.random.default_rng(5)
    for b, h in zip(rng.integers(0, B, 6), rng.integers(0, H, 6)):
        sl = {n: np.ascontiguousarray(d[n][b:b + 1, :, h:h + 1]) for n in ("q", "k", "v", "g", "beta")}
        o_ref, S_ref = oracle.recurrence(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                         S0=S0[b:b + 1, h:h + 1])
        assert rel_max(o[b:b + 1, :, h:h + 1], o_ref) <= TOL_F32
        assert rel_max(ST[b:b + 1, h:h + 1], S_ref) <= TOL_F32
