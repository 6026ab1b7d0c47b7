"""GPU parity of kda_bwd (gradients of the forward) against the float64 backward oracle."""
import numpy as np
import pytest
import torch

import oracle
from _metrics import TOL_BF16, TOL_F32, rel_max
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


def run(io, B, T, H, D, seed, s0=True, with_dO=True, with_dST=True, scale=1.0, gscale=1.0):
    d, S0 = rand_small(seed, B, T, H, D=D, io=io, s0=s0)
    d["g"] = (d["g"] * gscale).astype(np.float32)
    rng = np.random.default_rng(seed + 100)
    dO = rng.standard_normal((B, T, H, D)).astype(np.float32) if with_dO else None
    if dO is not None and io == "bf16":
        import synth
        dO = synth.bf16_round(dO)
    dST = rng.standard_normal((B, H, D, D)).astype(np.float32) if with_dST else None
    t = to_dev(d, io)
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dOt = None if dO is None else torch.from_numpy(dO).to(DEV).to(dt)
    dSTt = None if dST is None else torch.from_numpy(dST).to(DEV)
    S0t = None if S0 is None else torch.from_numpy(S0).to(DEV)
    gr = _kda().kda_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], dO=dOt, dS_T=dSTt, S0=S0t, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, dO=dO, dST=dST, scale=scale)
    return {n: gr[n].cpu().numpy() for n in GRADS}, ref


def errors(got, ref):
    """max|err| / rms(ref) per gradient; a gradient that is exactly zero (e.g. dq without dO) must
    come out exactly zero."""
    out = {}
    for n in GRADS:
        if not np.any(ref[n]):
            assert not np.any(got[n]), n
            out[n] = 0.0
        else:
            out[n] = rel_max(got[n], ref[n])
    return out


@pytest.mark.parametrize("D,T", [(64, 70), (128, 33), (64, 16), (128, 5)])
def test_bwd_f32_matches_oracle(D, T):
    """float32 inputs (16-token intervals): every gradient within 1e-4 of the float64 backward."""
    got, ref = run("f32", 2, T, 2, D, seed=41, scale=0.8)
    e = errors(got, ref)
    assert max(e.values()) <= TOL_F32, e


@pytest.mark.parametrize("T", [200, 64, 31])
def test_bwd_bf16_matches_oracle(T):
    """bf16 q/k/v/dO (32-token intervals, states from the matrix-core forward): every gradient within
    1e-2 of the float64 backward on the same rounded inputs."""
    got, ref = run("bf16", 1, T, 3, 128, seed=42)
    e = errors(got, ref)
    assert max(e.values()) <= TOL_BF16, e


@pytest.mark.parametrize("with_dO,with_dST,s0", [(True, False, False), (False, True, True)])
def test_bwd_partial_output_gradients(with_dO, with_dST, s0):
    """Only dO, or only dS_T (then dq is exactly zero).  Slower decay (g scaled by 0.2) keeps the
    state gradient that reaches S0 from dS_T well above float32 rounding of its larger early terms."""
    got, ref = run("f32", 1, 50, 2, 64, seed=43, s0=s0, with_dO=with_dO, with_dST=with_dST, gscale=0.2)
    e = errors(got, ref)
    assert max(e.values()) <= TOL_F32, e


def test_bwd_bf16_long_sequence():
    """B1 H4 T4096 (128 intervals): the state gradient carried through the whole sequence."""
    got, ref = run("bf16", 1, 4096, 4, 128, seed=44)
    e = errors(got, ref)
    assert max(e.values()) <= TOL_BF16, e


@pytest.mark.timeout(600)
def test_bwd_workload2_full_launch_sampled_heads():
    """The benchmark's backward: B4 H32 T16384 D128, bf16 q/k/v/dO, one kda_bwd over all 128
    sequences; the float64 backward recomputes 3 sampled (b, h) sequences, every gradient within 1e-2
    of it."""
    import synth
    d = synth.core_inputs(2, seed=0)
    B, T, H, D = d["k"].shape
    rng = np.random.default_rng(7)
    dO = synth.bf16_round(rng.standard_normal((B, T, H, D)).astype(np.float32))
    t = to_dev(d, "bf16")
    gr = _kda().kda_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"],
                        dO=torch.from_numpy(dO).to(DEV).to(torch.bfloat16))
    torch.cuda.synchronize()
    picks = [(0, 0), (3, 31), (int(rng.integers(B)), int(rng.integers(H)))]
    for b, h in picks:
        s = {n: d[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v", "g", "beta")}
        ref = oracle.backward(s["q"], s["k"], s["v"], s["g"], s["beta"], dO=dO[b:b + 1, :, h:h + 1])
        got = {n: (gr[n][b:b + 1, h:h + 1] if n == "dS0" else gr[n][b:b + 1, :, h:h + 1]).cpu().numpy()
               for n in GRADS}
        e = errors(got, ref)
        print(f"(b, h) = ({b}, {h}):", {n: f"{v:.2e}" for n, v in e.items()}, flush=True)
        assert max(e.values()) <= TOL_BF16, (b, h, e)


def test_bwd_unaligned_outputs_take_the_zeroing_kernel():
    """Output gradients at addresses that are not 16-byte aligned (4 bytes past an allocation) make
    the state pass leave the zeroing to a kernel of its own; the gradients are bitwise those of the
    aligned call (two addends per element onto zero, so their order does not matter)."""
    import linear_recurrent_attention_amd as kda
    from linear_recurrent_attention_amd import _lib
    B, T, H, D = 1, 200, 3, 128
    d, S0 = rand_small(45, B, T, H, D=D, io="bf16", s0=True)
    rng = np.random.default_rng(145)
    import synth
    dO = torch.from_numpy(synth.bf16_round(rng.standard_normal((B, T, H, D)).astype(np.float32))).to(DEV).to(torch.bfloat16)
    t = to_dev(d, "bf16")
    S0t = torch.from_numpy(S0).to(DEV)
    ref = kda.kda_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], dO=dO, S0=S0t)
    shapes = {"dq": (B, T, H, D), "dk": (B, T, H, D), "dv": (B, T, H, D), "dg": (B, T, H, D), "dbeta": (B, T, H),
              "dS0": (B, H, D, D)}
    bufs = {n: torch.full((int(np.prod(s)) + 1,), np.nan, dtype=torch.float32, device=DEV) for n, s in shapes.items()}
    desc, _, _ = kda._fwd_args(t["q"], t["k"], t["v"], t["g"], t["beta"], S0t, torch.bfloat16, False, t["q"], None, 0,
                               False, 1.0)
    ws = torch.empty(_lib.bwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    code = _lib.bwd_raw(desc, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                        t["beta"].data_ptr(), S0t.data_ptr(), dO.data_ptr(), 0,
                        *[bufs[n].data_ptr() + 4 for n in GRADS], ws.data_ptr(), ws.numel(),
                        torch.cuda.current_stream().cuda_stream)
    _lib.check(code)
    torch.cuda.synchronize()
    for n in GRADS:
        got = bufs[n][1:].view(shapes[n])
        assert torch.equal(got, ref[n]), n
