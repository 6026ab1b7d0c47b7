"""GPU: state checkpoints of kda_fwd_ckpt (the resume points of a KDA prefix cache) against the
float64 oracle run over each prefix, and resuming from a checkpoint against the uninterrupted call."""
import numpy as np
import pytest
import torch

import oracle
from _metrics import TOL_BF16, TOL_F32, rel_max
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


def run_ckpt(d, io, every, S0=None, precise=False):
    t = to_dev(d, io)
    S0t = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(DEV)
    o, ST, ck = _kda().kda_fwd_ckpt(t["q"], t["k"], t["v"], t["g"], t["beta"], every, S0=S0t, precise=precise)
    torch.cuda.synchronize()
    return t, o, ST, ck


def prefix(d, T):
    return {n: np.ascontiguousarray(d[n][:, :T]) for n in ("q", "k", "v", "g", "beta")}


CASES = [  # (io, B, T, H, D, every, precise)
    ("bf16", 2, 1100, 2, 128, 256, False),   # ragged end: 4 checkpoints, the last chunk is partial
    ("bf16", 1, 1024, 3, 128, 512, True),    # the page's 512-token spacing; last checkpoint at T
    ("f32", 2, 200, 2, 64, 48, False),       # 16-token chunks
]


@pytest.mark.parametrize("io,B,T,H,D,every,precise", CASES)
def test_checkpoints_are_the_prefix_states(io, B, T, H, D, every, precise):
    d, S0 = rand_small(11, B, T, H, D=D, io=io)
    _, _, ST, ck = run_ckpt(d, io, every, S0=S0, precise=precise)
    n = T // every
    assert tuple(ck.shape) == (B, H, n, D, D)
    tol = TOL_F32 if io == "f32" else TOL_BF16
    for m in range(n):
        p = prefix(d, (m + 1) * every)
        _, S_ref = oracle.recurrence(p["q"], p["k"], p["v"], p["g"], p["beta"], S0=S0, want_o=False)
        assert rel_max(ck[:, :, m].cpu().numpy(), S_ref) <= tol, m
    if T % every == 0:
        assert torch.equal(ck[:, :, n - 1], ST)  # the last boundary is the end of the sequence


@pytest.mark.parametrize("io,B,T,H,D,every,precise", CASES)
def test_resume_from_checkpoint_is_bitwise(io, B, T, H, D, every, precise):
    """Resuming at a checkpoint with kda_fwd reproduces the rest of o and S_T exactly."""
    d, S0 = rand_small(12, B, T, H, D=D, io=io)
    t, o, ST, ck = run_ckpt(d, io, every, S0=S0, precise=precise)
    for m in range(T // every):
        t0 = (m + 1) * every
        if t0 >= T:
            continue
        rest = {n: t[n][:, t0:].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o2, ST2 = _kda().kda_fwd(rest["q"], rest["k"], rest["v"], rest["g"], rest["beta"],
                                 S0=ck[:, :, m].contiguous(), precise=precise)
        torch.cuda.synchronize()
        assert torch.equal(o2, o[:, t0:]), m
        assert torch.equal(ST2, ST), m


def test_no_checkpoint_in_range_leaves_outputs_as_kda_fwd():
    """every > T: no checkpoint, and o / S_T equal those of kda_fwd bit for bit."""
    d, S0 = rand_small(13, 1, 100, 2)
    t, o, ST, ck = run_ckpt(d, "bf16", 128, S0=S0)
    assert ck.shape[2] == 0
    S0t = torch.from_numpy(S0).to(DEV)
    o1, ST1 = _kda().kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(ST, ST1)
