"""GPU parity of kda_fwd_cp (in-device context parallelism over segments of long sequences) against
the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from _metrics import TOL_BF16, rel_max, rel_max_bf16_out
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


@pytest.mark.parametrize("B,H,T,nseg,s0,precise", [
    (1, 4, 8192 + 37, 4, True, False),    # ragged: three segments of 2048 tokens, the last one 2085
    (2, 2, 4096, 4, True, False),         # T = 4 x 1024: both sequences' segments in one launch
    (2, 3, 3000, 2, False, True),         # ragged with two sequences, precise plan (1472 + 1528 tokens)
    (2, 16, 8192, 3, False, True),        # three segments (2720, 2720, 2752 tokens), first pass merged
    (1, 2, 70000, 0, True, False),        # automatic plan: 31 segments (30 of 2240 tokens, then 2800)
    (1, 16, 4096, 0, True, False),        # the B1 H16 T4096 forward workload's shape, automatic plan
])
def test_cp_matches_oracle(B, H, T, nseg, s0, precise):
    d, S0 = rand_small(31, B, T, H, s0=s0)
    t = to_dev(d, "bf16")
    S0t = None if S0 is None else torch.from_numpy(S0).to(DEV)
    o, ST = _kda().kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, nseg=nseg, precise=precise)
    o32, _ = _kda().kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, nseg=nseg, precise=precise,
                               o_dtype=torch.float32, want_state=False)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    assert rel_max_bf16_out(o.float().cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_max(o32.cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_max(ST.cpu().numpy(), S_ref) <= TOL_BF16


def test_cp_state_in_place_and_one_segment():
    """S_T may be S0; nseg = 1 is kda_fwd itself (bit for bit)."""
    d, S0 = rand_small(32, 1, 5000, 2)
    t = to_dev(d, "bf16")
    S = torch.from_numpy(S0).to(DEV)
    o, _ = _kda().kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S, nseg=4, state_out=S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    assert rel_max_bf16_out(o.float().cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_max(S.cpu().numpy(), S_ref) <= TOL_BF16
    S0t = torch.from_numpy(S0).to(DEV)
    o1, S1 = _kda().kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, nseg=1)
    o2, S2 = _kda().kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("gscale", [2e-3, 0.0])
def test_cp_state_carries_across_segments(gscale):
    """Slow or no decay (g in [-gscale, 0]) and small beta, so the state of one segment still shapes
    the outputs of the next ones: the scanned initial states are what is checked here.  The same
    inputs with each segment started from zero instead differ from the oracle by far more."""
    B, H, T, nseg = 1, 2, 4096, 4
    d, S0 = rand_small(33, B, T, H)
    rng = np.random.default_rng(34)
    d["g"] = (-gscale * rng.uniform(0, 1, d["g"].shape)).astype(np.float32)
    d["beta"] = (0.05 * rng.uniform(0, 1, d["beta"].shape)).astype(np.float32)
    t = to_dev(d, "bf16")
    S0t = torch.from_numpy(S0).to(DEV)
    o, ST = _kda().kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, nseg=nseg, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    o = o.cpu().numpy()
    assert rel_max(o, o_ref) <= TOL_BF16
    assert rel_max(ST.cpu().numpy(), S_ref) <= TOL_BF16
    # the check has teeth: the last segment run from a zero state is far off
    Ls = T // nseg
    tail = {n: np.ascontiguousarray(d[n][:, T - Ls:]) for n in ("q", "k", "v", "g", "beta")}
    o_cut, _ = oracle.recurrence(tail["q"], tail["k"], tail["v"], tail["g"], tail["beta"])
    assert rel_max(o_cut, o_ref[:, T - Ls:]) > 20 * TOL_BF16
