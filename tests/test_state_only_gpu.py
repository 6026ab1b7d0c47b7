"""GPU: the state-only forward (o = NULL on the bf16 path: the kernel instantiation that skips the
readout) gives the same final state and checkpoints as the full forward, bit for bit, and the
oracle's state."""
import numpy as np
import pytest
import torch

import oracle
from _metrics import TOL_BF16, rel_max
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


@pytest.mark.parametrize("B,T,H,precise,with_S0", [(2, 1000, 3, False, True), (1, 64, 4, True, False),
                                                   (3, 17, 2, False, True)])
def test_state_only_matches_full_forward(B, T, H, precise, with_S0):
    d, S0 = rand_small(21, B, T, H, D=128, io="bf16")
    if not with_S0:
        S0 = None
    t = to_dev(d, "bf16")
    S0t = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(DEV)
    kda = _kda()
    o_full, S_full = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, precise=precise)
    o_none, S_only = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, precise=precise,
                                 want_output=False)
    torch.cuda.synchronize()
    assert o_none is None and o_full is not None
    assert torch.equal(S_only, S_full)
    _, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, want_o=False)
    assert rel_max(S_only.cpu().numpy(), S_ref) <= TOL_BF16


def test_state_only_checkpoints_match_full_call():
    """Filling a prefix cache: checkpoints and S_T without the outputs, bit for bit those of the call
    with outputs."""
    d, S0 = rand_small(22, 2, 1100, 2, D=128, io="bf16")
    t = to_dev(d, "bf16")
    S0t = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(DEV)
    kda = _kda()
    _, S_full, ck_full = kda.kda_fwd_ckpt(t["q"], t["k"], t["v"], t["g"], t["beta"], 256, S0=S0t)
    o, S_only, ck_only = kda.kda_fwd_ckpt(t["q"], t["k"], t["v"], t["g"], t["beta"], 256, S0=S0t,
                                          want_output=False)
    torch.cuda.synchronize()
    assert o is None
    assert torch.equal(ck_only, ck_full)
    assert torch.equal(S_only, S_full)
