"""kda_fwd_cp_noalloc (the allocation-free context-parallel forward, through the C ABI) against
kda_fwd_cp with a caller workspace, on consecutive calls that share the library's static scratch
array, each smaller than the one before; and the first against the float64 oracle."""
import pytest
import torch

import oracle
from _metrics import TOL_BF16, rel_max, rel_max_bf16_out
from test_parity_gpu import rand_small, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(t, S0, nseg):
    from linear_recurrent_attention_amd import _lib
    B, T, H, D = t["q"].shape
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=DEV)
    ST = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    desc = _lib.FwdDesc(B, T, H, D, D, 0, _lib.KDA_BF16, _lib.KDA_BF16, 1.0, 0)
    stream = torch.cuda.current_stream().cuda_stream
    code = _lib.fwd_cp_noalloc_raw(desc, t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["g"].data_ptr(),
                                   t["beta"].data_ptr(), 0 if S0 is None else S0.data_ptr(), o.data_ptr(),
                                   ST.data_ptr(), nseg, stream)
    _lib.check(code)
    return o, ST


# (B, H, T, nseg, S0): 24 MiB of segment states (16 heads x 8 segments, ragged tail), then 3 MiB
# (a ragged 37-token tail), then 3 MiB over two sequences with no initial state
CALLS = [(1, 16, 16384 + 37, 8, True), (1, 4, 8192 + 37, 4, True), (2, 2, 4096, 4, False)]


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    from linear_recurrent_attention_amd import _lib, kda_fwd_cp
    ref = None
    for i, (B, H, T, nseg, s0) in enumerate(CALLS):
        print(f"kda_fwd_cp_noalloc call {i}: B={B} H={H} T={T} nseg={nseg} S0={s0}", flush=True)
        d, S0 = rand_small(71 + i, B, T, H, s0=s0)
        desc = _lib.FwdDesc(B, T, H, 128, 128, 0, _lib.KDA_BF16, _lib.KDA_BF16, 1.0, 0)
        need = _lib.cp_workspace_size(desc, nseg)
        assert 0 < need <= _lib.KDA_CP_NOALLOC_SCRATCH_BYTES
        t = to_dev(d, "bf16")
        S0t = None if S0 is None else torch.from_numpy(S0).to(DEV)
        o, ST = _noalloc(t, S0t, nseg)
        o_ws, ST_ws = kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, nseg=nseg)
        torch.cuda.synchronize()
        # the same kernels on the same plan: bit for bit
        assert torch.equal(o, o_ws)
        assert torch.equal(ST, ST_ws)
        if i == 1:
            ref = (d, S0, o, ST)
    d, S0, o, ST = ref
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    assert rel_max_bf16_out(o.float().cpu().numpy(), o_ref) <= TOL_BF16
    assert rel_max(ST.cpu().numpy(), S_ref) <= TOL_BF16
