"""GPU parity of the million-token segment: B1 H16 T=1,048,576 D128, bf16 q/k/v/o, S0 in, S_T out.

The inputs are streamed block by block (64K tokens) to the device and, in the same order, through the
float64 oracle, which carries the state across blocks in float64.  One kda_fwd call then runs the whole
segment; o is compared on a seeded 64K-token window and S_T after the last token.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from _metrics import TOL_BF16, rel_max, rel_max_bf16_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.timeout(900)
def test_workload3_million_tokens_window_and_final_state():
    import linear_recurrent_attention_amd as kda
    w = synth.WORKLOADS[3]
    B, T, H, D, TB = w.B, w.T, w.H, w.Dk, w.block
    W = 1 << 16
    ws = synth.window_start(T, W, seed=0)
    A, S0 = synth.gen.head_params(3, 0)
    log(f"workload 3: T={T} H={H} window [{ws}, {ws + W})")

    dev = {n: torch.empty((B, T, H, D), dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    dev["g"] = torch.empty((B, T, H, D), dtype=torch.float32, device=DEV)
    dev["beta"] = torch.empty((B, T, H), dtype=torch.float32, device=DEV)
    S = S0.astype(np.float64)
    o_win = np.empty((B, W, H, D))
    t_start = time.time()
    for j in range(T // TB):
        t0 = j * TB
        blk = synth.core_inputs_block(3, j, seed=0, A=A)
        for n, t in dev.items():
            t[:, t0:t0 + TB].copy_(torch.from_numpy(blk[n]).to(DEV))
        lo, hi = max(t0, ws), min(t0 + TB, ws + W)
        o, S = oracle.recurrence(blk["q"], blk["k"], blk["v"], blk["g"], blk["beta"], S0=S, want_o=lo < hi)
        if lo < hi:
            o_win[:, lo - ws:hi - ws] = o[:, lo - t0:hi - t0]
        del blk, o
        log(f"  block {j}: generated, uploaded, oracle carried ({time.time() - t_start:.1f} s)")

    S0d = torch.from_numpy(S0).to(DEV)
    # the plain kernel (2*H = 32 workgroups) and the in-device context-parallel path (automatic plan:
    # 8 segments, 256 workgroups per pass) on the same device inputs, each with a bf16 output (checked
    # net of the bf16 output rounding) and a float32 output (checked literally)
    f32 = torch.float32
    runs = (
        ("kda_fwd", False, lambda: kda.kda_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S0=S0d)),
        ("kda_fwd_cp", False, lambda: kda.kda_fwd_cp(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S0=S0d)),
        ("kda_fwd f32 o", True,
         lambda: kda.kda_fwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S0=S0d, o_dtype=f32)),
        ("kda_fwd_cp f32 o", True,
         lambda: kda.kda_fwd_cp(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], S0=S0d, o_dtype=f32)),
    )
    for name, literal, run in runs:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        o_gpu, ST = run()
        b.record()
        torch.cuda.synchronize()
        o_w = o_gpu[:, ws:ws + W].float().cpu().numpy()
        del o_gpu
        ST = ST.cpu().numpy()
        e_o = rel_max(o_w, o_win) if literal else rel_max_bf16_out(o_w, o_win)
        e_s = rel_max(ST, S)
        log(f"  {name}: {a.elapsed_time(b):.1f} ms, o window {e_o:.4g}  S_T {e_s:.4g}")
        assert e_o <= TOL_BF16
        assert e_s <= TOL_BF16
        del o_w
