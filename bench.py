"""Throughput of the KDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload ...]

One step = one kda_fwd call over the training-prefill workload B=4, H=32, T=16384, d_k = d_v = 128
(bf16 q/k/v/o, float32 g/beta/state, chunk 32) with its inputs already resident in HBM.  Prints one
JSON line with the whole-job tokens/s, the roofline position of the kernel (algorithmic bytes per
launch over the average launch time measured with HIP events on the launch stream; median and
minimum beside it, and the fraction of the HBM bandwidth a plain device copy reaches in the same
process) and the float64 CPU oracle's throughput on a bounded sample of the same workload.
--workload f32_small / bf16_4k time the two smaller forward workloads (B1 H2 T256 D64 in float32;
B1 H16 T4096 D128 bf16 with an initial state) the same way, one line each; bf16_4k_cp times the
second through kda_fwd_cp with the automatic segment plan.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s at H=32,d=128,T=16K + % bf16 MFMA peak (1 GPU)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X float32 vector
WORKLOAD = 2
COPY_BYTES = 512 << 20
CSRC = os.path.join(ROOT, "linear_recurrent_attention_amd", "csrc")
# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by the same counters on a
# 512 MiB copy (factors 2.0 and 1.0); valid only for the kernel source with the recorded hash.
MEASURED_TRAFFIC = {
    "core": {"sources": ("kda_fwd_bf16.hip", "kda_common.h"),
             "sha256": "9bbeb734738b0ab09f697de23b40b272d44bf3f233b3068f2ef463322f1d75a3",
             "bytes": (1343653 * 2.0 + 532480 * 1.0) * 1024,
             "profile": "profiles/kda_fwd_bf16_B4_H32_T16384_D128.md"},
    "decode": {"sources": ("kda_decode.hip", "kda_common.h"),
               "sha256": "27169bbf2dad64f9f864da57513ef39a0250b622edfad8163610ea21d502356f",
               "bytes": (135790 * 2.0 + 263168 * 1.0) * 1024,
               "profile": "profiles/kda_decode_bf16_B128_H32_T1_D128.md"},
}


def algorithmic_bytes(B, T, H, Dk, Dv, io_bytes=2, has_S0=False):
    """HBM bytes one launch must move: q, k, v, o (io dtype), g (float32), beta (float32), S_T (+ S0)."""
    per_token_head = (2 * Dk + 2 * Dv) * io_bytes + 4 * Dk + 4
    state = B * H * Dk * Dv * 4 * (2 if has_S0 else 1)
    return B * T * H * per_token_head + state


def algorithmic_flops(B, T, H, Dk, Dv, C=32):
    """Matrix-product flops of the chunkwise form the kernel evaluates, per launch (exact lower
    triangles, no padding, no split-precision repeats).  Per chunk of C tokens and head, in
    multiply-adds: L and A (C(C-1)/2 + C(C+1)/2 dot products of length Dk), (K*Gamma) S, (Q*Gamma) S
    and Kbar^T U (C Dk Dv each), T X and A U (C(C+1)/2 Dv each); 2 flops per multiply-add."""
    tri = C * (C + 1) // 2
    stri = C * (C - 1) // 2
    per_chunk = 2 * ((stri + tri) * Dk + 3 * C * Dk * Dv + 2 * tri * Dv)
    return B * H * (T / C) * per_chunk


def source_digest(names):
    """sha256 over the kernel sources a counter profile was taken on (concatenated in order)."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(which="core"):
    """HBM bytes per launch from the committed counter profile, or None if the kernel changed since."""
    m = MEASURED_TRAFFIC[which]
    return m["bytes"] if m["bytes"] is not None and source_digest(m["sources"]) == m["sha256"] else None


def cpu_baseline(d, threads):
    """float64 oracle over the whole workload (for the headline one, 4 x 32 sequences of 16384 tokens:
    about 1 s of CPU work on 16 threads)."""
    import oracle
    s = {n: np.ascontiguousarray(d[n]) for n in ("q", "k", "v", "g", "beta")}
    t = time.perf_counter()
    oracle.recurrence(s["q"], s["k"], s["v"], s["g"], s["beta"], S0=d.get("S0"), want_o=True, threads=threads)
    dt = time.perf_counter() - t
    B, T = s["q"].shape[:2]
    return {"value": B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload: B={B}, H={s['q'].shape[2]}, T={T} (float64 token recurrence, "
                      f"{dt:.1f} s wall on {threads} threads)"}


def time_steps(torch, step, stream, args):
    """W untimed warmup steps, then K steps between synchronisations, each bracketed by HIP events on
    the launch stream.  Returns (wall seconds for the K steps, per-step event milliseconds)."""
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        stream.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    return wall, [a.elapsed_time(b) for a, b in ev]


def launch_stats(launch_ms):
    """Mean, median and minimum of per-step event times, in milliseconds."""
    a = np.asarray(launch_ms, dtype=np.float64)
    return {"avg_launch_ms": float(a.mean()), "median_launch_ms": float(np.median(a)), "min_launch_ms": float(a.min())}


def copy_gbs(torch, stream, nbytes=COPY_BYTES, reps=10):
    """HBM bandwidth a plain device-to-device copy of nbytes reaches (read + write bytes over the
    median of reps event-timed copies on `stream`): the practical ceiling for a streaming kernel."""
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ms = []
    with torch.cuda.stream(stream):
        dst.copy_(src)
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
            ms.append((a, b))
        stream.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ms])) / 1e3
    del src, dst
    torch.cuda.synchronize()
    return 2 * nbytes / t / 1e9


def hbm_roofline(abytes, stats, copy, kernel, traffic=None):
    """The `roofline` object of an HBM-bound line: algorithmic bytes over the mean launch time against
    the spec peak, with the median/min launch times and the fraction of the measured copy rate."""
    gbs = abytes / (stats["avg_launch_ms"] / 1e3) / 1e9
    out = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
           "traffic": traffic, "kernel": kernel, **stats, "algorithmic_bytes": abytes}
    if copy:
        out["copy_measured_gbs"] = copy
        out["frac_of_copy"] = gbs / copy
        out["frac_of_copy_median"] = abytes / (stats["median_launch_ms"] / 1e3) / 1e9 / copy
    return out


def decode_bytes(B, H, D, T=1, io_bytes=2):
    """HBM bytes of one kda_decode call: the float32 state read and written once, plus q, k, v, o (io
    dtype), g and beta (float32) of each token."""
    return B * H * (2 * D * D * 4 + T * ((4 * D) * io_bytes + 4 * D + 4))


def bench_decode(args, torch, synth, kda):
    """kda_decode on B=128 sequences x H=32 heads, one new token each (D=128, bf16 q/k/v/o), with the
    state updated in place: tokens/s and HBM roofline (state read + write dominates)."""
    w = synth.DECODE
    B, H, D, T = w["B"], w["H"], w["D"], w["T"]
    d, S0 = synth.decode_inputs(seed=0)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v", "g", "beta")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    S = torch.from_numpy(S0).to(dev)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():  # the in-place update of a serving loop (the state keeps evolving across steps)
        kda.kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S, out=o, state_out=S)

    wall, launch_ms = time_steps(torch, step, stream, args)
    avg_s = float(np.mean(launch_ms)) / 1e3
    abytes = decode_bytes(B, H, D, T)
    gbs = abytes / avg_s / 1e9
    out = {
        "metric": "KDA decode tokens/s (B128 H32 D128, one token per sequence, state in place)",
        "value": B * T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w["name"], "B": B, "H": H, "T": T, "D": D,
                   "io": "bf16 q/k/v/o, float32 g/beta/state"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode"), "kernel": "kda_decode_kernel",
                     "avg_launch_ms": avg_s * 1e3, "algorithmic_bytes": abytes},
    }
    if not args.no_cpu:
        import oracle
        threads = len(os.sched_getaffinity(0))
        tc = time.perf_counter()
        oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, threads=threads)
        dt = time.perf_counter() - tc
        out["cpu_baseline"] = {"value": B * T / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"the whole decode workload ({B * H} heads, one token; float64 token "
                                         f"recurrence, {dt:.3f} s wall on {threads} threads)"}
    print(json.dumps(out), flush=True)


def bench_longctx(args, torch, synth, kda):
    """kda_fwd_cp (in-device context parallelism, automatic plan) on the million-token workload
    B=1, H=16, T=2^20, D=128 with S0: tokens/s, and the plain kda_fwd call timed once beside it."""
    w = synth.WORKLOADS[3]
    B, T, H, D, TB = w.B, w.T, w.H, w.Dk, w.block
    A, S0 = synth.gen.head_params(3, 0)
    dev = torch.device("cuda:0")
    t = {n: torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) for n in ("q", "k", "v")}
    t["g"] = torch.empty((B, T, H, D), dtype=torch.float32, device=dev)
    t["beta"] = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    first = None
    for j in range(T // TB):  # generated and uploaded block by block (the host never holds it all)
        blk = synth.core_inputs_block(3, j, seed=0, A=A)
        for n, x in t.items():
            x[:, j * TB:(j + 1) * TB].copy_(torch.from_numpy(blk[n]).to(dev))
        if j == 0:
            first = blk
        print(f"bench.py: longctx inputs, block {j + 1}/{T // TB} on the device", file=sys.stderr, flush=True)
    S0d = torch.from_numpy(S0).to(dev)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    from linear_recurrent_attention_amd import _lib
    desc = _lib.FwdDesc(B, T, H, D, D, 0, _lib.KDA_BF16, _lib.KDA_BF16, 1.0, 0)
    ws = torch.empty(max(1, _lib.cp_workspace_size(desc, 0)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        kda.kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0d, out=o, state_out=ST, workspace=ws)

    wall, launch_ms = time_steps(torch, step, stream, args)

    def plain():
        kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0d, out=o, state_out=ST)

    import types
    _, plain_ms = time_steps(torch, plain, stream, types.SimpleNamespace(steps=1, warmup=1))
    avg_s = float(np.mean(launch_ms)) / 1e3
    abytes = algorithmic_bytes(B, T, H, D, D, has_S0=True)
    gbs = abytes / avg_s / 1e9
    out = {
        "metric": "KDA long-context prefill tokens/s (B1 H16 T1M D128, in-device context parallelism)",
        "value": B * T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "D": D, "segments": "automatic (8)",
                   "io": "bf16 q/k/v/o, float32 g/beta/state"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "kda_fwd_cp (all passes)",
                     "avg_call_ms": avg_s * 1e3, "algorithmic_bytes": abytes},
        "plain_kda_fwd_ms": plain_ms[0],
    }
    if not args.no_cpu:
        import oracle
        threads = len(os.sched_getaffinity(0))
        tc = time.perf_counter()
        oracle.recurrence(first["q"], first["k"], first["v"], first["g"], first["beta"], S0=S0, threads=threads)
        dt = time.perf_counter() - tc
        out["cpu_baseline"] = {"value": B * TB / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"the first {TB}-token block of all {H} heads (float64 token recurrence, "
                                         f"{dt:.1f} s wall on {threads} threads)"}
    print(json.dumps(out), flush=True)


def bwd_bytes(B, T, H, D, io_bytes=2):
    """HBM bytes kda_bwd must move at least: q, k, v, dO (io dtype), g, beta read; dq, dk, dg, dv
    (float32) and dbeta written; the state gradient dS0 (float32)."""
    per_token_head = 4 * D * io_bytes + 4 * D + 4 + 4 * 4 * D + 4
    return B * T * H * per_token_head + B * H * D * D * 4


FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense float32 matrix


def bwd_flops(B, T, H, D, C=16):
    """Matrix-product flops of the chunkwise backward, per launch: per token and head, the products
    with the state, X = V - Kg S, dU = Kb dS, dKb = U dS^T, dQg = dO S^T, dKg = -dX S^T, and the state
    gradient's Qg^T dO and Kg^T dX (7 products of 2 D^2 flops), plus the chunk-sized ones (L, A, U,
    A^T dO, dA, dTm, dX, dM, dL Kh, dA Kh, dL^T Kg, dA^T Qg: 15 of 2 C D flops); the state recompute
    of the forward and the re-stepping inside 32-token intervals are not counted."""
    return B * T * H * (7 * 2 * D * D + 15 * 2 * C * D)


def bench_bwd(args, torch, synth, kda):
    """kda_bwd on the prefill workload B=4, H=32, T=16384, D=128 (bf16 q/k/v/dO, float32 gradients):
    one step = the whole backward (state recompute, reverse state-gradient pass, input gradients)."""
    w = synth.WORKLOADS[WORKLOAD]
    B, T, H, D = w.B, w.T, w.H, w.Dk
    d = synth.core_inputs(WORKLOAD, seed=0)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v", "g", "beta")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(0)
    dO = torch.randn((B, T, H, D), device=dev, generator=gen).to(torch.bfloat16)
    from linear_recurrent_attention_amd import _lib
    desc = _lib.FwdDesc(B, T, H, D, D, 0, _lib.KDA_BF16, _lib.KDA_BF16, 1.0, 0)
    ws = torch.empty(_lib.bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        kda.kda_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], dO=dO, workspace=ws)

    wall, launch_ms = time_steps(torch, step, stream, args)
    avg_s = float(np.mean(launch_ms)) / 1e3
    abytes = bwd_bytes(B, T, H, D)
    gbs = abytes / avg_s / 1e9
    aflops = bwd_flops(B, T, H, D)
    tflops = aflops / avg_s / 1e12
    out = {
        "metric": "KDA backward tokens/s at H=32,d=128,T=16K (1 GPU)", "value": B * T / (wall / args.steps),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "kda_bwd_bf16_B4_H32_T16384_D128", "B": B, "H": H, "T": T, "D": D,
                   "io": "bf16 q/k/v/dO, float32 g/beta and gradients"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP32_MFMA_PEAK_TFLOPS, "traffic": None, "kernel": "kda_bwd (all kernels)",
                     "avg_call_ms": avg_s * 1e3, "algorithmic_flops": aflops},
        "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                "algorithmic_bytes": abytes},
    }
    print(json.dumps(out), flush=True)


def layer_flops(B, T, d, H, D, R):
    """Matrix-product flops of one fused-layer call: the q, k, v, gate and output projections, beta,
    the rank-R decay projection, and the chunkwise core (as algorithmic_flops)."""
    HD = H * D
    per_token = 2 * (4 * d * HD + d * H + d * R + R * HD + HD * d)
    return B * T * per_token + algorithmic_flops(B, T, H, D, D)


def bench_layer(args, torch, synth, kda):
    """kda_layer_fwd on B=2, T=8192, d_model=2048, H=16, D=128, rank 128: tokens/s and matrix-core
    fraction.  Buffers are allocated once; every kernel of the layer is inside each timed call."""
    from linear_recurrent_attention_amd import _lib
    L = synth.gen.LAYER
    B, T, d, H, D, R = L["B"], L["T"], L["d"], L["H"], L["Dk"], L["rank"]
    x, p = synth.layer_inputs(seed=0)
    dev = torch.device("cuda:0")
    bf = ("Wq", "Wk", "Wv", "Wg", "Wo", "Wbeta", "Wdown", "Wup")
    W = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in p.items()}
    for n in bf:
        W[n] = W[n].to(torch.bfloat16)
    xt = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    desc = _lib.LayerDesc(B, T, d, H, D, D, R, 4, 1.0, 0)
    ws = torch.empty(_lib.layer_workspace_size(desc), dtype=torch.uint8, device=dev)
    y = torch.empty((B, T, d), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    cs = torch.empty((B, 3, 2 * H * D), dtype=torch.float32, device=dev)
    Wc = _lib.LayerWeights(*[W[n].data_ptr() for n in _lib.LAYER_WEIGHT_FIELDS])
    stream = torch.cuda.Stream(device=dev)

    def step():
        _lib.check(_lib.layer_fwd_raw(desc, xt.data_ptr(), Wc, 0, 0, y.data_ptr(), ST.data_ptr(), cs.data_ptr(),
                                      ws.data_ptr(), ws.numel(), stream.cuda_stream))

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    stream.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    avg_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    flops = layer_flops(B, T, d, H, D, R)
    tflops = flops / avg_s / 1e12
    out = {
        "metric": "KDA layer forward tokens/s (B2 T8192 d2048 H16 D128)", "value": B * T / (wall / args.steps),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": L["name"], "B": B, "T": T, "d_model": d, "H": H, "D": D, "rank": R, "conv": 4},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None, "kernel": "kda_layer_fwd (all kernels)",
                     "avg_call_ms": avg_s * 1e3, "algorithmic_flops": flops},
    }
    print(json.dumps(out), flush=True)


def bench_core(args, torch, synth, kda, wid, cp=False):
    """kda_fwd on forward workload wid (2: the headline B4 H32 T16384 D128 bf16 line; 0: B1 H2 T256 D64
    float32; 1: B1 H16 T4096 D128 bf16 with an initial state).  cp: kda_fwd_cp with the automatic
    segment plan instead (32 workgroups of workload 1 leave most of the chip idle; the plan cuts each
    sequence into segments that run side by side)."""
    w = synth.WORKLOADS[wid]
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    d = synth.core_inputs(wid, seed=0)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(d[n]).to(dev) for n in ("q", "k", "v", "g", "beta")}
    bf16 = w.io == "bf16"
    io_dt = torch.bfloat16 if bf16 else torch.float32
    for n in ("q", "k", "v"):
        t[n] = t[n].to(io_dt)
    S0 = None if d["S0"] is None else torch.from_numpy(d["S0"]).to(dev)
    o = torch.empty((B, T, H, Dv), dtype=io_dt, device=dev)
    ST = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)

    if cp:
        from linear_recurrent_attention_amd import _lib
        desc = _lib.FwdDesc(B, T, H, Dk, Dv, 0, _lib.KDA_BF16, _lib.KDA_BF16, 1.0, 0)
        nws = _lib.cp_workspace_size(desc, 0)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

        def step():
            kda.kda_fwd_cp(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0, nseg=0, out=o, state_out=ST,
                           workspace=ws)
    else:
        def step():
            kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0, out=o, state_out=ST)

    wall, launch_ms = time_steps(torch, step, stream, args)
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stats = launch_stats(launch_ms)
    copy = None if args.calibrate_copy else copy_gbs(torch, stream)
    avg_launch_s = stats["avg_launch_ms"] / 1e3
    ms_per_step = wall / args.steps * 1e3

    tokens = B * T
    value = tokens / (wall / args.steps)
    abytes = algorithmic_bytes(B, T, H, Dk, Dv, io_bytes=2 if bf16 else 4, has_S0=S0 is not None)
    aflops = algorithmic_flops(B, T, H, Dk, Dv, C=32 if bf16 else 16)
    achieved_tflops = aflops / avg_launch_s / 1e12
    kernel = ("kda_fwd_cp (all passes)" if cp else "kda_fwd_bf16_kernel") if bf16 else "kda_fwd_f32_kernel"
    mm_peak = BF16_PEAK_TFLOPS if bf16 else FP32_VALU_PEAK_TFLOPS

    out = {
        "metric": METRIC if wid == WORKLOAD and not cp else
                  f"KDA prefill tokens/s ({w.name}{', kda_fwd_cp automatic plan' if cp else ''})", "value": value,
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": w.name + ("_cp" if cp else ""), "B": B, "H": H, "T": T, "Dk": Dk, "Dv": Dv,
                   "chunk": 32 if bf16 else 16,
                   "io": ("bf16 q/k/v/o" if bf16 else "float32 q/k/v/o") + ", float32 g/beta/state"
                         + (", S0 given" if S0 is not None else "")},
        "roofline": hbm_roofline(abytes, stats, copy, kernel,
                                 measured_traffic() if wid == WORKLOAD and not cp else None),
        ("mfma" if bf16 else "valu"): {"achieved": achieved_tflops, "peak": mm_peak, "unit": "TFLOP/s",
                                       "frac": achieved_tflops / mm_peak, "algorithmic_flops": aflops},
    }
    if not args.no_cpu:
        try:
            threads = len(os.sched_getaffinity(0))
        except AttributeError:
            threads = os.cpu_count() or 1
        out["cpu_baseline"] = cpu_baseline(d, threads)
    print(json.dumps(out), flush=True)


def bench_layer_decode(args, torch, synth, kda):
    """kda_layer_decode: one new token for each of B=16 sequences through the layer of the prefill
    workload (d_model 2048, H=16, D=128, rank 128), state and window updated in place.  Bound by reading
    the weights (about 43 MB of bf16) and reading and writing the float32 state once per call; the
    projections are bf16 matrix-core products with float32 sums, the recurrence float32."""
    L = synth.gen.LAYER
    B, T, d, H, D, R = 16, 1, L["d"], L["H"], L["Dk"], L["rank"]
    x, p = synth.layer_inputs(seed=0, B=B, T=T)
    dev = torch.device("cuda:0")
    bf = ("Wq", "Wk", "Wv", "Wg", "Wo", "Wbeta", "Wdown", "Wup")
    W = {n: torch.from_numpy(np.ascontiguousarray(a)).to(dev) for n, a in p.items()}
    for n in bf:
        W[n] = W[n].to(torch.bfloat16)
    xt = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(0)
    S = torch.randn((B, H, D, D), device=dev, generator=gen) * 0.3
    cs = torch.randn((B, 3, 2 * H * D), device=dev, generator=gen)
    from linear_recurrent_attention_amd import _lib
    ws = torch.empty(_lib.layer_decode_workspace_size(_lib.LayerDesc(B, T, d, H, D, D, R, 4, 1.0, 0)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        kda.kda_layer_decode(xt, W, S, cs, workspace=ws)

    wall, launch_ms = time_steps(torch, step, stream, args)
    stats = launch_stats(launch_ms)
    wbytes = 2 * (d * (4 * H * D + R + H) + R * H * D + H * D * d)
    abytes = wbytes + B * H * D * D * 4 * 2 + B * T * d * 2 * 2
    out = {
        "metric": "KDA layer decode tokens/s (B16 one token each, d2048 H16 D128, state in place)",
        "value": B * T / (wall / args.steps), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "kda_layer_decode_bf16_B16_T1_d2048_H16_D128", "B": B, "T": T, "d_model": d, "H": H,
                   "D": D, "rank": R},
        "roofline": hbm_roofline(abytes, stats, None, "kda_layer_decode (all four kernels)"),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--workload", choices=("core", "f32_small", "bf16_4k", "bf16_4k_cp", "layer", "decode", "longctx",
                                           "bwd", "layer_decode"),
                    default="core",
                    help="core: kda_fwd on B4 H32 T16384 (the headline line); layer: kda_layer_fwd on "
                         "B2 T8192 d_model 2048 H16; decode: kda_decode on B128 H32, one token; longctx: "
                         "kda_fwd_cp on B1 H16 T1M; bwd: kda_bwd on B4 H32 T16384; f32_small: kda_fwd on "
                         "B1 H2 T256 D64 float32; bf16_4k: kda_fwd on B1 H16 T4096 (bf16_4k_cp: the same "
                         "through kda_fwd_cp, automatic plan); layer_decode: kda_layer_decode "
                         "on B16 one token each (separate lines)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU; --gpus N with N > 1 is not supported "
              "(heads are independent, so N GPUs would each take a share of B*H)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import linear_recurrent_attention_amd as kda

    if args.workload == "layer":
        bench_layer(args, torch, synth, kda)
        return
    if args.workload == "decode":
        bench_decode(args, torch, synth, kda)
        return
    if args.workload == "layer_decode":
        bench_layer_decode(args, torch, synth, kda)
        return
    if args.workload == "longctx":
        bench_longctx(args, torch, synth, kda)
        return
    if args.workload == "bwd":
        bench_bwd(args, torch, synth, kda)
        return
    if args.workload == "f32_small":
        bench_core(args, torch, synth, kda, 0)
        return
    if args.workload == "bf16_4k":
        bench_core(args, torch, synth, kda, 1)
        return
    if args.workload == "bf16_4k_cp":
        bench_core(args, torch, synth, kda, 1, cp=True)
        return
    bench_core(args, torch, synth, kda, WORKLOAD)


if __name__ == "__main__":
    main()
