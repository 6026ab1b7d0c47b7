"""GPU parity: libkda.so (through the C ABI) against the float64 CPU oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from _metrics import TOL_BF16, TOL_F32, rel_max, rel_max_bf16_out

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _kda():
    import linear_recurrent_attention_amd as kda
    return kda


def to_dev(d, io):
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    t = {n: torch.from_numpy(np.ascontiguousarray(d[n])).to(DEV) for n in ("q", "k", "v", "g", "beta")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(dt)
    return t


def gpu_fwd(d, io, S0=None, o_dtype=None, scale=1.0, precise=False):
    t = to_dev(d, io)
    S0t = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(DEV)
    o, ST = _kda().kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, scale=scale, o_dtype=o_dtype,
                           precise=precise)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), ST.cpu().numpy()


def sub(d, b=None, h=None, T=None):
    out = {}
    for n in ("q", "k", "v", "g", "beta"):
        a = d[n]
        if b is not None:
            a = a[b]
        if T is not None:
            a = a[:, :T]
        if h is not None:
            a = a[:, :, h]
        out[n] = np.ascontiguousarray(a)
    return out


def rand_small(seed, B, T, H, D=128, io="bf16", s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    rnd = synth.bf16_round if io == "bf16" else (lambda x: x.astype(np.float32))
    d = dict(q=rnd(q), k=rnd(k), v=rnd(rng.standard_normal((B, T, H, D))),
             g=(-5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, D)) * 1.5))).astype(np.float32),
             beta=(1 / (1 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32))
    S0 = (rng.standard_normal((B, H, D, D)) * 0.3).astype(np.float32) if s0 else None
    return d, S0


# ---- the workloads ------------------------------------------------------------------------------------

def test_workload0_f32():
    """B1 H2 T256 D64, float32 end to end: max|err|/rms <= 1e-4 on o and S_T."""
    d = synth.core_inputs(0, seed=0)
    o, ST = gpu_fwd(d, "f32")
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    assert rel_max(o, o_ref) <= TOL_F32
    assert rel_max(ST, S_ref) <= TOL_F32


def test_workload1_bf16():
    """B1 H16 T4096 D128 with S0: bf16 o (format allowance), float32 o (literal), S_T (literal)."""
    d = synth.core_inputs(1, seed=0)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    o, ST = gpu_fwd(d, "bf16", S0=d["S0"])
    assert rel_max_bf16_out(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    o32, ST32 = gpu_fwd(d, "bf16", S0=d["S0"], o_dtype=torch.float32)
    assert rel_max(o32, o_ref) <= TOL_BF16
    assert np.array_equal(ST32, ST)


def test_workload2_full_launch_all_heads():
    """B4 H32 T16384 D128 in the benchmark's launch; the oracle recomputes all 128 (b, h) sequences.
    The delivered bf16 o with the format allowance, the float32-output run literally, S_T literally."""
    d = synth.core_inputs(2, seed=0)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"])
    o, ST = gpu_fwd(d, "bf16")
    e_o, e_s = rel_max_bf16_out(o, o_ref), rel_max(ST, S_ref)
    del o
    o32, ST32 = gpu_fwd(d, "bf16", o_dtype=torch.float32)
    e_o32 = rel_max(o32, o_ref)
    print(f"workload 2: o(bf16, allowance) {e_o:.3g}  o(f32) {e_o32:.3g}  S_T {e_s:.3g}")
    assert e_o <= TOL_BF16 and e_o32 <= TOL_BF16 and e_s <= TOL_BF16
    assert np.array_equal(ST32, ST)


@pytest.mark.parametrize("precise", [False, True])
@pytest.mark.parametrize("scale", [2.0 ** -18, 2.0 ** 8])
def test_value_and_state_scale_invariance(scale, precise):
    """(o, S_T) is linear in (v, S0): with both scaled by 2^-18 or 2^8 the relative error must stay at the
    unit-scale level.  B1 H4 T2048 with workload-1 statistics; o_dtype float32 (literal) and bf16."""
    d, S0 = rand_small(21, 1, 2048, 4)
    d["v"] = (d["v"].astype(np.float64) * scale).astype(np.float32)  # exact: a power of two
    S0 = (S0.astype(np.float64) * scale).astype(np.float32)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    o32, ST = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32, precise=precise)
    ob, _ = gpu_fwd(d, "bf16", S0=S0, precise=precise)
    print(f"scale {scale:g} precise {precise}: o32 {rel_max(o32, o_ref):.3g} "
          f"o_bf16 {rel_max_bf16_out(ob, o_ref):.3g} S_T {rel_max(ST, S_ref):.3g}")
    assert rel_max(o32, o_ref) <= TOL_BF16
    assert rel_max_bf16_out(ob, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16


def test_validate_mode_accepts_clean_inputs_and_rejects_bad_ones():
    """KDA_VALIDATE: clean inputs give the plain call's result bit for bit; g below the -5 bound, g above 0,
    or a non-finite v, beta or S0 make kda_fwd return KDA_ERR_INVALID_ARG without computing."""
    kda = _kda()
    d, S0 = rand_small(22, 2, 100, 3)
    t = to_dev(d, "bf16")
    S0t = torch.from_numpy(S0).to(DEV)
    o1, S1 = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t)
    o2, S2 = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0t, validate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # the edges of the bound are accepted
    g = t["g"].clone()
    g[0, 0, 0, 0] = -5.0
    g[1, 99, 2, 127] = 0.0
    kda.kda_fwd(t["q"], t["k"], t["v"], g, t["beta"], S0=S0t, validate=True)
    bad = []
    for name, val, where in (("g", -5.001, (1, 50, 1, 7)), ("g", 1e-3, (0, 99, 2, 0)), ("g", float("nan"), (0, 3, 0, 3)),
                             ("v", float("inf"), (1, 7, 0, 1)), ("beta", float("nan"), (0, 10, 1)),
                             ("q", float("nan"), (1, 99, 2, 127))):
        a = {n: t[n].clone() for n in ("q", "k", "v", "g", "beta")}
        a[name][where] = val
        try:
            kda.kda_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], S0=S0t, validate=True)
        except kda.KdaError as e:
            bad.append(e.code)
        else:
            bad.append(None)
    S0n = S0t.clone()
    S0n[1, 2, 3, 4] = float("inf")
    try:
        kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S0n, validate=True)
    except kda.KdaError as e:
        bad.append(e.code)
    assert bad == [-1] * 7, bad


def correlated_keys(seed, B, T, H, D=128, cos=0.5):
    """bf16 inputs whose keys share one random direction per head (pairwise cosine about `cos`), as
    the layer's Swish-activated, convolved keys do; g and beta as in the workloads."""
    rng = np.random.default_rng(seed)
    d, _ = rand_small(seed, B, T, H, D, s0=False)
    u = rng.standard_normal((H, D))
    u *= np.sqrt(D * cos / (1 - cos)) / np.linalg.norm(u, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, D)) + u[None, None]
    d["k"] = synth.bf16_round(k / np.linalg.norm(k, axis=-1, keepdims=True))
    return d


def test_precise_flag_correlated_keys():
    """KDA_FWD_PRECISE on keys with pairwise cosine 0.5 (B1 H4 T2048, S0 in): o and S_T within 1e-2.
    The default plan's errors are printed for reference."""
    d = correlated_keys(11, 1, 2048, 4)
    S0 = (np.random.default_rng(12).standard_normal((1, 4, 128, 128)) * 0.3).astype(np.float32)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    o, ST = gpu_fwd(d, "bf16", S0=S0, precise=True)
    o_d, ST_d = gpu_fwd(d, "bf16", S0=S0)
    print(f"precise: o {rel_max_bf16_out(o, o_ref):.4g} S_T {rel_max(ST, S_ref):.4g}; "
          f"default: o {rel_max_bf16_out(o_d, o_ref):.4g} S_T {rel_max(ST_d, S_ref):.4g}")
    assert rel_max_bf16_out(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16
    o32, ST32 = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32, precise=True)
    assert rel_max(o32, o_ref) <= TOL_BF16
    assert np.array_equal(ST32, ST)


def test_precise_flag_workload1():
    """The precise plan also meets the bound on the B1 H16 T4096 workload, and is no worse there."""
    d = synth.core_inputs(1, seed=0)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"])
    o, ST = gpu_fwd(d, "bf16", S0=d["S0"], precise=True)
    o_d, ST_d = gpu_fwd(d, "bf16", S0=d["S0"])
    assert rel_max_bf16_out(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= min(TOL_BF16, 1.05 * rel_max(ST_d, S_ref))


# ---- edge cases ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 17, 31, 32, 33, 95, 160])
def test_ragged_lengths_bf16(T):
    d, S0 = rand_small(T, 1, T, 3)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    o, ST = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32)
    assert rel_max(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16


@pytest.mark.parametrize("T,D", [(1, 64), (15, 64), (16, 64), (47, 64), (100, 128)])
def test_ragged_lengths_f32(T, D):
    d, S0 = rand_small(T, 2, T, 2, D=D, io="f32")
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, scale=0.7)
    o, ST = gpu_fwd(d, "f32", S0=S0, scale=0.7)
    assert rel_max(o, o_ref) <= TOL_F32
    assert rel_max(ST, S_ref) <= TOL_F32


def test_batch_heads_not_multiple_of_eight():
    """B*H = 15 takes the plain workgroup mapping; scale != 1."""
    d, S0 = rand_small(5, 3, 70, 5)
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0, scale=0.5)
    o, ST = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32, scale=0.5)
    assert rel_max(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16


def test_decay_at_bound_and_no_decay():
    """g = -5 on half of the channels (largest in-chunk factors) and g = 0 (no decay) on the rest."""
    d, S0 = rand_small(6, 1, 96, 8)
    d["g"][..., ::2] = -5.0
    d["g"][..., 1::2] = 0.0
    o_ref, S_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=S0)
    o, ST = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32)
    assert rel_max(o, o_ref) <= TOL_BF16
    assert rel_max(ST, S_ref) <= TOL_BF16


def test_beta_zero_pure_decay_on_gpu():
    """beta = 0: S_T = Diag(exp(sum g)) S0 exactly in form; o_t = S0^T (exp(b_t) q_t)."""
    d, S0 = rand_small(7, 1, 64, 8)
    d["beta"][:] = 0
    d["g"] *= 0.01  # keep exp(sum g) well inside float32 range over 64 tokens
    o, ST = gpu_fwd(d, "bf16", S0=S0, o_dtype=torch.float32)
    bsum = np.cumsum(d["g"].astype(np.float64), axis=1)
    want_S = np.exp(bsum[:, -1])[..., None] * S0
    want_o = np.einsum("bhij,bthi->bthj", S0.astype(np.float64), np.exp(bsum) * d["q"])
    assert rel_max(ST, want_S) <= TOL_BF16
    assert rel_max(o, want_o) <= TOL_BF16


def test_empty_sequence_copies_state():
    kda = _kda()
    S0 = torch.randn(2, 3, 128, 128, device=DEV)
    e = torch.empty(2, 0, 3, 128, device=DEV, dtype=torch.bfloat16)
    o, ST = kda.kda_fwd(e, e, e, torch.empty(2, 0, 3, 128, device=DEV), torch.empty(2, 0, 3, device=DEV), S0=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128) and torch.equal(ST, S0)


def test_state_in_place_and_segment_split_bitwise():
    """S_T == S0 is allowed; two calls split on the chunk grid equal one call bit for bit."""
    kda = _kda()
    d, S0 = rand_small(8, 2, 128, 4)
    t = to_dev(d, "bf16")
    S = torch.from_numpy(S0).to(DEV)
    o_full, S_full = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=S)
    Sc = S.clone()
    o1, _ = kda.kda_fwd(*(t[n][:, :64].contiguous() for n in ("q", "k", "v", "g", "beta")), S0=Sc, state_out=Sc)
    o2, _ = kda.kda_fwd(*(t[n][:, 64:].contiguous() for n in ("q", "k", "v", "g", "beta")), S0=Sc, state_out=Sc)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=1), o_full)
    assert torch.equal(Sc, S_full)


def test_deterministic_across_runs():
    d, S0 = rand_small(9, 2, 200, 8)
    a = gpu_fwd(d, "bf16", S0=S0)
    b = gpu_fwd(d, "bf16", S0=S0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
