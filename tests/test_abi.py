"""C-ABI: the library loads, exports what include/kda.h declares, and rejects bad arguments
before touching the GPU (no compute call is made in these tests)."""
import ctypes
import os
import re

import pytest

from linear_recurrent_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b(kda_[a-z0-9_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    decl = declared_functions()
    assert "kda_fwd" in decl and "kda_error_string" in decl
    for name in decl:
        assert hasattr(L, name), name
    assert set(decl) == set(_lib.EXPORTS)


def test_version_and_error_strings():
    L = _lib.lib()
    assert L.kda_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert L.kda_error_string(code)


def desc(**kw):
    d = dict(B=1, T=64, H=2, Dk=128, Dv=128, chunk=0, io_dtype=_lib.KDA_BF16, o_dtype=_lib.KDA_BF16, scale=1.0,
             flags=0)
    d.update(kw)
    return _lib.FwdDesc(**d)


FAKE = 0x10000  # never dereferenced: validation fails first, or T = 0 makes no launch


def call(d, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, o=FAKE + 0x100000, S_T=0):
    return _lib.fwd_raw(d, q, k, v, g, beta, S0, o, S_T, None)


def test_null_descriptor():
    assert _lib.lib().kda_fwd(None, *([None] * 9), 0, None) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [("B", 0), ("H", 0), ("T", -1), ("Dk", 0), ("Dv", -3), ("flags", 4), ("flags", -1),
                                         ("io_dtype", 5), ("o_dtype", 9)])
def test_bad_sizes_and_enums(field, value):
    assert call(desc(**{field: value})) == _lib.KDA_ERR_INVALID_ARG


def test_precise_flag_accepted_with_empty_sequence():
    # T = 0 launches only the state copy; the flag is a valid request on either path
    for io in (_lib.KDA_BF16, _lib.KDA_F32):
        d = desc(T=0, flags=_lib.KDA_FWD_PRECISE, io_dtype=io, o_dtype=io)
        assert _lib.fwd_raw(d, 0, 0, 0, 0, 0, 0, 0, 0, None) == _lib.KDA_OK


def test_nan_scale():
    assert call(desc(scale=float("nan"))) == _lib.KDA_ERR_INVALID_ARG


def test_f32_inputs_need_f32_output():
    assert call(desc(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_BF16, Dk=64, Dv=64)) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("ptr", ["q", "k", "v", "g", "beta", "o"])
def test_null_required_pointer(ptr):
    assert call(desc(), **{ptr: 0}) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("ptr,off", [("q", 2), ("v", 1), ("g", 4), ("o", 2), ("S0", 4), ("S_T", 4)])
def test_misaligned_pointer(ptr, off):
    assert call(desc(), **{ptr: FAKE + 0x20000 + off}) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=64, Dv=64), dict(Dk=128, Dv=64), dict(chunk=16), dict(chunk=48),
                                dict(chunk=96), dict(chunk=-32),
                                dict(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=96, Dv=96),
                                dict(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64, chunk=24),
                                dict(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64, chunk=128)])
def test_unsupported_shapes(kw):
    assert call(desc(**kw)) == _lib.KDA_ERR_UNSUPPORTED


@pytest.mark.parametrize("io,chunk", [(_lib.KDA_BF16, 32), (_lib.KDA_BF16, 64), (_lib.KDA_F32, 16),
                                      (_lib.KDA_F32, 32), (_lib.KDA_F32, 64)])
def test_chunk_requests_served_by_kernel_blocking(io, chunk):
    # the workloads' C = 64 (and any multiple of the kernel's own chunk up to 64) is a valid request
    d = desc(T=0, chunk=chunk, io_dtype=io, o_dtype=io, Dk=64 if io == _lib.KDA_F32 else 128,
             Dv=64 if io == _lib.KDA_F32 else 128)
    assert _lib.fwd_raw(d, 0, 0, 0, 0, 0, 0, 0, 0, None) == _lib.KDA_OK


def test_workspace_size_query():
    assert _lib.fwd_workspace_size(desc()) == 0
    assert _lib.fwd_workspace_size(desc(flags=_lib.KDA_FWD_PRECISE)) == 0
    assert _lib.fwd_workspace_size(desc(flags=_lib.KDA_VALIDATE)) == 256
    assert _lib.lib().kda_fwd_workspace_size(None) == 0


@pytest.mark.parametrize("ws,ws_bytes", [(0, 0), (0, 256), (FAKE + 0x300000, 255), (FAKE + 0x300000 + 16, 256)])
def test_validate_needs_its_workspace(ws, ws_bytes):
    # missing, too small or misaligned workspace: rejected before any device call
    d = desc(flags=_lib.KDA_VALIDATE)
    assert _lib.fwd_raw(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE + 0x100000, 0, None, ws, ws_bytes) == \
        _lib.KDA_ERR_WORKSPACE


def test_validate_flag_only_on_kda_fwd():
    d = desc(flags=_lib.KDA_VALIDATE)
    assert _lib.fwd_ckpt_raw(d, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE + 0x100000, 0, FAKE + 0x200000, 32, None) == \
        _lib.KDA_ERR_INVALID_ARG
    assert _lib.decode_raw(desc(flags=_lib.KDA_VALIDATE, chunk=0), FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE + 0x100000,
                           0, None) == _lib.KDA_ERR_INVALID_ARG


def test_state_only_forward_needs_a_state_output():
    # o = NULL asks for the state alone (bf16 path): with no S_T (and no checkpoint) nothing is computed
    assert call(desc(), o=0, S_T=0) == _lib.KDA_ERR_INVALID_ARG
    # the float32 path always writes o
    assert call(desc(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64), o=0,
                S_T=FAKE + 0x300000) == _lib.KDA_ERR_INVALID_ARG
    assert call_ckpt(desc(T=64), 128, o=0, S_ckpt=0) == _lib.KDA_ERR_INVALID_ARG


def test_output_aliasing_input_rejected():
    assert call(desc(), o=FAKE) == _lib.KDA_ERR_INVALID_ARG


def test_empty_sequence_without_state_output_is_a_no_op():
    # T = 0 and S_T = NULL: nothing to compute, nothing launched
    assert call(desc(T=0), q=0, k=0, v=0, g=0, beta=0, o=0) == _lib.KDA_OK


def test_python_binding_checks_shapes():
    torch = pytest.importorskip("torch")
    import linear_recurrent_attention_amd as kda
    q = torch.zeros(1, 4, 2, 128)
    with pytest.raises(ValueError):
        kda.kda_fwd(q, q, q, q, torch.zeros(1, 4, 2))  # CPU tensors are rejected before any call


def call_ckpt(d, every, S_ckpt=FAKE + 0x200000, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, o=FAKE + 0x100000, S_T=0)
    a.update(kw)
    return _lib.fwd_ckpt_raw(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], S_ckpt,
                             every, None)


@pytest.mark.parametrize("every", [0, -32, 16, 48, 33])
def test_checkpoint_interval_must_be_a_chunk_multiple(every):
    # bf16 I/O runs 32-token chunks
    assert call_ckpt(desc(), every) == _lib.KDA_ERR_INVALID_ARG


def test_checkpoint_interval_f32_chunk():
    # float32 I/O runs 16-token chunks: 48 is valid (T = 0: nothing launched), 24 is not
    d = desc(T=0, io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64)
    assert _lib.fwd_ckpt_raw(d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 48, None) == _lib.KDA_OK
    assert _lib.fwd_ckpt_raw(d, 0, 0, 0, 0, 0, 0, 0, 0, 0, 24, None) == _lib.KDA_ERR_INVALID_ARG


def test_checkpoint_buffer_required_when_any_checkpoint_falls_in_range():
    assert call_ckpt(desc(T=64), 64, S_ckpt=0) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(S_ckpt=FAKE + 0x100000), dict(S_ckpt=FAKE + 0x200004)])
def test_checkpoint_buffer_aliasing_or_misaligned(kw):
    assert call_ckpt(desc(T=64), 32, **kw) == _lib.KDA_ERR_INVALID_ARG


def test_checkpoint_call_validates_the_descriptor_first():
    assert call_ckpt(desc(B=0), 32) == _lib.KDA_ERR_INVALID_ARG
    assert call_ckpt(desc(Dk=64, Dv=64), 32) == _lib.KDA_ERR_UNSUPPORTED


def call_decode(d, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, o=FAKE + 0x100000, S_T=0)
    a.update(kw)
    return _lib.decode_raw(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], None)


def test_decode_rejects_a_chunk_size():
    assert call_decode(desc(chunk=32)) == _lib.KDA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(Dk=96, Dv=96), dict(Dk=128, Dv=64), dict(Dk=32, Dv=32)])
def test_decode_unsupported_head_sizes(kw):
    assert call_decode(desc(**kw)) == _lib.KDA_ERR_UNSUPPORTED


def test_decode_shares_the_forward_argument_checks():
    assert call_decode(desc(B=0)) == _lib.KDA_ERR_INVALID_ARG
    assert call_decode(desc(), o=FAKE) == _lib.KDA_ERR_INVALID_ARG        # output aliases q
    assert call_decode(desc(), g=FAKE + 0x20004) == _lib.KDA_ERR_INVALID_ARG  # misaligned g
    # T = 0 with Dk = 64 bf16 (valid on this path) launches nothing without S_T
    assert call_decode(desc(T=0, Dk=64, Dv=64), q=0, k=0, v=0, g=0, beta=0, o=0) == _lib.KDA_OK


def test_cp_workspace_size_plan():
    # B=1, H=16, T=2^20: automatic plan = 8 segments of 2^17 tokens -> three [8, 16, 128, 128] float buffers
    d = desc(B=1, T=1 << 20, H=16)
    assert _lib.cp_workspace_size(d, 0) == 3 * 8 * 16 * 128 * 128 * 4
    assert _lib.cp_workspace_size(d, 4) == 3 * 4 * 16 * 128 * 128 * 4
    assert _lib.cp_workspace_size(d, 1) == 0                       # nseg = 1 is kda_fwd
    # enough heads already: the automatic plan is one segment
    assert _lib.cp_workspace_size(desc(B=4, T=16384, H=32), 0) == 0
    # a ragged T: the last segment takes the rest; every sequence's segments run together
    assert _lib.cp_workspace_size(desc(B=2, T=4096 + 5, H=2), 4) == 3 * 2 * 4 * 2 * 128 * 128 * 4
    assert _lib.cp_workspace_size(desc(B=2, T=4096, H=2), 4) == 3 * 2 * 4 * 2 * 128 * 128 * 4
    # the automatic plan for two sequences of 16 heads at 8192 tokens: three segments
    assert _lib.cp_workspace_size(desc(B=2, T=8192, H=16), 0) == 3 * 2 * 3 * 16 * 128 * 128 * 4
    # too short for the requested segments (T < nseg * 32)
    assert _lib.cp_workspace_size(desc(T=100), 4) == 0
    # invalid descriptors
    assert _lib.cp_workspace_size(desc(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32), 4) == 0
    assert _lib.cp_workspace_size(desc(B=0), 4) == 0
    assert _lib.cp_workspace_size(d, -1) == 0


def call_cp(d, nseg, ws=0, ws_bytes=0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, o=FAKE + 0x100000, S_T=0)
    a.update(kw)
    return _lib.fwd_cp_raw(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], nseg, ws,
                           ws_bytes, None)


def test_cp_argument_checks():
    d = desc(B=1, T=1 << 16, H=2)
    need = _lib.cp_workspace_size(d, 4)
    assert need > 0
    assert call_cp(d, 4) == _lib.KDA_ERR_WORKSPACE                                  # no workspace
    assert call_cp(d, 4, ws=FAKE + 0x400000, ws_bytes=need - 1) == _lib.KDA_ERR_WORKSPACE
    assert call_cp(d, 4, ws=FAKE + 0x400010, ws_bytes=need) == _lib.KDA_ERR_WORKSPACE  # not 256-aligned
    assert call_cp(d, -2) == _lib.KDA_ERR_INVALID_ARG
    assert call_cp(desc(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64), 2) == _lib.KDA_ERR_UNSUPPORTED
    assert call_cp(desc(B=0), 2) == _lib.KDA_ERR_INVALID_ARG
    # T = 0: the state copy only (nothing launched without S_T)
    assert call_cp(desc(T=0), 4, q=0, k=0, v=0, g=0, beta=0, o=0) == _lib.KDA_OK


def call_cp_noalloc(d, nseg, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, o=FAKE + 0x100000, S_T=0)
    a.update(kw)
    return _lib.fwd_cp_noalloc_raw(d, a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["o"], a["S_T"], nseg, None)


def test_cp_noalloc_argument_checks_and_scratch_limit():
    """kda_fwd_cp_noalloc checks what kda_fwd_cp checks, and refuses, before any device call, a plan
    whose segment states exceed its fixed scratch array."""
    limit = _lib.KDA_CP_NOALLOC_SCRATCH_BYTES
    big = desc(B=1, T=1 << 20, H=32)
    assert _lib.cp_workspace_size(big, 8) > limit
    assert call_cp_noalloc(big, 8) == _lib.KDA_ERR_SCRATCH_LIMIT
    assert call_cp_noalloc(desc(B=4, T=1 << 16, H=16), 4) == _lib.KDA_ERR_SCRATCH_LIMIT  # 4 rows x 4 segments x 16 heads
    assert _lib.cp_workspace_size(desc(B=1, T=1 << 20, H=16), 0) <= limit                # the long-context plan fits
    assert "SCRATCH_LIMIT" in _lib.lib().kda_error_string(_lib.KDA_ERR_SCRATCH_LIMIT).decode()
    assert call_cp_noalloc(big, -1) == _lib.KDA_ERR_INVALID_ARG
    assert call_cp_noalloc(desc(B=0), 2) == _lib.KDA_ERR_INVALID_ARG
    assert call_cp_noalloc(desc(io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32, Dk=64, Dv=64), 2) == _lib.KDA_ERR_UNSUPPORTED
    assert _lib.lib().kda_fwd_cp_noalloc(None, *([None] * 8), 2, None) == _lib.KDA_ERR_INVALID_ARG
    # T = 0: the state copy only (nothing launched without S_T), so no scratch is touched
    assert call_cp_noalloc(desc(T=0), 4, q=0, k=0, v=0, g=0, beta=0, o=0) == _lib.KDA_OK


def test_bwd_workspace_size():
    # bf16 inputs: 32-token intervals; float32 inputs: 16-token intervals; two [B, H, n, D, D] arrays
    assert _lib.bwd_workspace_size(desc(B=2, T=100, H=3)) == 2 * 2 * 3 * 4 * 128 * 128 * 4
    d32 = desc(B=1, T=100, H=2, Dk=64, Dv=64, io_dtype=_lib.KDA_F32, o_dtype=_lib.KDA_F32)
    assert _lib.bwd_workspace_size(d32) == 2 * 1 * 2 * 7 * 64 * 64 * 4
    assert _lib.bwd_workspace_size(desc(Dk=64, Dv=64)) == 0          # bf16 inputs need D = 128
    assert _lib.bwd_workspace_size(desc(B=0)) == 0


def call_bwd(d, ws=0, ws_bytes=0, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, S0=0, dO=FAKE + 0x100000, dST=0, dq=FAKE + 0x200000,
             dk=FAKE + 0x300000, dv=FAKE + 0x400000, dg=FAKE + 0x500000, dbeta=FAKE + 0x600000, dS0=0)
    a.update(kw)
    return _lib.bwd_raw(d, *[a[n] for n in ("q", "k", "v", "g", "beta", "S0", "dO", "dST", "dq", "dk", "dv", "dg",
                                            "dbeta", "dS0")], ws, ws_bytes, None)


def test_bwd_argument_checks():
    d = desc(T=64)
    need = _lib.bwd_workspace_size(d)
    ws = FAKE + 0x1000000
    assert call_bwd(d) == _lib.KDA_ERR_WORKSPACE
    assert call_bwd(d, ws=ws, ws_bytes=need - 4) == _lib.KDA_ERR_WORKSPACE
    assert call_bwd(desc(chunk=32), ws=ws, ws_bytes=need) == _lib.KDA_ERR_INVALID_ARG
    assert call_bwd(desc(Dk=64, Dv=64), ws=ws, ws_bytes=need) == _lib.KDA_ERR_UNSUPPORTED
    assert call_bwd(d, ws=ws, ws_bytes=need, dq=FAKE) == _lib.KDA_ERR_INVALID_ARG          # dq aliases q
    assert call_bwd(d, ws=ws, ws_bytes=need, dk=FAKE + 0x200000) == _lib.KDA_ERR_INVALID_ARG  # dk aliases dq
    assert call_bwd(d, ws=ws, ws_bytes=need, dg=FAKE + 0x500002) == _lib.KDA_ERR_INVALID_ARG  # misaligned
    assert call_bwd(desc(B=0), ws=ws, ws_bytes=need) == _lib.KDA_ERR_INVALID_ARG
    # T = 0: dS0 = dS_T; with dS0 = NULL nothing is launched
    assert call_bwd(desc(T=0), q=0, k=0, v=0, g=0, beta=0, dO=0) == _lib.KDA_OK


def call_layer(d_model=256, rank=32, x=FAKE, y=FAKE + 0x100000, **kw):
    d = _lib.LayerDesc(1, 8, d_model, 2, 128, 128, rank, 4, 1.0, 0)
    for k, v in kw.items():
        setattr(d, k, v)
    w = _lib.LayerWeights(*([FAKE + 0x200000] * len(_lib.LAYER_WEIGHT_FIELDS)))
    need = _lib.layer_workspace_size(d)
    return _lib.layer_fwd_raw(d, x, w, 0, 0, y, 0, 0, FAKE + 0x400000, need, None)


def test_layer_argument_checks():
    """The layer's GEMMs step k by 32 columns and move 16-byte chunks: other widths are unsupported and
    misaligned activations are rejected, before any device call."""
    assert call_layer(d_model=40) == _lib.KDA_ERR_UNSUPPORTED      # not a multiple of 32
    assert call_layer(rank=24) == _lib.KDA_ERR_UNSUPPORTED         # not a multiple of 16
    assert call_layer(x=FAKE + 8) == _lib.KDA_ERR_INVALID_ARG      # x not 16-byte aligned
    assert call_layer(y=FAKE + 0x100004) == _lib.KDA_ERR_INVALID_ARG
    assert call_layer(flags=1) == _lib.KDA_ERR_INVALID_ARG
    assert _lib.layer_workspace_size(_lib.LayerDesc(0, 8, 256, 2, 128, 128, 32, 4, 1.0, 0)) == 0


def test_layer_decode_argument_checks():
    """Rows per call, rank, flags and the speculative cache are checked before any device call."""
    def desc_(B=1, T=1, rank=32, flags=0):
        return _lib.LayerDesc(B, T, 256, 2, 128, 128, rank, 4, 1.0, flags)
    assert _lib.layer_decode_workspace_size(desc_()) > 0
    assert _lib.layer_decode_cache_bytes(desc_(B=2, T=3)) == 2 * 3 * (5 * 2 * 128 + 2) * 4
    assert _lib.layer_decode_workspace_size(desc_(B=4, T=5)) == 0         # 20 rows > 16
    assert _lib.layer_decode_workspace_size(desc_(rank=256)) == 0         # rank > 128
    w = _lib.LayerWeights(*([FAKE + 0x200000] * len(_lib.LAYER_WEIGHT_FIELDS)))
    d = desc_(flags=_lib.KDA_DECODE_SPECULATIVE)
    ws = _lib.layer_decode_workspace_size(d)
    assert _lib.layer_decode_raw(d, FAKE, w, FAKE, 0, FAKE, 0, FAKE, ws, None) == _lib.KDA_ERR_INVALID_ARG  # no cache
    assert _lib.layer_decode_raw(desc_(flags=2), FAKE, w, FAKE, 0, FAKE, 0, FAKE, ws, None) == _lib.KDA_ERR_INVALID_ARG
    assert _lib.layer_decode_raw(desc_(B=4, T=5), FAKE, w, FAKE, 0, FAKE, 0, FAKE, ws, None) == _lib.KDA_ERR_UNSUPPORTED
    assert _lib.layer_decode_raw(desc_(), FAKE, w, 0, 0, FAKE, 0, FAKE, ws, None) == _lib.KDA_ERR_INVALID_ARG  # no S
    assert _lib.layer_decode_raw(desc_(), FAKE, w, FAKE, 0, FAKE, 0, FAKE, ws - 1, None) == _lib.KDA_ERR_WORKSPACE
    assert _lib.layer_decode_commit_raw(desc_(T=4), FAKE, 5, FAKE, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert _lib.layer_decode_commit_raw(desc_(T=4), FAKE, -1, FAKE, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert _lib.layer_decode_commit_raw(desc_(T=4), 0, 2, FAKE, 0, None) == _lib.KDA_ERR_INVALID_ARG
    assert _lib.layer_decode_commit_raw(desc_(T=4), FAKE, 0, FAKE, 0, None) == _lib.KDA_OK  # nothing accepted
