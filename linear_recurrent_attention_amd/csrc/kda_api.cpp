// C-ABI entry points: argument validation and dispatch to the gfx950 kernels.
#include "../../include/kda.h"
#include "kda_internal.h"

#include <stdint.h>

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks shared by the forward entry points: sizes, dtypes, pointers, alignment, aliasing.
kda_status check_common(const kda_fwd_desc* d, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, const void* o, const float* S_T, bool need_o = true,
                        int allowed_flags = KDA_FWD_PRECISE) {
    if (!d) return KDA_ERR_INVALID_ARG;
    if (d->B < 1 || d->H < 1 || d->T < 0 || d->Dk < 1 || d->Dv < 1) return KDA_ERR_INVALID_ARG;
    if (d->flags & ~allowed_flags) return KDA_ERR_INVALID_ARG;
    if (d->io_dtype != KDA_F32 && d->io_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (d->o_dtype != KDA_F32 && d->o_dtype != KDA_BF16) return KDA_ERR_INVALID_ARG;
    if (d->io_dtype == KDA_F32 && d->o_dtype != KDA_F32) return KDA_ERR_INVALID_ARG;
    if (!(d->scale == d->scale)) return KDA_ERR_INVALID_ARG;  // NaN scale
    // sizes the kernels index with 32-bit ints: tokens and heads per call
    if ((long long)d->B * d->H > (1LL << 30) || d->T > (1 << 30)) return KDA_ERR_INVALID_ARG;
    if (d->T > 0 && (!q || !k || !v || !g || !beta || (need_o && !o))) return KDA_ERR_INVALID_ARG;
    if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(o, 4)) return KDA_ERR_INVALID_ARG;
    if (!aligned(g, 8) || !aligned(beta, 4) || !aligned(S0, 8) || !aligned(S_T, 8)) return KDA_ERR_INVALID_ARG;
    // outputs must not alias inputs (S_T == S0 is the one allowed overlap)
    if (o && (o == q || o == k || o == v || o == (const void*)g)) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

// The chunk a request names is served by the kernel's own blocking (32 tokens on the bf16 path, 16 on
// the float32 path): the chunkwise form gives the same result for any chunk length in exact
// arithmetic, so a request for a multiple of the kernel's chunk, up to 64, is accepted.
bool chunk_ok(const kda_fwd_desc* d, int kernel_chunk) {
    return d->chunk == 0 || (d->chunk >= kernel_chunk && d->chunk <= 64 && d->chunk % kernel_chunk == 0);
}

// allow_no_o: o may be NULL on the bf16 path (a state-only run; the float32 path always writes o)
kda_status check_fwd(const kda_fwd_desc* d, const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* S0, const void* o, const float* S_T,
                     int allowed_flags = KDA_FWD_PRECISE, bool allow_no_o = false) {
    const bool need_o = !(allow_no_o && d && d->io_dtype == KDA_BF16);
    const kda_status st = check_common(d, q, k, v, g, beta, S0, o, S_T, need_o, allowed_flags);
    if (st != KDA_OK) return st;
    if (d->io_dtype == KDA_BF16) {
        if (d->Dk != 128 || d->Dv != 128) return KDA_ERR_UNSUPPORTED;
        if (!chunk_ok(d, 32)) return KDA_ERR_UNSUPPORTED;
    } else {
        if (d->Dk != d->Dv || (d->Dk != 64 && d->Dk != 128)) return KDA_ERR_UNSUPPORTED;
        if (!chunk_ok(d, 16)) return KDA_ERR_UNSUPPORTED;
    }
    return KDA_OK;
}

constexpr size_t kValidateWs = 256;  // one flag word, padded to the workspace alignment

kda_status check_decode(const kda_fwd_desc* d, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, const void* o, const float* S_T) {
    const kda_status st = check_common(d, q, k, v, g, beta, S0, o, S_T);
    if (st != KDA_OK) return st;
    if (d->chunk != 0) return KDA_ERR_INVALID_ARG;  // no chunking on this path
    if (d->Dk != d->Dv || (d->Dk != 64 && d->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    if ((long long)d->B * d->H * (d->Dv / 64) > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;  // grid size
    return KDA_OK;
}

int chunk_of(const kda_fwd_desc* d) { return d->io_dtype == KDA_BF16 ? 32 : 16; }

kda_status run_fwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* S0, void* o, float* S_T, float* S_ckpt, int every,
                   hipStream_t stream) {
    kda::Params p{};  // zero: every optional field off
    p.S_ckpt = S_ckpt;
    p.ckpt_chunks = S_ckpt ? every / chunk_of(desc) : 1;
    p.n_ckpt = S_ckpt ? desc->T / every : 0;
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0; p.o = o; p.S_T = S_T;
    p.B = desc->B; p.T = desc->T; p.H = desc->H; p.Dk = desc->Dk; p.Dv = desc->Dv; p.tstride = desc->T;
    p.scale = desc->scale;
    p.o_f32 = desc->o_dtype == KDA_F32;
    p.in_f32 = 0;
    p.precise = (desc->flags & KDA_FWD_PRECISE) != 0;
    hipError_t e;
    if (desc->T == 0)
        e = kda::launch_state_copy(p, stream);
    else if (desc->io_dtype == KDA_BF16)
        e = kda::launch_fwd_bf16(p, stream);
    else
        e = kda::launch_fwd_f32(p, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Params of the context-parallel forward (the bf16 path; every optional field off).
kda::Params cp_params(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* S0, void* o, float* S_T) {
    kda::Params p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0; p.o = o; p.S_T = S_T;
    p.B = desc->B; p.T = desc->T; p.H = desc->H; p.Dk = desc->Dk; p.Dv = desc->Dv; p.tstride = desc->T;
    p.scale = desc->scale;
    p.o_f32 = desc->o_dtype == KDA_F32;
    p.precise = (desc->flags & KDA_FWD_PRECISE) != 0;
    p.ckpt_chunks = 1;
    return p;
}

}  // namespace

extern "C" {

size_t kda_fwd_workspace_size(const kda_fwd_desc* desc) {
    return (desc && (desc->flags & KDA_VALIDATE)) ? kValidateWs : 0;
}

kda_status kda_fwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* S0, void* o, float* S_T, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
    const kda_status st = check_fwd(desc, q, k, v, g, beta, S0, o, S_T, KDA_FWD_PRECISE | KDA_VALIDATE, true);
    if (st != KDA_OK) return st;
    if (desc->T > 0 && !o && !S_T) return KDA_ERR_INVALID_ARG;  // nothing to compute
    if ((desc->flags & KDA_VALIDATE) && desc->T > 0) {
        if (!ws || ws_bytes < kValidateWs || !aligned(ws, 256)) return KDA_ERR_WORKSPACE;
        kda::Params p{};
        p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0;
        p.B = desc->B; p.T = desc->T; p.H = desc->H; p.Dk = desc->Dk; p.Dv = desc->Dv;
        uint32_t* flag = static_cast<uint32_t*>(ws);
        if (kda::launch_validate(p, desc->io_dtype == KDA_BF16, flag, stream) != hipSuccess) return KDA_ERR_HIP;
        uint32_t found = 0;
        if (hipMemcpyAsync(&found, flag, sizeof(found), hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return KDA_ERR_HIP;
        if (found) return KDA_ERR_INVALID_ARG;
    }
    return run_fwd(desc, q, k, v, g, beta, S0, o, S_T, nullptr, 0, stream);
}

kda_status kda_fwd_ckpt(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, void* o, float* S_T, float* S_ckpt, int every,
                        hipStream_t stream) {
    const kda_status st = check_fwd(desc, q, k, v, g, beta, S0, o, S_T, KDA_FWD_PRECISE, true);
    if (st != KDA_OK) return st;
    if (every <= 0 || every % chunk_of(desc) != 0) return KDA_ERR_INVALID_ARG;
    const int n_ckpt = desc->T / every;
    if (n_ckpt > 0 && !S_ckpt) return KDA_ERR_INVALID_ARG;
    if (desc->T > 0 && !o && !S_T && n_ckpt == 0) return KDA_ERR_INVALID_ARG;  // nothing to compute
    if (!aligned(S_ckpt, 8)) return KDA_ERR_INVALID_ARG;
    if (S_ckpt && ((const void*)S_ckpt == o || S_ckpt == S_T || S_ckpt == S0)) return KDA_ERR_INVALID_ARG;
    return run_fwd(desc, q, k, v, g, beta, S0, o, S_T, n_ckpt > 0 ? S_ckpt : nullptr, every, stream);
}

kda_status kda_decode(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* S0, void* o, float* S_T, hipStream_t stream) {
    const kda_status st = check_decode(desc, q, k, v, g, beta, S0, o, S_T);
    if (st != KDA_OK) return st;
    kda::Params p{};  // zero: every optional field off
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0; p.o = o; p.S_T = S_T;
    p.B = desc->B; p.T = desc->T; p.H = desc->H; p.Dk = desc->Dk; p.Dv = desc->Dv; p.tstride = desc->T;
    p.scale = desc->scale;
    p.o_f32 = desc->o_dtype == KDA_F32;
    p.in_f32 = 0;
    p.precise = 0;
    p.S_ckpt = nullptr; p.ckpt_chunks = 1; p.n_ckpt = 0;
    const hipError_t e = desc->T == 0 ? kda::launch_state_copy(p, stream)
                                      : kda::launch_decode(p, desc->io_dtype == KDA_BF16, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_fwd_cp_workspace_size(const kda_fwd_desc* desc, int nseg) {
    if (!desc || nseg < 0 || desc->B < 1 || desc->H < 1 || desc->T < 0 || desc->io_dtype != KDA_BF16) return 0;
    if ((long long)desc->B * desc->H > (1LL << 30)) return 0;
    return kda::cp_workspace_bytes(desc->B, desc->T, desc->H, nseg);
}

kda_status kda_fwd_cp(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* S0, void* o, float* S_T, int nseg, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    const kda_status st = check_fwd(desc, q, k, v, g, beta, S0, o, S_T);
    if (st != KDA_OK) return st;
    if (nseg < 0 || nseg > 4096) return KDA_ERR_INVALID_ARG;
    if (desc->io_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((long long)desc->B * desc->H * (nseg ? nseg : 1) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    const size_t need = kda::cp_workspace_bytes(desc->B, desc->T, desc->H, nseg);
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return KDA_ERR_WORKSPACE;
    if (desc->T == 0) return run_fwd(desc, q, k, v, g, beta, S0, o, S_T, nullptr, 0, stream);
    const kda::Params p = cp_params(desc, q, k, v, g, beta, S0, o, S_T);
    const hipError_t e = kda::launch_fwd_cp(p, nseg, static_cast<float*>(ws), stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_fwd_cp_noalloc(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* S0, void* o, float* S_T, int nseg, hipStream_t stream) {
    const kda_status st = check_fwd(desc, q, k, v, g, beta, S0, o, S_T);
    if (st != KDA_OK) return st;
    if (nseg < 0 || nseg > 4096) return KDA_ERR_INVALID_ARG;
    if (desc->io_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if ((long long)desc->B * desc->H * (nseg ? nseg : 1) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (kda::cp_workspace_bytes(desc->B, desc->T, desc->H, nseg) > KDA_CP_NOALLOC_SCRATCH_BYTES)
        return KDA_ERR_SCRATCH_LIMIT;
    if (desc->T == 0) return run_fwd(desc, q, k, v, g, beta, S0, o, S_T, nullptr, 0, stream);
    const kda::Params p = cp_params(desc, q, k, v, g, beta, S0, o, S_T);
    const hipError_t e = kda::launch_fwd_cp_noalloc(p, nseg, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_bwd_workspace_size(const kda_fwd_desc* desc) {
    if (!desc || desc->B < 1 || desc->H < 1 || desc->T < 0 || desc->Dk != desc->Dv) return 0;
    if (desc->io_dtype == KDA_BF16 ? desc->Dk != 128 : (desc->Dk != 64 && desc->Dk != 128)) return 0;
    if ((long long)desc->B * desc->H > (1LL << 30)) return 0;
    return kda::bwd_workspace_bytes(desc->B, desc->T, desc->H, desc->Dk, desc->io_dtype == KDA_BF16);
}

kda_status kda_bwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* S0, const void* dO, const float* dS_T, float* dq, float* dk,
                   float* dv, float* dg, float* dbeta, float* dS0, void* ws, size_t ws_bytes, hipStream_t stream) {
    kda_status st = check_common(desc, q, k, v, g, beta, S0, dO, dS_T, /*need_o=*/false);
    if (st != KDA_OK) return st;
    if (desc->chunk != 0) return KDA_ERR_INVALID_ARG;
    if (desc->Dk != desc->Dv) return KDA_ERR_UNSUPPORTED;
    if (desc->io_dtype == KDA_BF16 ? desc->Dk != 128 : (desc->Dk != 64 && desc->Dk != 128)) return KDA_ERR_UNSUPPORTED;
    const float* outs[6] = {dq, dk, dv, dg, dbeta, dS0};
    const void* ins[8] = {q, k, v, g, beta, S0, dO, dS_T};
    for (const float* a : outs) {
        if (!a) continue;
        if (!aligned(a, 4)) return KDA_ERR_INVALID_ARG;
        for (const void* b : ins)
            if (b == a) return KDA_ERR_INVALID_ARG;
        int same = 0;
        for (const float* b : outs) same += (b == a);
        if (same > 1) return KDA_ERR_INVALID_ARG;
    }
    const size_t need = kda::bwd_workspace_bytes(desc->B, desc->T, desc->H, desc->Dk, desc->io_dtype == KDA_BF16);
    if (desc->T > 0 && (!ws || ws_bytes < need || !aligned(ws, 256))) return KDA_ERR_WORKSPACE;
    kda::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S0; p.dO = dO; p.dST = dS_T;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dbeta = dbeta; p.dS0 = dS0;
    p.B = desc->B; p.T = desc->T; p.H = desc->H; p.D = desc->Dk; p.scale = desc->scale;
    hipError_t e;
    if (desc->T == 0) {  // dS0 = dS_T (or zero)
        kda::Params c{};
        c.B = desc->B; c.H = desc->H; c.Dk = desc->Dk; c.Dv = desc->Dv; c.S0 = dS_T; c.S_T = dS0;
        e = kda::launch_state_copy(c, stream);
    } else {
        e = kda::launch_bwd(p, desc->io_dtype == KDA_BF16, desc->o_dtype == KDA_BF16,
                            (desc->flags & KDA_FWD_PRECISE) != 0 || desc->io_dtype == KDA_BF16, static_cast<float*>(ws),
                            stream);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

const char* kda_error_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: no kernel for this configuration";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error at launch";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_SCRATCH_LIMIT:
            return "KDA_ERR_SCRATCH_LIMIT: the problem needs more scratch than the fixed buffer of an allocation-free "
                   "entry point holds";
    }
    return "unknown kda_status";
}

int kda_version(void) { return 100; }

}  // extern "C"
