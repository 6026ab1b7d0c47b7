// Input checks of the opt-in validation mode of kda_fwd (KDA_VALIDATE).
//
// The chunkwise kernels rely on the lower bound log(alpha) >= g_min = -5 of the explainer page
// "Kimi K3：开放前沿智能", section 3.2 (paper Eq. 5): it keeps every decay factor they form inside
// float32's range.  This pass scans g for values outside [-5, 0] (NaN included) and q, k, v, beta
// and S0 for non-finite values, and ORs one bit per finding into a caller-provided word.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

// Word-wise scan: n32 32-bit words at p.  kind 0: bf16 pairs, any non-finite half sets `bit`;
// kind 1: float32, non-finite sets `bit`; kind 2: float32 log-decay, anything outside [-5, 0]
// (or NaN) sets `bit`.  Grid-stride loop; every thread that finds something ORs the bit once.
__global__ void __launch_bounds__(256) kda_validate_kernel(const uint32_t* __restrict__ p, size_t n32, int kind,
                                                           uint32_t bit, uint32_t* __restrict__ flags) {
    bool bad = false;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n32; i += stride) {
        const uint32_t w = p[i];
        if (kind == 0) {
            bad |= (w & 0x7f80u) == 0x7f80u || (w & 0x7f800000u) == 0x7f800000u;
        } else if (kind == 1) {
            bad |= (w & 0x7f800000u) == 0x7f800000u;
        } else {
            const float x = __uint_as_float(w);
            bad |= !(x >= -5.f && x <= 0.f);
        }
    }
    if (bad) atomicOr(flags, bit);
}

__global__ void kda_zero_word_kernel(uint32_t* w) { *w = 0u; }

hipError_t scan(const void* p, size_t bytes, int kind, uint32_t bit, uint32_t* flags, hipStream_t stream) {
    if (!p || bytes == 0) return hipSuccess;
    const size_t n32 = bytes / 4;  // every tensor scanned here is a whole number of 32-bit words
    const size_t blocks = (n32 + 255) / 256;
    hipLaunchKernelGGL(kda_validate_kernel, dim3((unsigned)(blocks < 2048 ? (blocks ? blocks : 1) : 2048)), dim3(256),
                       0, stream, static_cast<const uint32_t*>(p), n32, kind, bit, flags);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_validate(const Params& p, bool in_bf16, uint32_t* flags, hipStream_t stream) {
    hipLaunchKernelGGL(kda_zero_word_kernel, dim3(1), dim3(1), 0, stream, flags);
    hipError_t e = hipGetLastError();
    const size_t ntok = (size_t)p.B * p.T * p.H;
    const size_t qk_bytes = ntok * p.Dk * (in_bf16 ? 2 : 4), v_bytes = ntok * p.Dv * (in_bf16 ? 2 : 4);
    const int qkv_kind = in_bf16 ? 0 : 1;
    // (bf16 rows hold Dk or Dv elements, both even on every supported path: whole 32-bit words)
    if (e == hipSuccess) e = scan(p.g, ntok * p.Dk * 4, 2, VALIDATE_G_RANGE, flags, stream);
    if (e == hipSuccess) e = scan(p.q, qk_bytes, qkv_kind, VALIDATE_NONFINITE, flags, stream);
    if (e == hipSuccess) e = scan(p.k, qk_bytes, qkv_kind, VALIDATE_NONFINITE, flags, stream);
    if (e == hipSuccess) e = scan(p.v, v_bytes, qkv_kind, VALIDATE_NONFINITE, flags, stream);
    if (e == hipSuccess) e = scan(p.beta, ntok * 4, 1, VALIDATE_NONFINITE, flags, stream);
    if (e == hipSuccess && p.S0) e = scan(p.S0, (size_t)p.B * p.H * p.Dk * p.Dv * 4, 1, VALIDATE_NONFINITE, flags, stream);
    return e;
}

}  // namespace kda
