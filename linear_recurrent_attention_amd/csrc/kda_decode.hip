// Token-by-token KDA step for decoding, on gfx950.
//
// What is computed: the gated delta rule of the explainer page "Kimi K3：开放前沿智能",
// section 2.2 (paper Eq. 1), one token at a time in the order the page gives (decay, then the
// delta-rule erase and write), read out after the update (section 2.4):
//   S <- Diag(alpha_t) S,   w = S^T k_t,   S <- S + beta_t k_t (v_t - w)^T,   o_t = S^T (scale q_t).
// This is the decode-time step of section 13.10 (the state update and readout of one new token; the
// projections around it are the caller's).  With a handful of tokens per call the chunkwise form
// has nothing to amortise, and the cost is reading and writing the float32 state once per call:
// the kernel is bound by HBM bandwidth on S.
//
// Mapping: one workgroup of 256 threads per (batch, head, block of 64 value columns).  Thread
// (row group rg, column j) keeps rows rg*D/4 .. rg*D/4 + D/4 - 1 of column j of S in registers for
// all tokens of the call; each wave reads and writes 64 consecutive floats of a state row at a time.
// The two column sums (w and o) are reduced over the four row groups through LDS.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace decode {

constexpr int NTHR = 256;
constexpr int COLS = 64;  // value columns per workgroup
constexpr int RG = 4;     // row groups

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, size_t i) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
    else
        return reinterpret_cast<const float*>(p)[i];
}

template <int D, bool IN_BF16, bool OUT_BF16>
__global__ void __launch_bounds__(NTHR) kda_decode_kernel(Params p) {
    constexpr int ROWS = D / RG;
    constexpr int NCB = D / COLS;  // column blocks per head
    __shared__ float sq[D], sk[D], sa[D], sv[COLS], sbeta;
    __shared__ float pw[RG][COLS], po[RG][COLS];
    const int tid = threadIdx.x, j = tid & (COLS - 1), rg = tid / COLS;
    const int bh = blockIdx.x / NCB, cb = blockIdx.x - bh * NCB;
    const int b = bh / p.H, h = bh - b * p.H;
    const int col = cb * COLS + j;
    const size_t sbase = (size_t)bh * D * D + (size_t)(rg * ROWS) * D + col;

    float s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) s[i] = p.S0 ? p.S0[sbase + (size_t)i * D] : 0.f;

    for (int t = 0; t < p.T; ++t) {
        const size_t row = ((size_t)b * p.tstride + t) * p.H + h;  // token row of the [B, T, H, *] tensors
        if (tid < D) {
            sq[tid] = ld_in<IN_BF16>(p.q, row * D + tid);
            sk[tid] = ld_in<IN_BF16>(p.k, row * D + tid);
            sa[tid] = fexp(p.g[row * D + tid]);
        }
        if (tid < COLS) sv[tid] = ld_in<IN_BF16>(p.v, row * D + cb * COLS + tid);
        if (tid == 0) sbeta = p.beta[row];
        __syncthreads();
        // decay, then this row group's share of w = S^T k
        float w = 0.f;
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            s[i] *= sa[rg * ROWS + i];
            w = __builtin_fmaf(s[i], sk[rg * ROWS + i], w);
        }
        pw[rg][j] = w;
        __syncthreads();
        const float u = sbeta * (sv[j] - ((pw[0][j] + pw[1][j]) + (pw[2][j] + pw[3][j])));
        // write k u^T, then this row group's share of o = S^T q
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            s[i] = __builtin_fmaf(sk[rg * ROWS + i], u, s[i]);
            o = __builtin_fmaf(s[i], sq[rg * ROWS + i], o);
        }
        po[rg][j] = o;
        __syncthreads();
        if (rg == 0 && p.o) {  // (o == NULL: state only)
            const float ot = ((po[0][j] + po[1][j]) + (po[2][j] + po[3][j])) * p.scale;
            if constexpr (OUT_BF16) {
                const uint32_t pk = pack_bf16(ot, 0.f);
                reinterpret_cast<uint16_t*>(p.o)[row * D + col] = (uint16_t)(pk & 0xffffu);
            } else {
                reinterpret_cast<float*>(p.o)[row * D + col] = ot;
            }
        }
        // the next token's staging writes sq/sk/sa/sv only after every thread has passed the
        // barrier above, where all reads of them are done; pw and po are rewritten after the
        // next staging barrier, which row group 0 reaches only after its reads of po
    }
    if (p.S_T) {
#pragma unroll
        for (int i = 0; i < ROWS; ++i) p.S_T[sbase + (size_t)i * D] = s[i];
    }
}

template <int D>
void launch_d(const Params& p, bool in_bf16, bool out_bf16, hipStream_t stream) {
    const dim3 grid((unsigned)(p.B * p.H * (D / COLS))), block(NTHR);
    if (in_bf16 && out_bf16)
        hipLaunchKernelGGL((kda_decode_kernel<D, true, true>), grid, block, 0, stream, p);
    else if (in_bf16)
        hipLaunchKernelGGL((kda_decode_kernel<D, true, false>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((kda_decode_kernel<D, false, false>), grid, block, 0, stream, p);
}

}  // namespace decode

hipError_t launch_decode(const Params& p, bool in_bf16, hipStream_t stream) {
    const bool out_bf16 = !p.o_f32;
    if (p.Dk == 64)
        decode::launch_d<64>(p, in_bf16, out_bf16, stream);
    else
        decode::launch_d<128>(p, in_bf16, out_bf16, stream);
    return hipGetLastError();
}

}  // namespace kda
