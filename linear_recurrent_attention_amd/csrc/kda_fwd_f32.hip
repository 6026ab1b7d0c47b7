// Chunkwise KDA forward with float32 inputs, outputs and arithmetic (d_k = d_v = D in {64, 128}).
//
// Same method as the bf16 path (the gated delta rule of the explainer page "Kimi K3：开放前沿智能",
// section 2.2 / paper Eq. 1, read out after the update as in section 2.4, computed chunk by chunk
// as in section 2.5 / paper Eq. 4), but every product runs in float32 on the vector ALUs so the
// result tracks a float64 evaluation to about 1e-6.  Chunks are 16 tokens; the decay factors of a
// chunk are taken relative to its token 7, so they stay in [e^-40, e^40] under the g >= -5 bound
// of section 3.2.  One workgroup per (batch, head); the state lives in LDS.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace f32path {

constexpr int C = 16;
constexpr int NTHR = 256;

template <int D>
struct alignas(16) Smem {
    float S[D][D + 1];
    // (rows padded by four floats: the Gram products read 16 rows at one column across a wave, and
    // rows stay 16-byte aligned for 16-byte reads)
    float qm[C][D + 4], km[C][D + 4], kh[C][D + 4];  // sub-tile referenced factors
    float qg[C][D + 4], kg[C][D + 4], kb[C][D + 4];  // chunk-start / chunk-end referenced factors
    float w[C][D];                        // W = T Kg
    float u[C][D + 1];                    // U
    float vv[C][D];                       // the chunk's v rows (zeros past the end)
    float L[C][C + 1], A[C][C + 1], X[C][C + 1];
    float beta[C];
    float gamc[D];
};

template <int D>
__global__ void __launch_bounds__(NTHR, 1) kda_fwd_f32_kernel(Params p) {
    __shared__ Smem<D> sm;
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H;
    const size_t row0 = (size_t)b * p.tstride * p.H + h;  // (b*tstride + t)*H + h = row0 + t*H
    const float* q = (const float*)p.q;
    const float* k = (const float*)p.k;
    const float* v = (const float*)p.v;
    float* o = (float*)p.o;

    for (int e = tid; e < D * D; e += NTHR) {
        const int c = e / D, j = e % D;
        sm.S[c][j] = p.S0 ? p.S0[(size_t)bh * D * D + e] : 0.f;
    }
    const int nchunk = (p.T + C - 1) / C;
    for (int ch = 0; ch < nchunk; ++ch) {
        const int t0 = ch * C;
        const int n = min(C, p.T - t0);
        __syncthreads();
        // per-channel cumulative decay and the decay-scaled factors
        if (tid < D) {
            const int c = tid;
            float bcum[C];
            float a = 0.f;
            for (int r = 0; r < C; ++r) {
                const int tc = r < n ? t0 + r : p.T - 1;  // clamped: every address stays valid
                const float gv = p.g[(row0 + (size_t)tc * p.H) * D + c];
                const float gr = r < n ? gv : 0.f;
                a += gr;
                bcum[r] = a;
            }
            const float ref = bcum[7], last = bcum[C - 1];
            for (int r = 0; r < C; ++r) {
                const size_t idx = (row0 + (size_t)(r < n ? t0 + r : p.T - 1) * p.H) * D + c;
                const float qld = q[idx], kld = k[idx];
                const float qv = r < n ? qld : 0.f;
                const float kv = r < n ? kld : 0.f;
                const float e = fexp(bcum[r] - ref), rinv = fexp(ref - bcum[r]);
                sm.qm[r][c] = qv * e;
                sm.km[r][c] = kv * e;
                sm.kh[r][c] = kv * rinv;
                const float gam = fexp(bcum[r]);
                sm.qg[r][c] = qv * gam;
                sm.kg[r][c] = kv * gam;
                sm.kb[r][c] = kv * fexp(last - bcum[r]);
            }
            sm.gamc[c] = fexp(last);
        }
        if (tid < C) {
            const float bld = p.beta[row0 + (size_t)(tid < n ? t0 + tid : p.T - 1) * p.H];
            sm.beta[tid] = tid < n ? bld : 0.f;
        }
        {  // the chunk's v rows into LDS, every load of a thread in flight together
            constexpr int NV = C * D / NTHR;
            float vl[NV];
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const int e = tid + u * NTHR, r = e / D, j = e % D;
                vl[u] = v[(row0 + (size_t)(r < n ? t0 + r : p.T - 1) * p.H) * D + j];  // (clamped address)
            }
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const int e = tid + u * NTHR, r = e / D, j = e % D;
                sm.vv[r][j] = r < n ? vl[u] : 0.f;
            }
        }
        __syncthreads();
        // L (strictly lower) and A (lower with diagonal)
        {
            const int r = tid >> 4, s = tid & 15;
            float l = 0.f, a = 0.f;
            for (int c = 0; c < D; ++c) {
                l += sm.km[r][c] * sm.kh[s][c];
                a += sm.qm[r][c] * sm.kh[s][c];
            }
            sm.L[r][s] = s < r ? l : 0.f;
            sm.A[r][s] = s <= r ? a : 0.f;
        }
        __syncthreads();
        // X = (I + Diag(beta) L)^{-1} by forward substitution, one column per thread
        if (tid < C) {
            const int j = tid;
            float x[C];
            for (int i = 0; i < C; ++i) {
                float acc = (i == j) ? 1.f : 0.f;
                for (int m = 0; m < i; ++m) acc -= sm.beta[i] * sm.L[i][m] * x[m];
                x[i] = acc;
            }
            for (int i = 0; i < C; ++i) sm.X[i][j] = x[i] * sm.beta[j];  // T = X Diag(beta)
        }
        __syncthreads();
        // W = T Kg
        for (int e = tid; e < C * D; e += NTHR) {
            const int r = e / D, c = e % D;
            float w = 0.f;
            for (int s = 0; s <= r; ++s) w += sm.X[r][s] * sm.kg[s][c];
            sm.w[r][c] = w;
        }
        __syncthreads();
        // U = T V - W S.  Thread (column j, row group) takes the RB rows r = rg + k * RS of column j
        // together, so that each S[c][j] read from LDS serves all of them (every row's sum keeps its
        // own order).
        constexpr int RS = NTHR / D, RB = C / RS;  // row groups, rows per thread
        {
            const int j = tid % D, rg = tid / D;
            float u[RB];
#pragma unroll
            for (int k = 0; k < RB; ++k) {
                const int r = rg + k * RS;
                float a = 0.f;
                for (int s = 0; s <= r; ++s) a += sm.X[r][s] * sm.vv[s][j];
                u[k] = a;
            }
            for (int c = 0; c < D; ++c) {
                const float sc = sm.S[c][j];
#pragma unroll
                for (int k = 0; k < RB; ++k) u[k] -= sm.w[rg + k * RS][c] * sc;
            }
#pragma unroll
            for (int k = 0; k < RB; ++k) sm.u[rg + k * RS][j] = u[k];
        }
        __syncthreads();
        // O = Qg S + A U (skipped when o == NULL: a state-only run), rows grouped the same way
        if (o) {
            const int j = tid % D, rg = tid / D;
            float acc[RB];
#pragma unroll
            for (int k = 0; k < RB; ++k) acc[k] = 0.f;
            for (int c = 0; c < D; ++c) {
                const float sc = sm.S[c][j];
#pragma unroll
                for (int k = 0; k < RB; ++k) acc[k] += sm.qg[rg + k * RS][c] * sc;
            }
#pragma unroll
            for (int k = 0; k < RB; ++k) {
                const int r = rg + k * RS;
                for (int s = 0; s <= r; ++s) acc[k] += sm.A[r][s] * sm.u[s][j];
                if (r < n) o[(row0 + (size_t)(t0 + r) * p.H) * D + j] = acc[k] * p.scale;
            }
        }
        __syncthreads();
        // S <- Diag(Gamma_last) S + Kb^T U: thread (column j, row group) holds U's column j in
        // registers and updates rows cg, cg + RS, ... of it (entry tid + m * NTHR, m = 0, 1, ...)
        {
            const int j = tid % D, cg = tid / D;
            float uj[C];
#pragma unroll
            for (int s = 0; s < C; ++s) uj[s] = sm.u[s][j];
            for (int c = cg; c < D; c += RS) {
                float acc = sm.gamc[c] * sm.S[c][j];
#pragma unroll
                for (int s = 0; s < C; ++s) acc += sm.kb[s][c] * uj[s];
                sm.S[c][j] = acc;
            }
        }
        if (p.S_ckpt && (ch + 1) % p.ckpt_chunks == 0 && (ch + 1) / p.ckpt_chunks <= p.n_ckpt) {
            // the state after tokens [0, (ch+1)*C); each thread copies the entries it just wrote
            float* dst = p.S_ckpt + ((size_t)bh * p.n_ckpt + ((ch + 1) / p.ckpt_chunks - 1)) * D * D;
            for (int e = tid; e < D * D; e += NTHR) dst[e] = sm.S[e / D][e % D];
        }
    }
    __syncthreads();
    if (p.S_T)
        for (int e = tid; e < D * D; e += NTHR) p.S_T[(size_t)bh * D * D + e] = sm.S[e / D][e % D];
}

}  // namespace f32path

hipError_t launch_fwd_f32(const Params& p, hipStream_t stream) {
    const int nblk = p.B * p.H;
    if (p.Dk == 64)
        hipLaunchKernelGGL(f32path::kda_fwd_f32_kernel<64>, dim3(nblk), dim3(f32path::NTHR), 0, stream, p);
    else
        hipLaunchKernelGGL(f32path::kda_fwd_f32_kernel<128>, dim3(nblk), dim3(f32path::NTHR), 0, stream, p);
    return hipGetLastError();
}

// T = 0: the final state is the initial state (or zeros).
__global__ void kda_state_copy_kernel(const float* __restrict__ S0, float* __restrict__ S_T, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        S_T[i] = S0 ? S0[i] : 0.f;
}

hipError_t launch_state_copy(const Params& p, hipStream_t stream) {
    if (!p.S_T) return hipSuccess;
    const size_t n = (size_t)p.B * p.H * p.Dk * p.Dv;
    if (p.S0 == p.S_T) return hipSuccess;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(kda_state_copy_kernel, dim3(blocks), dim3(256), 0, stream, p.S0, p.S_T, n);
    return hipGetLastError();
}

}  // namespace kda
