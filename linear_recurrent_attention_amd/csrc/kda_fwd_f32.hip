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
    float gtot[NTHR / D][D];  // per token group: the sum of its tokens' decay logits
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
    // Thread (channel cc, token group tg) handles tokens tg*TG .. tg*TG + TG-1 of every chunk for the
    // decay sums and the factors.  A chunk's raw inputs (g, q, k of those tokens, the thread's share of
    // v, one beta) are loaded into registers during the chunk before it.
    constexpr int RS = NTHR / D, TG = C / RS, NV = C * D / NTHR;  // token groups, tokens per group
    static_assert(TG == 4 || TG == 8, "token 7 ends a token group");
    const int cc = tid % D, tg = tid / D;
    struct Raw { float g[TG], q[TG], k[TG], v[NV], beta; };
    auto load_raw = [&](int ch, Raw& R) {
        const int t0 = ch * C, n = min(C, p.T - t0);
#pragma unroll
        for (int i = 0; i < TG; ++i) {
            const int r = tg * TG + i;
            const size_t idx = (row0 + (size_t)(r < n ? t0 + r : p.T - 1) * p.H) * D + cc;  // (clamped address)
            R.g[i] = p.g[idx];
            R.q[i] = q[idx];
            R.k[i] = k[idx];
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const int e = tid + u * NTHR, r = e / D, j = e % D;
            R.v[u] = v[(row0 + (size_t)(r < n ? t0 + r : p.T - 1) * p.H) * D + j];
        }
        R.beta = tid < C ? p.beta[row0 + (size_t)(tid < n ? t0 + tid : p.T - 1) * p.H] : 0.f;
    };
    Raw cur, nxt;
    load_raw(0, cur);
    for (int ch = 0; ch < nchunk; ++ch) {
        const int t0 = ch * C;
        const int n = min(C, p.T - t0);
        __syncthreads();  // every read of the previous chunk's tiles is done
        if (ch + 1 < nchunk) load_raw(ch + 1, nxt);  // in flight during this chunk
        // decay sums within the token group, the chunk's v rows and beta
        float gl[TG];
        {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < TG; ++i) {
                a += tg * TG + i < n ? cur.g[i] : 0.f;
                gl[i] = a;
            }
            sm.gtot[tg][cc] = a;
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const int e = tid + u * NTHR, r = e / D, j = e % D;
                sm.vv[r][j] = r < n ? cur.v[u] : 0.f;
            }
            if (tid < C) sm.beta[tid] = tid < n ? cur.beta : 0.f;
        }
        __syncthreads();
        // cumulative decay b_r of the thread's tokens, relative to token 7 (ref) and to the chunk's
        // end (last), and the decay-scaled factors
        {
            float off = 0.f;
            for (int g2 = 0; g2 < tg; ++g2) off += sm.gtot[g2][cc];
            float ref = 0.f, last = 0.f;
            for (int g2 = 0; g2 < RS; ++g2) {
                last += sm.gtot[g2][cc];
                if (g2 == 7 / TG) ref = last;  // token 7 ends its group
            }
#pragma unroll
            for (int i = 0; i < TG; ++i) {
                const int r = tg * TG + i;
                const float b = off + gl[i];
                const float qv = r < n ? cur.q[i] : 0.f, kv = r < n ? cur.k[i] : 0.f;
                const float e = fexp(b - ref), rinv = fexp(ref - b);
                sm.qm[r][cc] = qv * e;
                sm.km[r][cc] = kv * e;
                sm.kh[r][cc] = kv * rinv;
                const float gam = fexp(b);
                sm.qg[r][cc] = qv * gam;
                sm.kg[r][cc] = kv * gam;
                sm.kb[r][cc] = kv * fexp(last - b);
            }
            if (tg == 0) sm.gamc[cc] = fexp(last);
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
        constexpr int RB = C / RS;  // rows per thread (RS row groups)
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
        cur = nxt;
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
