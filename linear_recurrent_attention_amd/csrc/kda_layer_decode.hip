// Decode step of the fused KDA layer, with a projection-input cache for speculative decoding, on gfx950.
//
// The explainer page "Kimi K3：开放前沿智能", section 13.10, lists a KDA decode kernel that does the
// projections, the state update and the attention readout of a new token in one fused call, with a
// cache of projection inputs; section 13.4 gives the reason for the cache: decoding updates the state
// in place, so when speculative decoding rejects draft tokens the state before them is gone, and
// keeping each token's projection inputs is far cheaper than keeping a state per token.
//
// Reading of the pages used here.  A call takes T new tokens of B sequences (M = B*T <= 16 rows) and
// runs the whole layer on them (the same operations as kda_layer_fwd): projections, short convolution
// + SiLU + L2 norm, decay gate, beta, the gated delta rule from the given state, readout, RMSNorm,
// output gate, output projection.  The cache entry of a token is what advancing the state and the
// convolution window needs and what the projections produced: k, v, g (log decay), beta after the
// gates, and the pre-convolution q and k rows, 5*H*D + H floats per token, against H*D*D floats for
// a state.  In speculative mode (KDA_DECODE_SPECULATIVE) the state and the window are read but not
// written, every draft token's entry goes to the cache, and its output is computed as if the drafts
// before it were accepted; kda_layer_decode_commit then advances the state and the window over the
// accepted tokens from their entries, without touching the projections again.
//
// One cooperative launch (every workgroup resident) in phases separated by grid barriers:
//   1. the input projections of the M rows (q, k, v, gate, decay-down, beta weights, as given,
//      [in][out]): work items of 1024 columns x 64 rows of the weight, partial sums per item, then
//      (after a barrier) the sums of the partials, one projected row per token;
//   2. one workgroup per (sequence, head): reads its columns of the projected rows, the decay
//      up-projection of its head, convolution window, gates, then the recurrence token by token
//      with the state in registers (thread (column j, half r) holds rows 64r..64r+63 of column j),
//      readout, RMSNorm and gate; writes the gated output rows, the cache entries and (unless
//      speculative) the state and window;
//   3. the output projection of the gated rows, partial sums per item of 16 weight rows;
//   4. the sum of those partials, to bf16 y.
// The weights are read once per call, so with a few rows the call is bound by reading them and the
// state; the products are plain float32 FMAs with the rows of x staged in LDS.
#include <hip/hip_cooperative_groups.h>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace ldec {

namespace cg = cooperative_groups;

constexpr int D = 128;
constexpr int NTHR = 256;
constexpr int KSL1 = 64;   // weight rows per input-projection work item
constexpr int KSL3 = 16;   // weight rows per output-projection work item
constexpr int KMAX = 64;
constexpr int CB = 1024;  // weight columns per projection work item (four per thread)
constexpr float EPS = 1e-6f;

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + fexp(-x)); }

// Sum over the 128 threads 0..127 (two waves) of v; every one of them gets the total.  red: 2 floats.
__device__ __forceinline__ float sum128(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int tid = threadIdx.x;
    __syncthreads();  // earlier readers of red are done
    if (tid == 0 || tid == 64) red[tid >> 6] = v;
    __syncthreads();
    return red[0] + red[1];
}

// part[(ks * M + m) * ldp + off + n] = sum over rows k of slice ks of in(m, k) * W[k][n], for the
// four columns n .. n + 3 of each thread.  ROWS: M rounded up to a supported count.  The weight rows
// are loaded sixteen at a time before they are used, so that each thread keeps sixteen loads in flight.
template <int ROWS, typename In>
__device__ void gemv_item(const uint16_t* W_, int nw, bool quad_ok, int k0, int kn, int cb, int M, In in,
                          float (*xs)[16], float* __restrict__ part, int ks, int ldp, int off) {
    typedef __attribute__((address_space(1))) const uint16_t g16;
    typedef __attribute__((address_space(1))) const u32x2 g32x2;
    g16* W = (g16*)(W_);  // the weights are global memory
    const int tid = threadIdx.x;
    __syncthreads();  // the previous item's reads of xs are done
    for (int e = tid; e < KMAX * 16; e += NTHR) {
        const int kk = e >> 4, m = e & 15;
        xs[kk][m] = (m < M && kk < kn) ? in(m, k0 + kk) : 0.f;
    }
    __syncthreads();
    const int n = cb * CB + 4 * tid;
    if (n >= nw) return;
    float acc[ROWS][4];
#pragma unroll
    for (int m = 0; m < ROWS; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = 0.f;
#define KDA_FMA_ROW(kk, w0, w1, w2, w3)                             \
    _Pragma("unroll") for (int m = 0; m < ROWS; ++m) {              \
        const float xv = xs[kk][m];                                 \
        acc[m][0] = __builtin_fmaf(xv, (w0), acc[m][0]);            \
        acc[m][1] = __builtin_fmaf(xv, (w1), acc[m][1]);            \
        acc[m][2] = __builtin_fmaf(xv, (w2), acc[m][2]);            \
        acc[m][3] = __builtin_fmaf(xv, (w3), acc[m][3]);            \
    }
    if (quad_ok && n + 3 < nw) {
        // four whole columns: 8-byte loads, sixteen rows in flight
        g16* wp = W + (size_t)k0 * nw + n;
        for (int kb = 0; kb < kn; kb += 16) {
            u32x2 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = *reinterpret_cast<g32x2*>(wp + (size_t)min(kb + u, kn - 1) * nw);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (kb + u < kn) {
                    const float w0 = __uint_as_float(v[u][0] << 16), w1 = __uint_as_float(v[u][0] & 0xffff0000u);
                    const float w2 = __uint_as_float(v[u][1] << 16), w3 = __uint_as_float(v[u][1] & 0xffff0000u);
                    KDA_FMA_ROW(kb + u, w0, w1, w2, w3)
                }
            }
        }
    } else {
        // the ragged edge (or an unaligned matrix): element loads
        for (int kk = 0; kk < kn; ++kk) {
            g16* r = W + (size_t)(k0 + kk) * nw + n;
            const float w0 = bf(r[0]), w1 = n + 1 < nw ? bf(r[1]) : 0.f;
            const float w2 = n + 2 < nw ? bf(r[2]) : 0.f, w3 = n + 3 < nw ? bf(r[3]) : 0.f;
            KDA_FMA_ROW(kk, w0, w1, w2, w3)
        }
    }
#undef KDA_FMA_ROW
#pragma unroll
    for (int m = 0; m < ROWS; ++m) {
        if (m < M) {
            float* dst = part + ((size_t)ks * M + m) * ldp + off + n;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (n + c < nw) dst[c] = acc[m][c];
        }
    }
}

template <typename In>
__device__ void gemv_dispatch(const uint16_t* W, int nw, bool quad_ok, int k0, int kn, int cb, int M, In in,
                              float (*xs)[16], float* part, int ks, int ldp, int off) {
    if (M <= 1) gemv_item<1>(W, nw, quad_ok, k0, kn, cb, M, in, xs, part, ks, ldp, off);
    else if (M <= 2) gemv_item<2>(W, nw, quad_ok, k0, kn, cb, M, in, xs, part, ks, ldp, off);
    else if (M <= 4) gemv_item<4>(W, nw, quad_ok, k0, kn, cb, M, in, xs, part, ks, ldp, off);
    else if (M <= 8) gemv_item<8>(W, nw, quad_ok, k0, kn, cb, M, in, xs, part, ks, ldp, off);
    else gemv_item<16>(W, nw, quad_ok, k0, kn, cb, M, in, xs, part, ks, ldp, off);
}

// dst[e .. e+3] = sum over ks < nks of src[ks * stride + e .. +3] for every e = 4i < n (n and stride
// multiples of 4), grid-stride; the slices are read sixteen at a time, all in flight together
template <typename Store>
__device__ __forceinline__ void sum_slices4(const float* __restrict__ src, size_t stride, int nks, long n, Store st) {
    for (long e = 4 * ((long)blockIdx.x * blockDim.x + threadIdx.x); e < n; e += 4L * gridDim.x * blockDim.x) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < nks; k0 += 16) {
            f32x4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                v[u] = k0 + u < nks ? *reinterpret_cast<const f32x4*>(src + (size_t)(k0 + u) * stride + e)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 16; ++u) a += v[u];
        }
        st(e, a);
    }
}

struct Smem {
    float xs[KMAX][16];
    uint16_t wup[128][D];  // the decay up-projection's columns of this head (rank <= 128)
    float qp[D], kp[D], vv[D], gl[D], q[D], k[D], ga[D], dn[128];
    float cw[2][3][D];  // convolution window of this head: [q/k][oldest..newest][channel]
    float pw[2][D], po[2][D];
    float red[2];
    float beta;
};

__global__ void __launch_bounds__(NTHR) kda_layer_decode_kernel(LayerDecodeParams p) {
    __shared__ Smem sm;
    cg::grid_group grid = cg::this_grid();
    const int tid = threadIdx.x;
    const int M = p.B * p.T, HD = p.H * D, dm = p.dm, R = p.R;
    const int ntot = (p.noff[6] + 3) & ~3;  // row length of the partial sums and projected rows

    // ---------------- 1. input projections: partial sums over slices of KSL1 weight rows
    const int nks1 = (dm + KSL1 - 1) / KSL1;
    {
        int items = 0;
        for (int i = 0; i < 6; ++i) items += ((p.wn[i] + CB - 1) / CB) * nks1;
        auto xin = [&](int m, int k) { return bf(p.x[(size_t)m * dm + k]); };
        for (int it = blockIdx.x; it < items; it += gridDim.x) {
            int i = 0, rem = it;
            while (rem >= ((p.wn[i] + CB - 1) / CB) * nks1) { rem -= ((p.wn[i] + CB - 1) / CB) * nks1; ++i; }
            const int cb = rem / nks1, ks = rem - cb * nks1;
            const int k0 = ks * KSL1, kn = min(KSL1, dm - k0);
            const bool quad_ok = (p.wn[i] & 3) == 0 && (reinterpret_cast<uintptr_t>(p.W[i]) & 7) == 0;
            gemv_dispatch(p.W[i], p.wn[i], quad_ok, k0, kn, cb, M, xin, sm.xs, p.part, ks, ntot, p.noff[i]);
        }
    }
    grid.sync();
    // ---------------- 1b. the projected rows: sums of the slices' partials
    sum_slices4(p.part, (size_t)M * ntot, nks1, (long)M * ntot,
                [&](long e, f32x4 a) { *reinterpret_cast<f32x4*>(p.proj + e) = a; });
    grid.sync();

    // ---------------- 2. per (sequence, head): gates, convolution, recurrence, readout, norm
    for (int bh = blockIdx.x; bh < p.B * p.H; bh += gridDim.x) {
        const int b = bh / p.H, h = bh - b * p.H;
        const int j = tid & (D - 1), rh = tid >> 7;  // state column, row half
        float s[64];
        {
            const float* Sb = p.S + (size_t)bh * D * D + (size_t)(64 * rh) * D + j;
#pragma unroll
            for (int i = 0; i < 64; ++i) s[i] = p.S ? Sb[(size_t)i * D] : 0.f;
        }
        for (int e = tid; e < 2 * 3 * D; e += NTHR) {
            const int qk = e / (3 * D), r = (e / D) % 3, c = e % D;
            sm.cw[qk][r][c] = p.conv ? p.conv[((size_t)b * 3 + r) * 2 * HD + qk * HD + h * D + c] : 0.f;
        }
        const float ea = fexp(p.A[h]);
        // this head's columns of the decay up-projection, 16 bytes per load
        if ((reinterpret_cast<uintptr_t>(p.Wup) & 15) == 0) {
            for (int e = tid; e < R * (D / 8); e += NTHR) {
                const int r = e >> 4, c8 = 8 * (e & 15);
                *reinterpret_cast<u32x4*>(&sm.wup[r][c8]) =
                    *reinterpret_cast<const u32x4*>(p.Wup + (size_t)r * HD + h * D + c8);
            }
        } else {
            for (int e = tid; e < R * D; e += NTHR) sm.wup[e >> 7][e & 127] = p.Wup[(size_t)(e >> 7) * HD + h * D + (e & 127)];
        }
        for (int t = 0; t < p.T; ++t) {
            const int m = b * p.T + t;
            __syncthreads();  // every read of the previous token's rows (and of the window) is done
            // this token's projected row: q, k (threads 0-127), v, gate (128-255); decay-down; beta
            {
                const float* pr = p.proj + (size_t)m * ntot;
                const int c = j, base = rh ? 2 * HD : 0;
                const float a = pr[base + h * D + c], bb = pr[base + HD + h * D + c];
                if (rh == 0) { sm.qp[c] = a; sm.kp[c] = bb; } else { sm.vv[c] = a; sm.gl[c] = bb; }
                for (int r = tid; r < R; r += NTHR) sm.dn[r] = pr[4 * HD + r];
                if (tid == NTHR - 1) sm.beta = sigm(pr[4 * HD + R + h]);
            }
            __syncthreads();
            // short convolution + SiLU of q (threads 0-127) and k (128-255); decay gate (0-127)
            float act;
            {
                const int c = j, hc = h * D + c;
                const float* taps = (rh ? p.conv_k : p.conv_q) + (size_t)hc * 4;
                const float xcur = rh ? sm.kp[c] : sm.qp[c];
                const float y = taps[0] * sm.cw[rh][0][c] + taps[1] * sm.cw[rh][1][c] + taps[2] * sm.cw[rh][2][c] +
                                taps[3] * xcur;
                act = y * sigm(y);
                if (rh == 0) {
                    float z[4] = {p.b_alpha[hc], 0.f, 0.f, 0.f};
                    int r = 0;
                    for (; r + 4 <= R; r += 4) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) z[u] = __builtin_fmaf(sm.dn[r + u], bf(sm.wup[r + u][c]), z[u]);
                    }
                    for (; r < R; ++r) z[0] = __builtin_fmaf(sm.dn[r], bf(sm.wup[r][c]), z[0]);
                    sm.ga[c] = -5.f * sigm(ea * ((z[0] + z[1]) + (z[2] + z[3])));
                }
            }
            // L2 norms: q over threads 0-127, k over 128-255 (each half sums its own two waves)
            {
                float v = act * act;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
                __syncthreads();
                if ((tid & 63) == 0) sm.pw[0][tid >> 6] = v;
                __syncthreads();
                const float ss = rh ? sm.pw[0][2] + sm.pw[0][3] : sm.pw[0][0] + sm.pw[0][1];
                const float nv = act / sqrtf(ss + EPS);
                if (rh == 0) sm.q[j] = nv; else sm.k[j] = nv;
            }
            // cache entry of this token (before the window moves): k, v, g, beta, pre-conv q and k rows
            if (p.cache) {
                const size_t tok = (size_t)b * p.T + t, stride = (size_t)p.B * p.T;
                float* cbase = p.cache;
                __syncthreads();
                if (rh == 0) {
                    cbase[tok * HD + h * D + j] = sm.k[j];                       // k
                    cbase[(stride + tok) * HD + h * D + j] = sm.vv[j];           // v
                    cbase[(2 * stride + tok) * HD + h * D + j] = sm.ga[j];       // g
                    cbase[3 * stride * HD + (size_t)p.H * stride + tok * HD + h * D + j] = sm.qp[j];   // pre-conv q
                } else {
                    cbase[4 * stride * HD + (size_t)p.H * stride + tok * HD + h * D + j] = sm.kp[j];   // pre-conv k
                }
                if (tid == 0) cbase[3 * stride * HD + tok * p.H + h] = sm.beta;  // beta
            }
            __syncthreads();
            // move the window: newest pre-conv row in
            {
                const float xcur = rh ? sm.kp[j] : sm.qp[j];
                const float w1 = sm.cw[rh][1][j], w2 = sm.cw[rh][2][j];
                __syncthreads();
                sm.cw[rh][0][j] = w1;
                sm.cw[rh][1][j] = w2;
                sm.cw[rh][2][j] = xcur;
            }
            // the gated delta rule for this token: decay, w = S^T k, S += beta k (v - w)^T, o = S^T q
            float w = 0.f;
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                s[i] *= fexp(sm.ga[64 * rh + i]);
                w = __builtin_fmaf(s[i], sm.k[64 * rh + i], w);
            }
            sm.pw[rh][j] = w;
            __syncthreads();
            const float u = sm.beta * (sm.vv[j] - (sm.pw[0][j] + sm.pw[1][j]));
            float o = 0.f;
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                s[i] = __builtin_fmaf(sm.k[64 * rh + i], u, s[i]);
                o = __builtin_fmaf(s[i], sm.q[64 * rh + i], o);
            }
            sm.po[rh][j] = o;
            __syncthreads();
            // RMSNorm over the head's 128 outputs, times rms_w and the output gate
            {
                const float ot = (sm.po[0][j] + sm.po[1][j]) * p.scale;
                const float ss = sum128(rh == 0 ? ot * ot : 0.f, sm.red);
                if (rh == 0) {
                    const float on = ot / sqrtf(ss * (1.f / D) + EPS) * p.rms_w[j] * sigm(sm.gl[j]);
                    p.gated[(size_t)m * HD + h * D + j] = on;
                }
            }
        }
        if (!p.spec) {
            float* Sb = p.S + (size_t)bh * D * D + (size_t)(64 * rh) * D + j;
#pragma unroll
            for (int i = 0; i < 64; ++i) Sb[(size_t)i * D] = s[i];
            if (p.conv) {
                __syncthreads();
                for (int e = tid; e < 2 * 3 * D; e += NTHR) {
                    const int qk = e / (3 * D), r = (e / D) % 3, c = e % D;
                    p.conv[((size_t)b * 3 + r) * 2 * HD + qk * HD + h * D + c] = sm.cw[qk][r][c];
                }
            }
        }
        __syncthreads();  // the next (sequence, head) rewrites the shared arrays
    }
    grid.sync();

    // ---------------- 3. output projection of the gated rows: partial sums over slices of KSL3 rows
    const int nks3 = (HD + KSL3 - 1) / KSL3;
    {
        const int items = ((dm + CB - 1) / CB) * nks3;
        auto gin = [&](int m, int k) { return p.gated[(size_t)m * HD + k]; };
        const bool quad_ok = (dm & 3) == 0 && (reinterpret_cast<uintptr_t>(p.Wo) & 7) == 0;
        for (int it = blockIdx.x; it < items; it += gridDim.x) {
            const int cb = it / nks3, ks = it - cb * nks3;
            const int k0 = ks * KSL3, kn = min(KSL3, HD - k0);
            gemv_dispatch(p.Wo, dm, quad_ok, k0, kn, cb, M, gin, sm.xs, p.part, ks, dm, 0);
        }
    }
    grid.sync();

    // ---------------- 4. y = bf16(sum of the partials)
    sum_slices4(p.part, (size_t)M * dm, nks3, (long)M * dm, [&](long e, f32x4 a) {
        *reinterpret_cast<u32x2*>(p.y + e) = u32x2{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])};
    });
}

// Advance the convolution window over the first n tokens of the cache: the last 3 of
// [window rows, pre-conv rows of tokens 0..n-1].
__global__ void window_commit_kernel(float* __restrict__ conv, const float* __restrict__ qpre,
                                     const float* __restrict__ kpre, int B, int T, int HD, int n) {
    const long total = (long)B * 2 * HD;
    for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
        const int ch = (int)(e % (2 * HD));
        const int b = (int)(e / (2 * HD));
        const int qk = ch / HD, c = ch % HD;
        const float* pre = qk ? kpre : qpre;
        float w[3];
        for (int r = 0; r < 3; ++r) w[r] = conv[((size_t)b * 3 + r) * 2 * HD + ch];
        float out[3];
        for (int r = 0; r < 3; ++r) {
            const int src = n - 3 + r;  // index into [window (as -3..-1), tokens 0..n-1]
            out[r] = src >= 0 ? pre[((size_t)b * T + src) * HD + c] : w[3 + src];
        }
        for (int r = 0; r < 3; ++r) conv[((size_t)b * 3 + r) * 2 * HD + ch] = out[r];
    }
}

}  // namespace ldec

size_t layer_decode_part_floats(int M, int dm, int HD, int ntot) {
    const size_t a = (size_t)((dm + ldec::KSL1 - 1) / ldec::KSL1) * M * ntot;
    const size_t b = (size_t)((HD + ldec::KSL3 - 1) / ldec::KSL3) * M * dm;
    return a > b ? a : b;
}

hipError_t launch_layer_decode(const LayerDecodeParams& p, hipStream_t stream) {
    int dev = 0, ncu = 0, occ = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(ldec::kda_layer_decode_kernel),
                                                         ldec::NTHR, 0);
    if (e != hipSuccess) return e;
    if (occ < 1 || ncu < 1) return hipErrorLaunchFailure;
    // one workgroup per compute unit, all resident: every workgroup's barrier fences write back and
    // invalidate its XCD's L2, so more workgroups per XCD make each grid barrier dearer
    const dim3 grid((unsigned)ncu), block(ldec::NTHR);
    LayerDecodeParams pc = p;
    void* args[] = {&pc};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(ldec::kda_layer_decode_kernel), grid, block, args,
                                      0, stream);
}

hipError_t launch_window_commit(float* conv, const float* qpre, const float* kpre, int B, int T, int HD, int n,
                                hipStream_t stream) {
    const long total = (long)B * 2 * HD;
    const unsigned blocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(ldec::window_commit_kernel, dim3(blocks), dim3(256), 0, stream, conv, qpre, kpre, B, T, HD, n);
    return hipGetLastError();
}

}  // namespace kda
