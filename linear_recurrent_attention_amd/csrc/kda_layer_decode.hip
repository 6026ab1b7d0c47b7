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
// Four launches:
//   1. ldec_proj_kernel: the input projections of the M rows (q, k, v, gate, decay-down, beta weights,
//      as given, [in][out]): one workgroup of 16 waves per (64 columns of one weight, half of the
//      input rows; a sixteenth for the narrow decay-down and beta weights, so that those add short
//      workgroups rather than a second round), one column per lane, the rows of x staged in LDS; the
//      16 waves' sums meet in LDS;
//   2. ldec_head_kernel, one workgroup per (sequence, head): its columns of the projected rows (the
//      partials' sums), the decay up-projection of its head, convolution window, gates, then the
//      recurrence token by token with the state in registers (thread (column j, half r) holds rows
//      64r..64r+63 of column j), readout, RMSNorm and gate; writes the gated output rows, the cache
//      entries and (unless speculative) the state and window;
//   3. ldec_proj_kernel over the output projection of the gated rows: 64 columns x one eighth of the
//      rows per workgroup;
//   4. the sum of those eight partials, to bf16 y.
// The weights are read once per call, so with a few rows the call is bound by reading them and the
// state; the products are plain float32 FMAs.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace ldec {

constexpr int D = 128;
constexpr int NTHR = 256;
constexpr int MW = 8;        // waves of a projection workgroup
constexpr int MT = 64 * MW;  // its threads
constexpr int MCOLS = 128;   // weight columns per projection workgroup: 8 per lane, 16 lanes
constexpr int KS1 = 3;       // splits of the input rows: input projections (66 x 3 workgroups at H = 16)
constexpr int KS3 = 8;       // splits of the input rows: output projection
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

// Rows k..k+7, columns n..n+7 of a [K][nw] bf16 weight as eight 16-byte rows (zeros past row k1 or
// column nw).  vec: 16-byte loads (nw a multiple of 8, W 16-byte aligned).
__device__ __forceinline__ void load_w8(const uint16_t* __restrict__ W, int nw, int k1, int k, int n, bool vec,
                                        u32x4 (&r)[8]) {
    if (vec && n + 8 <= nw) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            r[i] = u32x4{0u, 0u, 0u, 0u};
            if (k + i < k1) r[i] = *reinterpret_cast<const u32x4*>(W + (size_t)(k + i) * nw + n);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t w[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) w[c] = k + i < k1 && n + c < nw ? W[(size_t)(k + i) * nw + n + c] : 0u;
            r[i] = u32x4{w[0] | w[1] << 16, w[2] | w[3] << 16, w[4] | w[5] << 16, w[6] | w[7] << 16};
        }
    }
}

// Column c of an 8 x 8 bf16 block held as eight rows: its eight elements in row order, two per word
// (the operand layout of one lane of a 16x16x32 product: contraction indices 8g .. 8g+7).
template <int c>
__device__ __forceinline__ u32x4 col8(const u32x4 (&r)[8]) {
    u32x4 o;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
        const uint32_t a = r[2 * kp][c >> 1], b = r[2 * kp + 1][c >> 1];
        o[kp] = (c & 1) ? (a >> 16) | (b & 0xffff0000u) : (a & 0xffffu) | (b << 16);
    }
    return o;
}

// Elements k..k+7 of row m of x (zeros past column k1 or row M): bf16 x as is; float32 x as bf16
// hi + lo halves (x = hi + lo to about 2^-17 relative).
__device__ __forceinline__ void load_x8(const uint16_t* __restrict__ x, int ldx, int M, int k1, int m, int k,
                                        bool vec, u32x4& hi, u32x4&) {
    hi = u32x4{0u, 0u, 0u, 0u};
    if (m >= M) return;
    if (vec && k + 8 <= k1) {
        hi = *reinterpret_cast<const u32x4*>(x + (size_t)m * ldx + k);
    } else {
        uint32_t w[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) w[c] = k + c < k1 ? x[(size_t)m * ldx + k + c] : 0u;
        hi = u32x4{w[0] | w[1] << 16, w[2] | w[3] << 16, w[4] | w[5] << 16, w[6] | w[7] << 16};
    }
}
__device__ __forceinline__ void load_x8(const float* __restrict__ x, int ldx, int M, int k1, int m, int k, bool vec,
                                        u32x4& hi, u32x4& lo) {
    float v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = 0.f;
    if (m < M) {
        if (vec && k + 8 <= k1) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(x + (size_t)m * ldx + k);
            const f32x4 b = *reinterpret_cast<const f32x4*>(x + (size_t)m * ldx + k + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) { v[c] = a[c]; v[4 + c] = b[c]; }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) v[c] = k + c < k1 ? x[(size_t)m * ldx + k + c] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t h, l;
        split_bf16(v[2 * i], v[2 * i + 1], h, l);
        hi[i] = h;
        lo[i] = l;
    }
}

// part[m * ldp + col0 + c] = sum over k in [k0, k1) of x[m][k] * W[k][n0 + c] for c < 128 with
// n0 + c < nw, m < M (M <= 16), on the matrix cores (16x16x32 bf16, float32 sums).  Lane (l16, g)
// of a wave reads weight rows k + 8g .. k + 8g + 7, columns n0 + 8 l16 .. + 7 (one 16-byte load per
// row, coalesced along the rows) for each 32-row step k, and transposes that 8 x 8 block in
// registers into the operands of eight products, product c covering columns n0 + 8j + c (j < 16),
// with x's rows as the other operand; a float32 x takes two products, its bf16 hi and lo halves.
// Wave w takes the steps w, w + 8, ..., NB at a time in flight; the waves' sums meet in LDS and
// are added in wave order.  red: [8][16][128] floats.
template <int NB, typename X>
__device__ void mproj_block(const uint16_t* __restrict__ W, int nw, int n0, int k0, int k1, int M,
                            const X* __restrict__ x, int ldx, float* red, float* __restrict__ part, int ldp, int col0) {
    constexpr bool XF32 = sizeof(X) == 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;
    const int n = n0 + 8 * l16;
    const bool wvec = (nw & 7) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
    const bool xvec = (ldx & 7) == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0;
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const u32x4 (&r)[8], u32x4 xh, u32x4 xl) {  // columns in word order, so that the
        auto one = [&](auto cc) {                                     // rows' words die as they are used
            constexpr int c = decltype(cc)::value;
            const u32x4 b = col8<c>(r);
            acc[c] = mfma_bf16(xh, b, acc[c]);
            if constexpr (XF32) acc[c] = mfma_bf16(xl, b, acc[c]);
        };
        one(std::integral_constant<int, 0>{}); one(std::integral_constant<int, 1>{});
        one(std::integral_constant<int, 2>{}); one(std::integral_constant<int, 3>{});
        one(std::integral_constant<int, 4>{}); one(std::integral_constant<int, 5>{});
        one(std::integral_constant<int, 6>{}); one(std::integral_constant<int, 7>{});
    };
    const int nsteps = (k1 - k0 + 31) / 32;
    for (int s0 = wave; s0 < nsteps; s0 += NB * MW) {
        u32x4 r[NB][8], xh[NB], xl[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (s0 + u * MW < nsteps) load_w8(W, nw, k1, k0 + 32 * (s0 + u * MW) + 8 * g, n, wvec, r[u]);  // (wave-uniform)
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (s0 + u * MW < nsteps) load_x8(x, ldx, M, k1, l16, k0 + 32 * (s0 + u * MW) + 8 * g, xvec, xh[u], xl[u]);
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (s0 + u * MW < nsteps) step(r[u], xh[u], xl[u]);
    }
    // lane (l16, g) holds rows 4g .. 4g+3 (element e of each product), columns n0 + 8 l16 + c
    float* rw = red + wave * (16 * MCOLS);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float* row = rw + (4 * g + e) * MCOLS + 8 * l16;
        *reinterpret_cast<f32x4*>(row) = f32x4{acc[0][e], acc[1][e], acc[2][e], acc[3][e]};
        *reinterpret_cast<f32x4*>(row + 4) = f32x4{acc[4][e], acc[5][e], acc[6][e], acc[7][e]};
    }
    __syncthreads();
    const int m = tid >> 5, c4 = 4 * (tid & 31);  // thread: row m, columns c4 .. c4+3
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < MW; ++w) v += *reinterpret_cast<const f32x4*>(red + (w * 16 + m) * MCOLS + c4);
    if (m < M) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n0 + c4 + e < nw) part[(size_t)m * ldp + col0 + c4 + e] = v[e];
    }
}
static_assert(MT == 16 * (MCOLS / 4), "one thread per (row, 4 columns) in the reduction");

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

struct alignas(16) Smem {
    uint16_t wupT[D][128 + 8];  // this head's columns of the decay up-projection, channel-major (rank
                                // <= 128, zeros past R; rows padded so 16-byte reads spread over banks)
    float qp[D], kp[D], vv[D], gl[D], q[D], k[D], ga[D], ega[D], dn[128];
    float zp[2][D];  // the decay logit's two half-sums over the rank
    float cw[2][3][D];  // convolution window of this head: [q/k][oldest..newest][channel]
    float pw[2][D], po[2][D];
    float red[2];
    float beta;
};

// Column blocks of weight i of the input projections.
__device__ __forceinline__ int nblk(const LayerDecodeParams& p, int i) { return (p.wn[i] + MCOLS - 1) / MCOLS; }

// Rows of x per split of k: a multiple of the 32-row step
__host__ __device__ __forceinline__ int split_rows(int K, int nks) { return ((K + nks - 1) / nks + 31) & ~31; }

// 1. the input projections: workgroup (column block of weight i, row split ks) -> part[ks][m][column]
__global__ void __launch_bounds__(MT) ldec_proj_kernel(LayerDecodeParams p) {
    __shared__ float red[MW * 16 * MCOLS];
    const int M = p.B * p.T, dm = p.dm;
    const int ntot = (p.noff[6] + 3) & ~3;  // row length of the partial sums
    int blk = blockIdx.x / KS1, i = 0;
    const int ks = blockIdx.x - blk * KS1;
    while (i < 5 && blk >= nblk(p, i)) { blk -= nblk(p, i); ++i; }  // (workgroup-uniform)
    const int kper = split_rows(dm, KS1), k0 = min(dm, ks * kper), k1 = min(dm, k0 + kper);
    mproj_block<3>(p.W[i], p.wn[i], MCOLS * blk, k0, k1, M, p.x, dm, red, p.part + (size_t)ks * M * ntot, ntot,
                p.noff[i] + MCOLS * blk);
}

// 3. the output projection of the gated rows: workgroup (column block, row split ks) -> part[ks][m][column]
__global__ void __launch_bounds__(MT) ldec_out_kernel(LayerDecodeParams p) {
    __shared__ float red[MW * 16 * MCOLS];
    const int M = p.B * p.T, dm = p.dm, HD = p.H * D;
    const int blk = blockIdx.x / KS3, ks = blockIdx.x - blk * KS3;
    const int kper = split_rows(HD, KS3), k0 = min(HD, ks * kper), k1 = min(HD, k0 + kper);
    mproj_block<1>(p.Wo, dm, MCOLS * blk, k0, k1, M, p.gated, HD, red, p.part + (size_t)ks * M * dm, dm, MCOLS * blk);
}

// 4. y = bf16(sum of the output projection's partials, in split order)
__global__ void ldec_sum_kernel(LayerDecodeParams p) {
    const int M = p.B * p.T, dm = p.dm;
    sum_slices4(p.part, (size_t)M * dm, KS3, (long)M * dm, [&](long e, f32x4 a) {
        *reinterpret_cast<u32x2*>(p.y + e) = u32x2{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3])};
    });
}

// 2. per (sequence, head): gates, convolution, recurrence, readout, norm
__global__ void __launch_bounds__(NTHR) ldec_head_kernel(LayerDecodeParams p) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int M = p.B * p.T, HD = p.H * D, R = p.R;
    const int ntot = (p.noff[6] + 3) & ~3;
    // the projected rows: the sums of the input projection's KS1 row-split partials, in split order,
    // all loads issued together
    auto proj = [&](int m, int col) {
        float v[KS1];
#pragma unroll
        for (int s = 0; s < KS1; ++s) v[s] = p.part[((size_t)s * M + m) * ntot + col];
        float r = 0.f;
#pragma unroll
        for (int s = 0; s < KS1; ++s) r += v[s];
        return r;
    };
    for (int bh = blockIdx.x; bh < p.B * p.H; bh += gridDim.x) {
        const int b = bh / p.H, h = bh - b * p.H;
        const int j = tid & (D - 1), rh = tid >> 7;  // state column, row half
        const int hc = h * D + j;
        // Every global load that does not depend on the token is issued here, together, so that the
        // head pays about one memory round trip before its first token: this thread's convolution taps,
        // decay bias and RMSNorm weight, the state, the window, the up-projection's columns of this
        // head, and the first token's projected values.
        float taps[4];
        {
            const float* tp = (rh ? p.conv_k : p.conv_q) + (size_t)hc * 4;
#pragma unroll
            for (int u = 0; u < 4; ++u) taps[u] = tp[u];
        }
        const float balpha = rh == 0 ? p.b_alpha[hc] : 0.f;
        const float rw = p.rms_w[j];
        const float ea = fexp(p.A[h]);
        float s[64];
        {
            const float* Sb = p.S + (size_t)bh * D * D + (size_t)(64 * rh) * D + j;
#pragma unroll
            for (int i = 0; i < 64; ++i) s[i] = p.S ? Sb[(size_t)i * D] : 0.f;
        }
        float cwv[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int e = tid + u * NTHR, qk = e / (3 * D), r = (e / D) % 3, c = e % D;
            cwv[u] = p.conv ? p.conv[((size_t)b * 3 + r) * 2 * HD + qk * HD + h * D + c] : 0.f;
        }
        static_assert(2 * 3 * D == 3 * NTHR, "three window values per thread");
        // the up-projection's 8 x 8 block (ranks 8rb.., channels 8cb..) of thread (rb, cb), 16-byte loads
        const bool wal = (reinterpret_cast<uintptr_t>(p.Wup) & 15) == 0;
        const int rb = tid >> 4, cb = tid & 15;
        u32x4 wv[8];
        if (wal) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                wv[i] = u32x4{0u, 0u, 0u, 0u};
                if (8 * rb + i < R) wv[i] = *reinterpret_cast<const u32x4*>(p.Wup + (size_t)(8 * rb + i) * HD + h * D + 8 * cb);
            }
        }
        static_assert(NTHR == (128 / 8) * (D / 8), "one 8 x 8 block of the up-projection per thread");
        // this token's projected values: q, k (threads 0-127) or v, gate (128-255) of column j;
        // decay-down column tid (tid < R); beta (the last thread)
        struct Tok { float a, bb, dn, beta; };
        auto fetch = [&](int t) {
            const int m = b * p.T + t, base = rh ? 2 * HD : 0;
            Tok v;
            v.a = proj(m, base + hc);
            v.bb = proj(m, base + HD + hc);
            v.dn = tid < R ? proj(m, 4 * HD + tid) : 0.f;
            v.beta = tid == NTHR - 1 ? proj(m, 4 * HD + R + h) : 0.f;
            return v;
        };
        Tok cur = fetch(0);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int e = tid + u * NTHR;
            sm.cw[e / (3 * D)][(e / D) % 3][e % D] = cwv[u];
        }
        if (wal) {  // transposed in registers: channel 8cb + c gets ranks 8rb .. 8rb+7 in one 16-byte write
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 0][8 * rb]) = col8<0>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 1][8 * rb]) = col8<1>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 2][8 * rb]) = col8<2>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 3][8 * rb]) = col8<3>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 4][8 * rb]) = col8<4>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 5][8 * rb]) = col8<5>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 6][8 * rb]) = col8<6>(wv);
            *reinterpret_cast<u32x4*>(&sm.wupT[8 * cb + 7][8 * rb]) = col8<7>(wv);
        } else {
            for (int e = tid; e < 128 * D; e += NTHR) {
                const int r = e >> 7, c = e & 127;
                sm.wupT[c][r] = r < R ? p.Wup[(size_t)r * HD + h * D + c] : (uint16_t)0;
            }
        }
        for (int t = 0; t < p.T; ++t) {
            const int m = b * p.T + t;
            __syncthreads();  // every read of the previous token's rows (and of the window) is done
            if (rh == 0) { sm.qp[j] = cur.a; sm.kp[j] = cur.bb; } else { sm.vv[j] = cur.a; sm.gl[j] = cur.bb; }
            if (tid < 128) sm.dn[tid] = cur.dn;  // (zero past R)
            if (tid == NTHR - 1) sm.beta = sigm(cur.beta);
            if (t + 1 < p.T) cur = fetch(t + 1);  // in flight during this token's work
            __syncthreads();
            // short convolution + SiLU of q (threads 0-127) and k (128-255); the decay logit's half-sum of
            // channel j over ranks 64rh .. 64rh+63
            float act;
            {
                const int c = j;
                const float xcur = rh ? sm.kp[c] : sm.qp[c];
                const float y = taps[0] * sm.cw[rh][0][c] + taps[1] * sm.cw[rh][1][c] + taps[2] * sm.cw[rh][2][c] +
                                taps[3] * xcur;
                act = y * sigm(y);
                const u32x4* wr = reinterpret_cast<const u32x4*>(&sm.wupT[c][64 * rh]);
                const f32x4* dr = reinterpret_cast<const f32x4*>(&sm.dn[64 * rh]);
                float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const u32x4 w8 = wr[u];
                    const f32x4 d0 = dr[2 * u], d1 = dr[2 * u + 1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float de = e < 2 ? d0[2 * e] : d1[2 * e - 4], dodd = e < 2 ? d0[2 * e + 1] : d1[2 * e - 3];
                        z[e] = __builtin_fmaf(de, __uint_as_float(w8[e] << 16), z[e]);
                        z[e] = __builtin_fmaf(dodd, __uint_as_float(w8[e] & 0xffff0000u), z[e]);
                    }
                }
                sm.zp[rh][c] = (z[0] + z[1]) + (z[2] + z[3]);
            }
            // L2 norms: q over threads 0-127, k over 128-255 (each half sums its own two waves); the decay
            // gate g and exp(g) of channel j (threads 0-127)
            {
                float v = act * act;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
                __syncthreads();
                if ((tid & 63) == 0) sm.pw[0][tid >> 6] = v;
                __syncthreads();
                const float ss = rh ? sm.pw[0][2] + sm.pw[0][3] : sm.pw[0][0] + sm.pw[0][1];
                const float nv = act / sqrtf(ss + EPS);
                if (rh == 0) {
                    sm.q[j] = nv;
                    const float ga = -5.f * sigm(ea * (balpha + (sm.zp[0][j] + sm.zp[1][j])));
                    sm.ga[j] = ga;
                    sm.ega[j] = fexp(ga);
                } else {
                    sm.k[j] = nv;
                }
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
                s[i] *= sm.ega[64 * rh + i];
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
                    const float on = ot / sqrtf(ss * (1.f / D) + EPS) * rw * sigm(sm.gl[j]);
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
    (void)HD;
    const size_t a = (size_t)ldec::KS1 * M * ((ntot + 3) & ~3);
    const size_t b = (size_t)ldec::KS3 * M * dm;
    return a > b ? a : b;
}

hipError_t launch_layer_decode(const LayerDecodeParams& p, hipStream_t stream) {
    using namespace ldec;
    int nb = 0;
    for (int i = 0; i < 6; ++i) nb += (p.wn[i] + MCOLS - 1) / MCOLS;
    hipLaunchKernelGGL(ldec_proj_kernel, dim3((unsigned)(nb * KS1)), dim3(MT), 0, stream, p);
    hipLaunchKernelGGL(ldec_head_kernel, dim3((unsigned)(p.B * p.H)), dim3(NTHR), 0, stream, p);
    hipLaunchKernelGGL(ldec_out_kernel, dim3((unsigned)(((p.dm + MCOLS - 1) / MCOLS) * KS3)), dim3(MT), 0, stream, p);
    const long n4 = (long)p.B * p.T * p.dm / 4;
    hipLaunchKernelGGL(ldec_sum_kernel, dim3((unsigned)((n4 + 255) / 256 < 2048 ? (n4 + 255) / 256 : 2048)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_window_commit(float* conv, const float* qpre, const float* kpre, int B, int T, int HD, int n,
                                hipStream_t stream) {
    const long total = (long)B * 2 * HD;
    const unsigned blocks = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
    hipLaunchKernelGGL(ldec::window_commit_kernel, dim3(blocks), dim3(256), 0, stream, conv, qpre, kpre, B, T, HD, n);
    return hipGetLastError();
}

}  // namespace kda
