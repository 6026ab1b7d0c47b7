// Fused KDA layer forward on gfx950: projections, short convolution, gates, the KDA core, norm.
//
// The layer of the explainer page "Kimi K3：开放前沿智能":
//   section 2.4 (paper Eq. 2): q, k = L2norm(Swish(ShortConv(x W))), v = x W_v;
//   section 2.3 (paper Eq. 2): decay logit z = W_up W_down x + b_alpha (low-rank), and
//   section 3.2 (paper Eq. 5): log(alpha) = -5 * sigmoid(exp(A_h) z), A a per-head log-scale;
//   beta = sigmoid(x W_beta) (not stated on the page; the plainest reading);
//   section 2.2/2.4: the gated delta rule and its readout (the bf16 KDA core of this library);
//   section 3.3 (paper Eq. 6): per-head RMSNorm, then a full-rank data-dependent gate
//   sigmoid(x W_g) with W_g of size d x d; finally the output projection W_o.
// Short convolution: causal, depthwise, 4 taps, no bias, tap 3 on the current token; the window
// of the previous 3 tokens comes from conv_state_in (zeros if absent) and the last 3 pre-conv
// rows go to conv_state_out.  L2 and RMSNorm use eps = 1e-6 inside the square root.
//
// The projections run on the library's bf16 matrix-core GEMM (float32 sums): one product over the
// concatenated q, k, v, gate, decay-down and beta weights, whose column segments land in separate
// buffers (the decay-down one as bf16 hi + lo halves, the up-projection's input); the rank-R decay
// up-projection as a product over those halves (about 16 significant bits), and the output
// projection.  The weights are taken into the products' [out][in] form in the workspace on each call.
// The element-wise work around the core:
//   T a multiple of 256: the input projection's epilogue applies the short conv, SiLU and L2 to q
//             and k on all rows but the first three of each 256-row tile; qk_fixup_kernel finishes
//             those from the raw rows the product kept, computes beta and the outgoing window;
//   otherwise: prologue_kernel, one wave per (token block, head): short conv + SiLU + L2 on q and
//             k, beta; conv_state_kernel for the window;
//   (q, k, v stay float32: the core's float32-input variant reads them, so the per-head RMSNorm does
//   not amplify a bf16 rounding of the core's inputs);
//   epilogue_kernel: RMSNorm of the core output, times sigmoid(gate), to bf16 for the output
//             projection.
#include "kda_common.h"
#include "kda_internal.h"
#include "../../include/kda.h"

namespace kda {
namespace layer {

constexpr int D = 128;  // head size (key and value)
constexpr float EPS = 1e-6f;

struct ProParams {
    int B, T, H, HD;
    const float* pq;       // [B*T, HD] pre-conv q projection
    const float* pk;       // [B*T, HD] pre-conv k projection
    const float* pv;       // [B*T, HD]
    const float* pbeta;    // [B*T, H]  beta logit
    const float* conv_q;   // [HD, 4]
    const float* conv_k;   // [HD, 4]
    const float* state_in; // [B, 3, 2*HD] or null
    float* q;              // [B*T, HD] = [B, T, H, D]
    float* k;
    float* v;
    float* beta;           // [B*T, H]
};

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + fexp(-x)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Prologue: one wave per (batch, head, block of PRO_TOK tokens); lane l holds channels c, c+1 with
// c = h*D + 2l.  The short convolution's window (the 3 previous pre-conv rows of q and k) is carried
// in registers along the tokens, so each projection row is read once.
constexpr int PRO_TOK = 32;
constexpr int PRO_U = 8;  // tokens whose rows are read together

__device__ __forceinline__ float silu(float x) { return x * sigmoidf_(x); }

__global__ void __launch_bounds__(256) prologue_kernel(ProParams p) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nblk = (p.T + PRO_TOK - 1) / PRO_TOK;
    const long gw = (long)blockIdx.x * 4 + wave;  // ((b * H) + h) * nblk + blk
    if (gw >= (long)p.B * p.H * nblk) return;
    const int blk = (int)(gw % nblk);
    const long bh = gw / nblk;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    const int c = h * D + 2 * lane;
    const int t0 = blk * PRO_TOK, t1 = min(t0 + PRO_TOK, p.T);

    float wq[2][4], wk[2][4];  // taps of channels c, c+1; tap 3 multiplies the current token
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const float4 a = *reinterpret_cast<const float4*>(p.conv_q + (size_t)(c + e) * 4);
        const float4 k = *reinterpret_cast<const float4*>(p.conv_k + (size_t)(c + e) * 4);
        wq[e][0] = a.x; wq[e][1] = a.y; wq[e][2] = a.z; wq[e][3] = a.w;
        wk[e][0] = k.x; wk[e][1] = k.y; wk[e][2] = k.z; wk[e][3] = k.w;
    }
    // window: rows t0-3, t0-2, t0-1 (from this call's projections, the incoming window, or zeros)
    float2 xq[3], xk[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = t0 - 3 + j;
        xq[j] = xk[j] = make_float2(0.f, 0.f);
        if (tt >= 0) {
            xq[j] = *reinterpret_cast<const float2*>(p.pq + ((size_t)b * p.T + tt) * p.HD + c);
            xk[j] = *reinterpret_cast<const float2*>(p.pk + ((size_t)b * p.T + tt) * p.HD + c);
        } else if (p.state_in) {
            const float* sw = p.state_in + ((size_t)b * 3 + (3 + tt)) * 2 * p.HD;
            xq[j] = *reinterpret_cast<const float2*>(sw + c);
            xk[j] = *reinterpret_cast<const float2*>(sw + p.HD + c);
        }
    }
    // PRO_U tokens at a time: all their projection rows are read first (rows past t1 read row t1 - 1
    // and are not used), so that each wave keeps 3 * PRO_U reads in flight instead of 3
    for (int t = t0; t < t1; t += PRO_U) {
        float2 cq[PRO_U], ck[PRO_U];
        float bl[PRO_U];
#pragma unroll
        for (int u = 0; u < PRO_U; ++u) {
            const size_t row = (size_t)b * p.T + min(t + u, t1 - 1);
            cq[u] = *reinterpret_cast<const float2*>(p.pq + row * p.HD + c);
            ck[u] = *reinterpret_cast<const float2*>(p.pk + row * p.HD + c);
            bl[u] = p.pbeta[row * p.H + h];
        }
#pragma unroll
        for (int u = 0; u < PRO_U; ++u) {
            if (t + u >= t1) break;  // (wave-uniform)
            const size_t row = (size_t)b * p.T + t + u;
            const size_t rc = row * p.HD + c;
            float q0 = 0.f, q1 = 0.f, k0 = 0.f, k1 = 0.f;
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                q0 += wq[0][j] * xq[j].x; q1 += wq[1][j] * xq[j].y;
                k0 += wk[0][j] * xk[j].x; k1 += wk[1][j] * xk[j].y;
            }
            q0 += wq[0][3] * cq[u].x; q1 += wq[1][3] * cq[u].y;
            k0 += wk[0][3] * ck[u].x; k1 += wk[1][3] * ck[u].y;
            xq[0] = xq[1]; xq[1] = xq[2]; xq[2] = cq[u];
            xk[0] = xk[1]; xk[1] = xk[2]; xk[2] = ck[u];
            q0 = silu(q0); q1 = silu(q1); k0 = silu(k0); k1 = silu(k1);
            const float qn = rsqrtf(wave_sum(q0 * q0 + q1 * q1) + EPS);
            const float kn = rsqrtf(wave_sum(k0 * k0 + k1 * k1) + EPS);
            *reinterpret_cast<float2*>(p.q + rc) = make_float2(q0 * qn, q1 * qn);
            *reinterpret_cast<float2*>(p.k + rc) = make_float2(k0 * kn, k1 * kn);
            if (lane == 0) p.beta[row * p.H + h] = sigmoidf_(bl[u]);
        }
    }
}

// Last three pre-conv rows of each sequence (from this call's projections, or the incoming window
// when T < 3): the window the next segment continues from.
__global__ void conv_state_kernel(int B, int T, int HD, const float* pq, const float* pk, const float* state_in,
                                  float* state_out) {
    const long n = (long)B * 3 * 2 * HD;
    for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int ch = (int)(e % (2 * HD));
        const long r = e / (2 * HD);
        const int s = (int)(r % 3), b = (int)(r / 3);
        const int tt = T - 3 + s;
        float val = 0.f;
        if (tt >= 0) {
            const float* src = ch < HD ? pq : pk;
            val = src[((size_t)b * T + tt) * HD + (ch % HD)];
        } else if (state_in) {
            val = state_in[((size_t)b * 3 + (3 + tt)) * 2 * HD + ch];
        }
        state_out[e] = val;
    }
}

// The fused path (T a multiple of 256): the input projection's epilogue already applied the short
// convolution, SiLU and L2 to q and k except on rows 0-2 of each 256-row tile, whose window reaches
// into the tile above; it kept each tile's first and last three raw rows in side[tile][6][2*HD] (q
// columns, then k).  This kernel finishes those rows, one wave per (tile, head of q or k, row) with
// two channels per lane (the window from the tile above, or from the incoming window at a sequence
// start), and beyond those waves computes beta = sigmoid(beta logit) for every row.
struct FixParams {
    int B, T, H, HD;
    const float* side;
    const float* conv_q;    // [HD, 4]
    const float* conv_k;
    const float* state_in;  // [B, 3, 2*HD] or null
    const float* pbeta;     // [B*T, H] beta logit
    float* q;               // [B*T, HD]
    float* k;
    float* beta;            // [B*T, H]
    float* state_out;       // [B, 3, 2*HD] or null: the outgoing window
    int fix_blocks;         // workgroups of the row fixups; the rest compute beta and the window
};

__global__ void __launch_bounds__(256) qk_fixup_kernel(FixParams p) {
    if ((int)blockIdx.x >= p.fix_blocks) {
        // beta for every row, then the outgoing window: the last three raw rows of each sequence,
        // kept in the side buffer by the tile that ends it
        const long nb = (long)p.B * p.T * p.H;
        const size_t qkc = 2 * (size_t)p.HD;
        const long n = nb + (p.state_out ? (long)p.B * 3 * (long)qkc : 0);
        for (long e = (long)(blockIdx.x - p.fix_blocks) * blockDim.x + threadIdx.x; e < n;
             e += (long)(gridDim.x - p.fix_blocks) * blockDim.x) {
            if (e < nb) {
                p.beta[e] = sigmoidf_(p.pbeta[e]);
            } else {
                const long f = e - nb;
                const int ch = (int)(f % (long)qkc);
                const long r = f / (long)qkc;
                const int s = (int)(r % 3), b = (int)(r / 3);
                const long tr_last = ((long)(b + 1) * p.T) / 256 - 1;
                p.state_out[f] = p.side[((size_t)tr_last * 6 + 3 + s) * qkc + ch];
            }
        }
        return;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int ntile = p.B * p.T / 256, nhg = 2 * p.H;
    const long gw = (long)blockIdx.x * 4 + wave;
    if (gw >= (long)ntile * nhg * 3) return;
    const int r = (int)(gw % 3), hg = (int)((gw / 3) % nhg), tr = (int)(gw / (3L * nhg));
    const int ch = 128 * hg + 2 * lane;  // column in [0, 2*HD): q, then k
    const size_t qkc = 2 * (size_t)p.HD;
    const long m = 256L * tr + r;
    const int b = (int)(m / p.T);
    float2 x[4];  // raw rows m-3 .. m
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const long g = m - 3 + j;
        const float* src;
        if (g >= 256L * tr) src = p.side + ((size_t)tr * 6 + (size_t)(g - 256L * tr)) * qkc;
        else if (g >= (long)b * p.T) src = p.side + ((size_t)(tr - 1) * 6 + 3 + (size_t)(g - (256L * tr - 3))) * qkc;
        else if (p.state_in) src = p.state_in + ((size_t)b * 3 + 3 + (g - (long)b * p.T)) * qkc;
        else src = nullptr;
        x[j] = src ? *reinterpret_cast<const float2*>(src + ch) : make_float2(0.f, 0.f);
    }
    const bool isq = ch < p.HD;
    const float* taps = isq ? p.conv_q + (size_t)ch * 4 : p.conv_k + (size_t)(ch - p.HD) * 4;
    const float4 w0 = *reinterpret_cast<const float4*>(taps), w1 = *reinterpret_cast<const float4*>(taps + 4);
    const float a0[4] = {w0.x, w0.y, w0.z, w0.w}, a1[4] = {w1.x, w1.y, w1.z, w1.w};
    float y0 = 0.f, y1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        y0 += a0[j] * x[j].x;
        y1 += a1[j] * x[j].y;
    }
    y0 = silu(y0);
    y1 = silu(y1);
    const float inv = rsqrtf(wave_sum(y0 * y0 + y1 * y1) + EPS);
    float* dst = isq ? p.q + (size_t)m * p.HD + ch : p.k + (size_t)m * p.HD + (ch - p.HD);
    *reinterpret_cast<float2*>(dst) = make_float2(y0 * inv, y1 * inv);
}

__global__ void __launch_bounds__(256) epilogue_kernel(int rows, int H, int HD, const float* o, const float* pg,
                                                      const float* rms_w, uint16_t* gated) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long gw = (long)blockIdx.x * 4 + wave;
    if (gw >= (long)rows * H) return;
    const long row = gw / H;
    const int h = (int)(gw - row * H);
    const size_t rc = (size_t)row * HD + h * D + 2 * lane;
    const float2 ov = *reinterpret_cast<const float2*>(o + rc);
    const float inv = rsqrtf(wave_sum(ov.x * ov.x + ov.y * ov.y) * (1.f / D) + EPS);
    const float2 w = *reinterpret_cast<const float2*>(rms_w + 2 * lane);
    const float2 gl = *reinterpret_cast<const float2*>(pg + rc);
    *reinterpret_cast<uint32_t*>(gated + rc) =
        pack_bf16(ov.x * inv * w.x * sigmoidf_(gl.x), ov.y * inv * w.y * sigmoidf_(gl.y));
}

__global__ void bf16_to_f32_kernel(const uint16_t* src, float* dst, long n) {
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
        dst[i] = __uint_as_float((uint32_t)src[i] << 16);
}

struct Workspace {
    float *pq, *pk, *pv, *pg, *pbeta, *g, *beta, *o, *q, *k, *cp, *side;
    uint16_t *gated, *wcat, *wup2, *wo, *down2;
    size_t bytes;
};

Workspace carve(const kda_layer_desc* d, char* base) {
    const size_t BT = (size_t)d->B * d->T, HD = (size_t)d->H * D;
    size_t off = 0;
    auto take = [&](size_t nbytes) {
        char* p = base ? base + off : nullptr;
        off += (nbytes + 255) & ~(size_t)255;
        return p;
    };
    Workspace w;
    w.pq = (float*)take(BT * HD * 4);
    w.pk = (float*)take(BT * HD * 4);
    w.pv = (float*)take(BT * HD * 4);
    w.pg = (float*)take(BT * HD * 4);
    w.pbeta = (float*)take(BT * d->H * 4);
    w.g = (float*)take(BT * HD * 4);
    w.beta = (float*)take(BT * d->H * 4);
    w.o = (float*)take(BT * HD * 4);
    w.q = (float*)take(BT * HD * 4);
    w.k = (float*)take(BT * HD * 4);
    w.gated = (uint16_t*)take(BT * HD * 2);
    const size_t ncat = 4 * HD + d->rank + d->H;  // rows of the concatenated input-projection weights
    w.wcat = (uint16_t*)take(ncat * d->d_model * 2);
    w.wup2 = (uint16_t*)take(HD * 2 * d->rank * 2);
    w.wo = (uint16_t*)take((size_t)d->d_model * HD * 2);
    w.down2 = (uint16_t*)take(BT * 2 * d->rank * 2);
    w.cp = (float*)take(cp_workspace_bytes(d->B, d->T, d->H, 0));  // the core's context parallelism
    w.side = (float*)take((BT + 255) / 256 * 6 * 2 * HD * 4);      // raw rows at the q/k product's tile edges
    w.bytes = off;
    return w;
}

}  // namespace layer
}  // namespace kda

using namespace kda::layer;

namespace {
kda_status check_layer(const kda_layer_desc* d, const void* x, const kda_layer_weights* w, const void* y) {
    if (!d || !w || !x || !y) return KDA_ERR_INVALID_ARG;
    if (d->B < 1 || d->T < 1 || d->H < 1 || d->d_model < 1 || d->rank < 1 || d->flags != 0) return KDA_ERR_INVALID_ARG;
    if (d->Dk != D || d->Dv != D || d->conv != 4) return KDA_ERR_UNSUPPORTED;
    if (d->d_model % 32 != 0 || d->rank % 16 != 0) return KDA_ERR_UNSUPPORTED;  // the GEMMs' k steps
    if ((reinterpret_cast<uintptr_t>(x) & 15) != 0 || (reinterpret_cast<uintptr_t>(y) & 15) != 0)
        return KDA_ERR_INVALID_ARG;
    if ((long long)d->B * d->T > (1LL << 30) || (long long)d->B * d->T * d->H * D > (1LL << 40)) return KDA_ERR_INVALID_ARG;
    if (!w->Wq || !w->Wk || !w->Wv || !w->Wg || !w->Wo || !w->Wbeta || !w->Wdown || !w->Wup || !w->conv_q ||
        !w->conv_k || !w->b_alpha || !w->A || !w->rms_w)
        return KDA_ERR_INVALID_ARG;
    if (!(d->scale == d->scale)) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}
}  // namespace

extern "C" {

size_t kda_layer_workspace_size(const kda_layer_desc* desc) {
    if (!desc || desc->B < 1 || desc->T < 1 || desc->H < 1 || desc->rank < 1) return 0;
    return carve(desc, nullptr).bytes;
}

kda_status kda_layer_fwd(const kda_layer_desc* d, const void* x, const kda_layer_weights* w, const float* S0,
                         const float* conv_state_in, void* y, float* S_T, float* conv_state_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
    const kda_status st = check_layer(d, x, w, y);
    if (st != KDA_OK) return st;
    const Workspace W = carve(d, (char*)ws);
    if (!ws || ws_bytes < W.bytes) return KDA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return KDA_ERR_INVALID_ARG;

    const int M = d->B * d->T, HD = d->H * D, dm = d->d_model, R = d->rank;
    // every 256-row tile of the q/k product inside one sequence: the short convolution, SiLU and L2 run
    // in the product's epilogue and a small kernel finishes the tile-edge rows (else the prologue kernel)
    const bool fused = d->T % 256 == 0;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    auto wb = [](const void* p) { return static_cast<const uint16_t*>(p); };
    // weights in the products' [out][in] form: [Wq | Wk | Wv | Wg | Wdown | Wbeta]^T, [Wup^T | Wup^T]
    // (the up-projection runs over the hi and lo halves of its input), Wo^T
    const int ncat = 4 * HD + R + d->H;
    const int noff[6] = {0, HD, 2 * HD, 3 * HD, 4 * HD, 4 * HD + R};
    const void* wsrc[6] = {w->Wq, w->Wk, w->Wv, w->Wg, w->Wdown, w->Wbeta};
    const int wn[6] = {HD, HD, HD, HD, R, d->H};
    {
        kda::TransposeBatch tb{};
        auto job = [&](const void* src, int lds, int K, int N, uint16_t* dst, int ldd) {
            kda::TransposeJob& J = tb.job[tb.njobs++];
            J.src = wb(src); J.lds = lds; J.K = K; J.N = N; J.dst = dst; J.ldd = ldd;
        };
        for (int i = 0; i < 6; ++i) job(wsrc[i], wn[i], dm, wn[i], W.wcat + (size_t)noff[i] * dm, dm);
        job(w->Wup, HD, R, HD, W.wup2, 2 * R);
        job(w->Wup, HD, R, HD, W.wup2 + R, 2 * R);
        job(w->Wo, dm, HD, dm, W.wo, HD);
        if (kda::launch_transpose_batch(tb, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    {
        kda::GemmOut go{};
        void* dst[6] = {W.pq, W.pk, W.pv, W.pg, W.down2, W.pbeta};
        for (int i = 0; i < 6; ++i) {
            go.ptr[i] = dst[i];
            go.start[i] = noff[i];
            go.ld[i] = wn[i];
        }
        go.ld[4] = 2 * R;  // the decay-down projection as bf16 [hi | lo] halves, the up-projection's input
        go.split_segs = 1 << 4;
        go.start[6] = ncat;
        go.nseg = 6;
        if (fused) {  // q and k come out convolved, activated and normalised (but for the tile-edge rows)
            go.ptr[0] = W.q;
            go.ptr[1] = W.k;
            go.epi = kda::GEMM_QKCONV;
            go.conv_q = w->conv_q;
            go.conv_k = w->conv_k;
            go.side = W.side;
            go.qk_cols = 2 * HD;
            go.qk_hd = HD;
            go.eps = EPS;
        }
        if (kda::launch_gemm_nt(xb, dm, W.wcat, dm, go, true, M, ncat, dm, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    {  // the rank-R up-projection, with the decay gate -5 sigmoid(exp(A_h) (z + b_alpha)) on the way out
        kda::GemmOut go{};
        go.ptr[0] = W.g;
        go.start[0] = 0;
        go.start[1] = HD;
        go.ld[0] = HD;
        go.nseg = 1;
        go.epi = kda::GEMM_GATE;
        go.bias = w->b_alpha;
        go.head_scale = w->A;
        if (kda::launch_gemm_nt(W.down2, 2 * R, W.wup2, 2 * R, go, true, M, HD, 2 * R, stream) != hipSuccess)
            return KDA_ERR_HIP;
    }

    ProParams pp;
    pp.B = d->B; pp.T = d->T; pp.H = d->H; pp.HD = HD;
    pp.pq = W.pq; pp.pk = W.pk; pp.pv = W.pv; pp.pbeta = W.pbeta;
    pp.conv_q = w->conv_q; pp.conv_k = w->conv_k;
    pp.state_in = conv_state_in;
    pp.q = W.q; pp.k = W.k; pp.v = nullptr; pp.beta = W.beta;
    const long nw = (long)M * d->H;
    if (fused) {
        FixParams fp;
        fp.B = d->B; fp.T = d->T; fp.H = d->H; fp.HD = HD;
        fp.side = W.side; fp.conv_q = w->conv_q; fp.conv_k = w->conv_k; fp.state_in = conv_state_in;
        fp.pbeta = W.pbeta; fp.q = W.q; fp.k = W.k; fp.beta = W.beta; fp.state_out = conv_state_out;
        const long nfw = (long)(M / 256) * 2 * d->H * 3;  // fixup waves
        fp.fix_blocks = (int)((nfw + 3) / 4);
        hipLaunchKernelGGL(qk_fixup_kernel, dim3((unsigned)(fp.fix_blocks + 256)), dim3(256), 0, stream, fp);
    } else {
        const long npw = (long)d->B * d->H * ((d->T + PRO_TOK - 1) / PRO_TOK);  // prologue waves
        hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)((npw + 3) / 4)), dim3(256), 0, stream, pp);
        if (conv_state_out)
            hipLaunchKernelGGL(conv_state_kernel, dim3(256), dim3(256), 0, stream, d->B, d->T, HD, W.pq, W.pk,
                               conv_state_in, conv_state_out);
    }

    kda::Params p{};  // zero: every optional field off
    // the core reads q, k, v in float32 (v straight from the projection output): rounding them to
    // bf16 first would be amplified by the per-head RMSNorm wherever a head's output is small
    p.q = W.q; p.k = W.k; p.v = W.pv; p.g = W.g; p.beta = W.beta; p.S0 = S0; p.o = W.o; p.S_T = S_T;
    p.B = d->B; p.T = d->T; p.tstride = d->T; p.H = d->H; p.Dk = D; p.Dv = D; p.scale = d->scale;
    p.o_f32 = 1; p.in_f32 = 1; p.precise = 1;
    p.S_ckpt = nullptr; p.ckpt_chunks = 1; p.n_ckpt = 0;
    // few heads (2*B*H workgroups well under the 256 CUs) run as segments side by side
    if (kda::launch_fwd_cp(p, 0, W.cp, stream) != hipSuccess) return KDA_ERR_HIP;

    hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)((nw + 3) / 4)), dim3(256), 0, stream, M, d->H, HD, W.o, W.pg,
                       w->rms_w, W.gated);
    {
        kda::GemmOut go{};
        go.ptr[0] = y;
        go.start[0] = 0;
        go.start[1] = dm;
        go.ld[0] = dm;
        go.nseg = 1;
        if (kda::launch_gemm_nt(W.gated, HD, W.wo, HD, go, false, M, dm, HD, stream) != hipSuccess) return KDA_ERR_HIP;
    }
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ------------------------------------------------------------------------------------------------
// Decode step with the projection-input cache (kda_layer_decode.hip)

namespace {
constexpr int kDecodeMaxRows = 16;  // B*T rows per decode call
constexpr int kDecodeMaxRank = 128;

kda_status check_decode(const kda_layer_desc* d) {
    if (!d || d->B < 1 || d->T < 1 || d->H < 1 || d->d_model < 1 || d->rank < 1) return KDA_ERR_INVALID_ARG;
    if (d->flags & ~KDA_DECODE_SPECULATIVE) return KDA_ERR_INVALID_ARG;
    if (d->Dk != D || d->Dv != D || d->conv != 4) return KDA_ERR_UNSUPPORTED;
    if ((long long)d->B * d->T > kDecodeMaxRows || d->rank > kDecodeMaxRank || d->d_model % 4) return KDA_ERR_UNSUPPORTED;
    if (!(d->scale == d->scale)) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

size_t decode_cache_floats(const kda_layer_desc* d) {
    return (size_t)d->B * d->T * (5 * (size_t)d->H * D + d->H);
}

struct DecodeWs {
    float *part, *gated;
    size_t bytes;
};
DecodeWs carve_decode(const kda_layer_desc* d, char* base) {
    const int M = d->B * d->T, HD = d->H * D;
    const int ntot = (4 * HD + d->rank + d->H + 3) & ~3;  // padded row length
    size_t off = 0;
    auto take = [&](size_t nbytes) {
        char* p = base ? base + off : nullptr;
        off += (nbytes + 255) & ~(size_t)255;
        return p;
    };
    DecodeWs w;
    w.part = (float*)take(kda::layer_decode_part_floats(M, d->d_model, HD, ntot) * 4);
    w.gated = (float*)take((size_t)M * HD * 4);
    w.bytes = off;
    return w;
}
}  // namespace

size_t kda_layer_decode_workspace_size(const kda_layer_desc* desc) {
    if (check_decode(desc) != KDA_OK) return 0;
    return carve_decode(desc, nullptr).bytes;
}

size_t kda_layer_decode_cache_bytes(const kda_layer_desc* desc) {
    if (check_decode(desc) != KDA_OK) return 0;
    return decode_cache_floats(desc) * sizeof(float);
}

kda_status kda_layer_decode(const kda_layer_desc* d, const void* x, const kda_layer_weights* w, float* S,
                            float* conv_state, void* y, float* cache, void* ws, size_t ws_bytes, hipStream_t stream) {
    kda_status st = check_decode(d);
    if (st != KDA_OK) return st;
    if (!x || !w || !S || !y) return KDA_ERR_INVALID_ARG;
    if ((d->flags & KDA_DECODE_SPECULATIVE) && !cache) return KDA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 15)) return KDA_ERR_INVALID_ARG;
    if (!w->Wq || !w->Wk || !w->Wv || !w->Wg || !w->Wo || !w->Wbeta || !w->Wdown || !w->Wup || !w->conv_q ||
        !w->conv_k || !w->b_alpha || !w->A || !w->rms_w)
        return KDA_ERR_INVALID_ARG;
    const DecodeWs W = carve_decode(d, (char*)ws);
    if (!ws || ws_bytes < W.bytes) return KDA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return KDA_ERR_INVALID_ARG;
    const int HD = d->H * D, R = d->rank;
    kda::LayerDecodeParams p{};
    p.x = static_cast<const uint16_t*>(x);
    const void* wsrc[6] = {w->Wq, w->Wk, w->Wv, w->Wg, w->Wdown, w->Wbeta};
    const int wn[6] = {HD, HD, HD, HD, R, d->H};
    int off = 0;
    for (int i = 0; i < 6; ++i) {
        p.W[i] = static_cast<const uint16_t*>(wsrc[i]);
        p.wn[i] = wn[i];
        p.noff[i] = off;
        off += wn[i];
    }
    p.noff[6] = off;
    p.Wup = static_cast<const uint16_t*>(w->Wup);
    p.Wo = static_cast<const uint16_t*>(w->Wo);
    p.conv_q = w->conv_q; p.conv_k = w->conv_k; p.b_alpha = w->b_alpha; p.A = w->A; p.rms_w = w->rms_w;
    p.S = S; p.conv = conv_state; p.y = static_cast<uint16_t*>(y); p.cache = cache;
    p.part = W.part; p.gated = W.gated;
    p.B = d->B; p.T = d->T; p.H = d->H; p.dm = d->d_model; p.R = R;
    p.spec = (d->flags & KDA_DECODE_SPECULATIVE) ? 1 : 0;
    p.scale = d->scale;
    return kda::launch_layer_decode(p, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_layer_decode_commit(const kda_layer_desc* d, const float* cache, int n_accept, float* S,
                                   float* conv_state, hipStream_t stream) {
    kda_layer_desc dd;
    if (!d) return KDA_ERR_INVALID_ARG;
    dd = *d;
    dd.flags = 0;
    kda_status st = check_decode(&dd);
    if (st != KDA_OK) return st;
    if (!cache || !S || n_accept < 0 || n_accept > d->T) return KDA_ERR_INVALID_ARG;
    if (n_accept == 0) return KDA_OK;
    const size_t HD = (size_t)d->H * D, ntok = (size_t)d->B * d->T;
    const float* k = cache;
    const float* v = cache + ntok * HD;
    const float* g = cache + 2 * ntok * HD;
    const float* beta = cache + 3 * ntok * HD;
    const float* qpre = beta + ntok * d->H;
    const float* kpre = qpre + ntok * HD;
    kda::Params p{};  // the token-by-token step over the accepted entries, state in place, no output
    p.q = k; p.k = k; p.v = v; p.g = g; p.beta = beta; p.S0 = S; p.S_T = S; p.o = nullptr;
    p.B = d->B; p.T = n_accept; p.tstride = d->T; p.H = d->H; p.Dk = D; p.Dv = D; p.scale = 1.f;
    p.o_f32 = 1; p.in_f32 = 1; p.ckpt_chunks = 1;
    if (kda::launch_decode(p, false, stream) != hipSuccess) return KDA_ERR_HIP;
    if (conv_state && kda::launch_window_commit(conv_state, qpre, kpre, d->B, d->T, (int)HD, n_accept, stream) !=
                          hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // extern "C"
