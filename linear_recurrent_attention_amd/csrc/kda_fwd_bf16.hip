// Chunkwise KDA forward for bf16 q/k/v, float32 g/beta/state, d_k = d_v = 128, on gfx950.
//
// What is computed: the gated delta rule of the explainer page "Kimi K3：开放前沿智能",
// section 2.2 (paper Eq. 1) with the readout of section 2.4, in the chunkwise-parallel form of
// section 2.5 (paper Eq. 4): per chunk of C = 32 tokens an inter-chunk term Gamma*Q*S, an
// intra-chunk lower-triangular term A*V_hat, and a hand-off of the 128 x 128 state.  Within a
// chunk, with incoming state S, cumulative log-decay b_r = sum_{j<=r} g_j and Gamma = exp(b):
//   L = strictly lower part of (K*Gamma)(K/Gamma)^T,  A = lower part of (Q*Gamma)(K/Gamma)^T,
//   T = (I + Diag(beta) L)^{-1} Diag(beta)            (the triangular "UT" inverse),
//   W = T (K*Gamma),  U_tilde = T V,  U = U_tilde - W S,
//   O = (Q*Gamma) S + A U,
//   S <- Diag(Gamma_last) S + (K*exp(b_last - b))^T U.
// The 1/Gamma factors are formed only inside 16-token sub-tiles, relative to the cumulative decay
// at the sub-tile's midpoint token, so every factor lies in [e^-40, e^40] (section 3.1-3.2: the
// lower bound g >= -5 is what keeps these in range).  A product that couples the two sub-tiles
// moves the earlier sub-tile's factor to the later sub-tile's reference first.
//
// Mapping: one workgroup of 4 waves per (batch, head, value half): the 128 value columns are
// split over two workgroups that recompute the key-side products, so 2*B*H workgroups fill the
// chip.  Each wave owns 16 value columns of the float32 state in matrix-core accumulator layout
// for the whole sequence; chunk inputs are prefetched one chunk ahead into registers.
//
// Matrix-core operands (v_mfma_f32_16x16x32_{bf16,f16}, float32 accumulate):
//   L = Km Kh^T                      bf16
//   A = Qm Kh^T                      split bf16 (hi*hi + hi*lo + lo*hi)
//   W = T Kg                         f16
//   U_tilde = T V                    T split bf16, V bf16
//   U = U_tilde - W S, Q S           f16
//   A U                              split bf16
//   Kbar^T U                         f16
// The inverse T is a float32 forward substitution on the two 16x16 diagonal blocks plus one
// off-diagonal block product.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace bf16path {

constexpr int C = 32;       // tokens per chunk
constexpr int SUB = 16;     // tokens per sub-tile
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVH = 64;     // value columns per workgroup
constexpr int NTHR = 256;   // 4 waves
constexpr int LDK = DK + 8; // padded row (16-bit elements) of token-major [C][DK] tiles
constexpr int LDT = C + 8;  // padded row of channel-major [DK][C] tiles
constexpr int LDA = C + 8;  // padded row of [C][C] 16-bit tiles
constexpr int LDF = C + 1;  // padded row of [C][C] float tiles
constexpr int LDO = DVH + 4;

struct alignas(16) Smem {
    uint16_t qmh[C][LDK], qml[C][LDK];     // Q * exp(b - b_mid)      split bf16
    uint16_t km[C][LDK];                   // K * exp(b - b_mid)      bf16
    uint16_t khh[C][LDK], khl[C][LDK];     // K * exp(b_mid - b)      split bf16
    uint16_t k1h[SUB][LDK], k1l[SUB][LDK]; // sub-tile 0 rows of K/Gamma at sub-tile 1's reference
    uint16_t qg[C][LDK];                   // Q * Gamma               f16
    uint16_t wn[C][LDK];                   // -W = -T (K * Gamma)     f16
    uint16_t kgt[DK][LDT];                 // (K * Gamma)^T           f16
    uint16_t kbt[DK][LDT];                 // (K * exp(b_last - b))^T f16
    uint16_t vt[DVH][LDT];                 // V^T (this value half)   bf16
    uint16_t ah[C][LDA], al[C][LDA];       // A                       split bf16
    uint16_t th[C][LDA], tl[C][LDA];       // T                       split bf16
    uint16_t tf[C][LDA];                   // T                       f16
    float lf[C][LDF];                      // L (strictly lower)
    float xf[C][LDF];                      // (I + Diag(beta) L)^{-1}
    float yf[SUB][SUB + 1];
    float ost[C][LDO];                     // output staging
    float tot[4][DK];                      // per 8-token octet sums of g
    float gamc[DK];                        // Gamma of the chunk's last token
    float beta[C];
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// Two 8-byte pieces: elements [p0, p0+4) and [p1, p1+4).
__device__ __forceinline__ u32x4 ld8x2(const uint16_t* p0, const uint16_t* p1) {
    u32x2 a = *reinterpret_cast<const u32x2*>(p0);
    u32x2 b = *reinterpret_cast<const u32x2*>(p1);
    return u32x4{a.x, a.y, b.x, b.y};
}

struct Raw {  // one thread's share of one chunk of input, as loaded
    uint32_t q[8], k[8], v[8];
    float2 g[8];
    float beta;
};

__device__ __forceinline__ void load_chunk(Raw& r, const Params& p, size_t bh_tok0, int t0, int wave, int lane,
                                           int half) {
    // tokens t0 + 8*wave + i; this thread's key channels 2*lane, 2*lane+1; value columns
    // half*64 + 2*lane (+1) for lane < 32; beta for token t0 + 8*wave + lane for lane < 8.
    // Tokens past the end read a clamped (valid) address and are replaced by zeros, which leaves
    // the state unchanged (k = v = 0, beta = 0, g = 0).  Requires T >= 1.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t = t0 + 8 * wave + i;
        const bool ok = t < p.T;
        const size_t row = bh_tok0 + (size_t)(ok ? t : p.T - 1) * p.H;  // (b*T + t)*H + h
        const size_t tk = row * DK + 2 * lane;
        const uint32_t qv = *reinterpret_cast<const uint32_t*>((const uint16_t*)p.q + tk);
        const uint32_t kv = *reinterpret_cast<const uint32_t*>((const uint16_t*)p.k + tk);
        const float2 gv = *reinterpret_cast<const float2*>(p.g + tk);
        const uint32_t vv = *reinterpret_cast<const uint32_t*>((const uint16_t*)p.v + row * DV + half * DVH +
                                                               2 * (lane & 31));
        r.q[i] = ok ? qv : 0u;
        r.k[i] = ok ? kv : 0u;
        r.g[i] = ok ? gv : make_float2(0.f, 0.f);
        r.v[i] = (ok && lane < 32) ? vv : 0u;
    }
    const int tb = t0 + 8 * wave + (lane & 7);
    const bool okb = lane < 8 && tb < p.T;
    const float bv = p.beta[bh_tok0 + (size_t)(tb < p.T ? tb : p.T - 1) * p.H];
    r.beta = okb ? bv : 0.f;
}

template <bool OUT_F32>
__global__ void __launch_bounds__(NTHR, 1) kda_fwd_bf16_kernel(Params p) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;

    // workgroup -> (batch*head, value half); siblings of one head land on the same XCD
    int bh, half;
    const int nbh = p.B * p.H;
    if ((nbh & 7) == 0) {
        const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
        half = local & 1;
        bh = (local >> 1) * 8 + xcd;
    } else {
        bh = blockIdx.x >> 1;
        half = blockIdx.x & 1;
    }
    const int b = bh / p.H, h = bh - b * p.H;
    const size_t bh_tok0 = (size_t)b * p.T * p.H + h;  // row index of token 0: (b*T + 0)*H + h

    // zero the parts of the [C][C] tiles that no chunk writes (upper block of A, T)
    for (int e = tid; e < SUB * SUB; e += NTHR) {
        const int r = e >> 4, c = SUB + (e & 15);
        sm.ah[r][c] = 0; sm.al[r][c] = 0; sm.th[r][c] = 0; sm.tl[r][c] = 0; sm.tf[r][c] = 0;
    }

    // state: st[cb][r] = S[16*cb + 4*g4 + r][half*64 + 16*wave + l16]
    f32x4 st[8];
    const int col = half * DVH + 16 * wave + l16;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g4 + r;
            st[cb][r] = p.S0 ? p.S0[((size_t)bh * DK + c) * DV + col] : 0.f;
        }
    }
    // state as f16 B operands of the channel contraction, K-step m covering channels 32m..32m+31 in
    // the order {32m + 4*g4 + r} then {32m + 16 + 4*g4 + r}
    u32x4 sb[4];
    auto make_sb = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            sb[m] = u32x4{pack_f16(st[2 * m][0], st[2 * m][1]), pack_f16(st[2 * m][2], st[2 * m][3]),
                          pack_f16(st[2 * m + 1][0], st[2 * m + 1][1]), pack_f16(st[2 * m + 1][2], st[2 * m + 1][3])};
    };
    make_sb();

    Raw raw;
    if (p.T > 0) load_chunk(raw, p, bh_tok0, 0, wave, lane, half);
    const int nchunk = (p.T + C - 1) / C;
    const int c0 = 2 * lane;       // this thread's key channels c0, c0 + 1
    const int sig = wave >> 1;     // sub-tile of this thread's octet
    const int hf = wave & 1;       // first or second octet of the sub-tile

    for (int ch = 0; ch < nchunk; ++ch) {
        const int t0 = ch * C;
        // ---- element-wise key side, part 1: cumulative decay within the octet, sub-tile factors
        float s0[8], s1[8];
        {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a0 += raw.g[i].x; a1 += raw.g[i].y;
                s0[i] = a0; s1[i] = a1;
            }
        }
        *reinterpret_cast<float2*>(&sm.tot[wave][c0]) = make_float2(s0[7], s1[7]);
        // reference = cumulative decay at the sub-tile's token 7 (end of its first octet)
        const float ref0 = hf ? 0.f : s0[7], ref1 = hf ? 0.f : s1[7];
        float qm0[8], qm1[8], km0[8], km1[8], kh0[8], kh1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 8 * wave + i;
            const float x0 = s0[i] - ref0, x1 = s1[i] - ref1;
            const float e0 = fexp(x0), e1 = fexp(x1);
            const float r0 = fexp(-x0), r1 = fexp(-x1);
            const float q0 = bf16lo_to_f(raw.q[i]), q1 = bf16hi_to_f(raw.q[i]);
            const float k0 = bf16lo_to_f(raw.k[i]), k1 = bf16hi_to_f(raw.k[i]);
            qm0[i] = q0 * e0; qm1[i] = q1 * e1;
            km0[i] = k0 * e0; km1[i] = k1 * e1;
            kh0[i] = k0 * r0; kh1[i] = k1 * r1;
            uint32_t hi, lo;
            split_bf16(qm0[i], qm1[i], hi, lo);
            *reinterpret_cast<uint32_t*>(&sm.qmh[t][c0]) = hi;
            *reinterpret_cast<uint32_t*>(&sm.qml[t][c0]) = lo;
            *reinterpret_cast<uint32_t*>(&sm.km[t][c0]) = pack_bf16(km0[i], km1[i]);
            split_bf16(kh0[i], kh1[i], hi, lo);
            *reinterpret_cast<uint32_t*>(&sm.khh[t][c0]) = hi;
            *reinterpret_cast<uint32_t*>(&sm.khl[t][c0]) = lo;
        }
        if (lane < 32) {  // V^T for value columns 2*lane, 2*lane+1 of this half
            uint32_t a[4], bb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = (raw.v[2 * i] & 0xffffu) | (raw.v[2 * i + 1] << 16);
                bb[i] = (raw.v[2 * i] >> 16) | (raw.v[2 * i + 1] & 0xffff0000u);
            }
            *reinterpret_cast<u32x4*>(&sm.vt[2 * lane][8 * wave]) = u32x4{a[0], a[1], a[2], a[3]};
            *reinterpret_cast<u32x4*>(&sm.vt[2 * lane + 1][8 * wave]) = u32x4{bb[0], bb[1], bb[2], bb[3]};
        }
        if (lane < 8) sm.beta[8 * wave + lane] = raw.beta;

        // the raw registers are consumed: prefetch the next chunk
        if (ch + 1 < nchunk) load_chunk(raw, p, bh_tok0, t0 + C, wave, lane, half);
        lds_barrier();

        // ---- element-wise key side, part 2: factors referenced to the chunk start and chunk end
        {
            float tt0[4], tt1[4];
#pragma unroll
            for (int o = 0; o < 4; ++o) { tt0[o] = sm.tot[o][c0]; tt1[o] = sm.tot[o][c0 + 1]; }
            const float pA0 = tt0[0], pA1 = tt1[0];                          // b at token 7
            const float pB0 = tt0[0] + tt0[1] + tt0[2], pB1 = tt1[0] + tt1[1] + tt1[2];  // b at token 23
            const float bC0 = pB0 + tt0[3], bC1 = pB1 + tt1[3];              // b at token 31
            const float p0 = sig ? pB0 : pA0, p1 = sig ? pB1 : pA1;
            const float eP0 = fexp(p0), eP1 = fexp(p1);
            const float eC0 = fexp(bC0 - p0), eC1 = fexp(bC1 - p1);
            uint16_t kg0[8], kg1[8], kb0[8], kb1[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * wave + i;
                *reinterpret_cast<uint32_t*>(&sm.qg[t][c0]) = pack_f16(qm0[i] * eP0, qm1[i] * eP1);
                const uint32_t kg = pack_f16(km0[i] * eP0, km1[i] * eP1);
                const uint32_t kb = pack_f16(kh0[i] * eC0, kh1[i] * eC1);
                kg0[i] = kg & 0xffffu; kg1[i] = kg >> 16;
                kb0[i] = kb & 0xffffu; kb1[i] = kb >> 16;
            }
            auto pack8 = [](const uint16_t* e) {
                return u32x4{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                             e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
            };
            *reinterpret_cast<u32x4*>(&sm.kgt[c0][8 * wave]) = pack8(kg0);
            *reinterpret_cast<u32x4*>(&sm.kgt[c0 + 1][8 * wave]) = pack8(kg1);
            *reinterpret_cast<u32x4*>(&sm.kbt[c0][8 * wave]) = pack8(kb0);
            *reinterpret_cast<u32x4*>(&sm.kbt[c0 + 1][8 * wave]) = pack8(kb1);
            if (sig == 0) {
                // K/Gamma rows of sub-tile 0 moved to sub-tile 1's reference: factor exp(b_23 - b_7) <= 1
                const float f0 = fexp(pB0 - pA0), f1 = fexp(pB1 - pA1);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int t = 8 * wave + i;
                    uint32_t hi, lo;
                    split_bf16(kh0[i] * f0, kh1[i] * f1, hi, lo);
                    *reinterpret_cast<uint32_t*>(&sm.k1h[t][c0]) = hi;
                    *reinterpret_cast<uint32_t*>(&sm.k1l[t][c0]) = lo;
                }
            }
            if (wave == 0) *reinterpret_cast<float2*>(&sm.gamc[c0]) = make_float2(fexp(bC0), fexp(bC1));
        }
        lds_barrier();

        // ---- Gram matrices on the matrix cores: A(0,0), A(1,0), A(1,1) split bf16; L blocks bf16
        if (wave < 3) {
            const int R = wave == 0 ? 0 : 1;  // row sub-tile
            const int S = wave == 2 ? 1 : 0;  // column sub-tile
            const uint16_t(*rh)[LDK] = (wave == 1) ? sm.k1h : (S ? sm.khh + SUB : sm.khh);
            const uint16_t(*rl)[LDK] = (wave == 1) ? sm.k1l : (S ? sm.khl + SUB : sm.khl);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kc = 32 * m + 8 * g4;
                const u32x4 aH = ld16(&sm.qmh[SUB * R + l16][kc]);
                const u32x4 aL = ld16(&sm.qml[SUB * R + l16][kc]);
                const u32x4 bH = ld16(&rh[l16][kc]);
                const u32x4 bL = ld16(&rl[l16][kc]);
                acc = mfma_bf16(aH, bH, acc);
                acc = mfma_bf16(aH, bL, acc);
                acc = mfma_bf16(aL, bH, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const int i0 = 4 * g4 + r;
                float v0 = acc[r], v1 = acc[r + 1];
                if (R == S) {  // keep the lower triangle including the diagonal
                    if (l16 > i0) v0 = 0.f;
                    if (l16 > i0 + 1) v1 = 0.f;
                }
                // rows i0 and i0+1, column l16: store element-wise
                const uint32_t hi0 = pack_bf16(v0, v1);
                const uint32_t lo0 = pack_bf16(v0 - bf16lo_to_f(hi0), v1 - bf16hi_to_f(hi0));
                sm.ah[SUB * R + i0][SUB * S + l16] = hi0 & 0xffffu;
                sm.ah[SUB * R + i0 + 1][SUB * S + l16] = hi0 >> 16;
                sm.al[SUB * R + i0][SUB * S + l16] = lo0 & 0xffffu;
                sm.al[SUB * R + i0 + 1][SUB * S + l16] = lo0 >> 16;
            }
        } else {
#pragma unroll
            for (int blk = 0; blk < 3; ++blk) {
                const int R = blk == 0 ? 0 : 1, S = blk == 2 ? 1 : 0;
                const uint16_t(*rh)[LDK] = (blk == 1) ? sm.k1h : (S ? sm.khh + SUB : sm.khh);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int kc = 32 * m + 8 * g4;
                    acc = mfma_bf16(ld16(&sm.km[SUB * R + l16][kc]), ld16(&rh[l16][kc]), acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * g4 + r;
                    float v = acc[r];
                    if (R == S && l16 >= i) v = 0.f;  // strictly lower
                    sm.lf[SUB * R + i][SUB * S + l16] = v;
                }
            }
        }
        lds_barrier();

        // ---- UT inverse: X = (I + Diag(beta) L)^{-1}, diagonal 16x16 blocks by forward substitution
        if (wave == 0 && lane < 32) {
            const int o = SUB * (lane >> 4), j = l16;
            float acc[SUB];
#pragma unroll
            for (int i = 0; i < SUB; ++i) acc[i] = 0.f;
            float x[SUB];
#pragma unroll
            for (int m = 0; m < SUB; ++m) {
                x[m] = (m == j) ? 1.f : -acc[m];
#pragma unroll
                for (int i = m + 1; i < SUB; ++i) acc[i] += sm.beta[o + i] * sm.lf[o + i][o + m] * x[m];
            }
#pragma unroll
            for (int i = 0; i < SUB; ++i) sm.xf[o + i][o + j] = x[i];
        }
        lds_barrier();
        {
            // Y = Diag(beta_1) L_10 X_00, then X_10 = -X_11 Y
            const int i = tid >> 4, j = tid & 15;
            float y = 0.f;
#pragma unroll
            for (int m = 0; m < SUB; ++m) y += sm.lf[SUB + i][m] * sm.xf[m][j];
            sm.yf[i][j] = sm.beta[SUB + i] * y;
        }
        lds_barrier();
        {
            const int i = tid >> 4, j = tid & 15;
            float x10 = 0.f;
#pragma unroll
            for (int m = 0; m < SUB; ++m) x10 -= sm.xf[SUB + i][SUB + m] * sm.yf[m][j];
            // T = X Diag(beta): blocks (0,0), (1,1) and (1,0), entry (i, j) of each
            const float b0 = sm.beta[j], b1 = sm.beta[SUB + j];
            const float t00 = sm.xf[i][j] * b0, t11 = sm.xf[SUB + i][SUB + j] * b1, t10 = x10 * b0;
            auto put = [&](int r, int c, float v) {
                const uint32_t hi = pack_bf16(v, 0.f);
                sm.th[r][c] = hi & 0xffffu;
                sm.tl[r][c] = pack_bf16(v - bf16lo_to_f(hi), 0.f) & 0xffffu;
                sm.tf[r][c] = pack_f16(v, 0.f) & 0xffffu;
            };
            put(i, j, t00);
            put(SUB + i, SUB + j, t11);
            put(SUB + i, j, t10);
        }
        lds_barrier();

        // ---- W = T (K*Gamma) (stored negated) and this wave's U_tilde = T V
        f32x4 ut[2];
        {
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                const u32x4 tfa = ld16(&sm.tf[SUB * R + l16][8 * g4]);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int ct = 2 * wave + cc;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    acc = mfma_f16(tfa, ld16(&sm.kgt[16 * ct + l16][8 * g4]), acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sm.wn[SUB * R + 4 * g4 + r][16 * ct + l16] = pack_f16(-acc[r], 0.f) & 0xffffu;
                }
                const u32x4 bv = ld16(&sm.vt[16 * wave + l16][8 * g4]);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma_bf16(ld16(&sm.th[SUB * R + l16][8 * g4]), bv, acc);
                acc = mfma_bf16(ld16(&sm.tl[SUB * R + l16][8 * g4]), bv, acc);
                ut[R] = acc;
            }
        }
        lds_barrier();

        // ---- state-dependent part (this wave's 16 value columns)
        // U = U_tilde - W S
#pragma unroll
        for (int R = 0; R < 2; ++R) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int cbase = 32 * m + 4 * g4;
                ut[R] = mfma_f16(ld8x2(&sm.wn[SUB * R + l16][cbase], &sm.wn[SUB * R + l16][cbase + 16]), sb[m], ut[R]);
            }
        }
        // U as B operands over the chunk's tokens, in the order {4*g4 + r} then {16 + 4*g4 + r}
        const u32x4 uf = {pack_f16(ut[0][0], ut[0][1]), pack_f16(ut[0][2], ut[0][3]), pack_f16(ut[1][0], ut[1][1]),
                          pack_f16(ut[1][2], ut[1][3])};
        uint32_t uh0, uh1, uh2, uh3, ul0, ul1, ul2, ul3;
        split_bf16(ut[0][0], ut[0][1], uh0, ul0);
        split_bf16(ut[0][2], ut[0][3], uh1, ul1);
        split_bf16(ut[1][0], ut[1][1], uh2, ul2);
        split_bf16(ut[1][2], ut[1][3], uh3, ul3);
        const u32x4 uh = {uh0, uh1, uh2, uh3}, ul = {ul0, ul1, ul2, ul3};
        // O = (Q*Gamma) S + A U
#pragma unroll
        for (int R = 0; R < 2; ++R) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int cbase = 32 * m + 4 * g4;
                acc = mfma_f16(ld8x2(&sm.qg[SUB * R + l16][cbase], &sm.qg[SUB * R + l16][cbase + 16]), sb[m], acc);
            }
            const u32x4 aH = ld8x2(&sm.ah[SUB * R + l16][4 * g4], &sm.ah[SUB * R + l16][SUB + 4 * g4]);
            const u32x4 aL = ld8x2(&sm.al[SUB * R + l16][4 * g4], &sm.al[SUB * R + l16][SUB + 4 * g4]);
            acc = mfma_bf16(aH, uh, acc);
            acc = mfma_bf16(aH, ul, acc);
            acc = mfma_bf16(aL, uh, acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.ost[SUB * R + 4 * g4 + r][16 * wave + l16] = acc[r] * p.scale;
        }
        // S <- Diag(Gamma_last) S + Kbar^T U
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) st[cb][r] *= sm.gamc[16 * cb + 4 * g4 + r];
            const u32x4 a = ld8x2(&sm.kbt[16 * cb + l16][4 * g4], &sm.kbt[16 * cb + l16][SUB + 4 * g4]);
            st[cb] = mfma_f16(a, uf, st[cb]);
        }
        make_sb();
        lds_barrier();

        // ---- store this chunk's output rows (32 tokens x 64 columns)
        {
            const int r = tid >> 3, cseg = (tid & 7) * 8;
            const int t = t0 + r;
            if (t < p.T) {
                const size_t off = (bh_tok0 + (size_t)t * p.H) * DV + half * DVH + cseg;
                const float* src = &sm.ost[r][cseg];
                if constexpr (OUT_F32) {
                    float4* dst = reinterpret_cast<float4*>((float*)p.o + off);
                    dst[0] = make_float4(src[0], src[1], src[2], src[3]);
                    dst[1] = make_float4(src[4], src[5], src[6], src[7]);
                } else {
                    *reinterpret_cast<u32x4*>((uint16_t*)p.o + off) =
                        u32x4{pack_bf16(src[0], src[1]), pack_bf16(src[2], src[3]), pack_bf16(src[4], src[5]),
                              pack_bf16(src[6], src[7])};
                }
            }
        }
    }

    if (p.S_T) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = 16 * cb + 4 * g4 + r;
                p.S_T[((size_t)bh * DK + c) * DV + col] = st[cb][r];
            }
        }
    }
}

}  // namespace bf16path

hipError_t launch_fwd_bf16(const Params& p, hipStream_t stream) {
    const int nblk = 2 * p.B * p.H;
    if (p.o_f32)
        hipLaunchKernelGGL(bf16path::kda_fwd_bf16_kernel<true>, dim3(nblk), dim3(bf16path::NTHR), 0, stream, p);
    else
        hipLaunchKernelGGL(bf16path::kda_fwd_bf16_kernel<false>, dim3(nblk), dim3(bf16path::NTHR), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
