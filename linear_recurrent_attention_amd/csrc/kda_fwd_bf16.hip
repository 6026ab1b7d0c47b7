// Chunkwise KDA forward for bf16 q/k/v, float32 g/beta/state, d_k = d_v = 128, on gfx950.
//
// What is computed: the gated delta rule of the explainer page "Kimi K3：开放前沿智能",
// section 2.2 (paper Eq. 1) with the readout of section 2.4, in the chunkwise-parallel form of
// section 2.5 (paper Eq. 4): per chunk of C = 32 tokens an inter-chunk term Gamma*Q*S, an
// intra-chunk lower-triangular term A*V_hat, and a hand-off of the 128 x 128 state.  Within a
// chunk, with incoming state S, cumulative log-decay b_r = sum_{j<=r} g_j and Gamma = exp(b):
//   L = strictly lower part of (K*Gamma)(K/Gamma)^T,  A = lower part of (Q*Gamma)(K/Gamma)^T,
//   T = (I + Diag(beta) L)^{-1} Diag(beta)            (the triangular "UT" inverse),
//   U = T (V - (K*Gamma) S),
//   O = (Q*Gamma) S + A U,
//   S <- Diag(Gamma_last) S + (K*exp(b_last - b))^T U.
// The factors exp(+-(b - b_15)) are taken relative to the cumulative decay at the chunk's token 15,
// so with the lower bound g >= -5 of sections 3.1-3.2 each lies in [e^-80, e^80], inside the
// normal range of float32 and bf16; the products that enter L and A (t >= s) are at most 1.  The
// 32x32 products are formed as 16x16 blocks (two 16-token sub-tiles).
//
// Mapping.  One workgroup per (batch, head, value half): the 128 value columns are split over two
// workgroups that both compute the key-side products, so 2*B*H workgroups fill the chip; the two
// halves of a head are placed on the same XCD so their common reads of q, k, g share its L2.
// Each workgroup runs 12 waves as a two-stage pipeline over chunks:
//   key waves 0-7    chunk n:   wave kw owns tokens 4kw..4kw+3 (two key channels per lane): quad
//                               decay sums, then all decay factors, then the Gram products (waves
//                               0-3); the chunk's value-side tiles are written at the start of the
//                               next step;
//   value waves 8-11 chunk n-1: UT inverse, then the state-dependent products and the output;
//                               wave 8+w owns 16 value columns of the float32 state in matrix-core
//                               accumulator layout for the whole run.
// Both groups execute the same three workgroup barriers per step; data passes from the key waves
// to the value waves through LDS buffers indexed by chunk parity.  Chunk inputs are prefetched
// one chunk ahead into registers.
//
// Matrix-core operands (v_mfma_f32_16x16x32_{bf16,f16}, float32 accumulate):
//   L = Km Kh^T                      bf16                  HP: bf16 Km, split bf16 Kh
//   A = Qm Kh^T                      split bf16 (hi*hi + hi*lo + lo*hi)
//   X = V - Kg S,  Q S               f16
//   U = T X                          split bf16 (by blocks: U0 = T00 X0, U1 = T11 (X1 - L10 U0))
//   A U                              split bf16
//   Kbar^T U                         f16                   HP: split bf16
// HP is the variant for correlated keys (the layer's Swish-activated ones): the rounding of L and
// of Kbar^T U grows with the conditioning of I + Diag(beta) L, and HP takes both to split bf16.
// The inverse solves the two 16x16 diagonal blocks of (I + Diag(beta) L) by forward substitution
// in float32, one matrix row per lane, spread over the four value waves.
#include "kda_common.h"
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace bf16path {

constexpr int C = 32;       // tokens per chunk
constexpr int SUB = 16;     // tokens per sub-tile
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVH = 64;     // value columns per workgroup
constexpr int NKW = 8;      // key waves, one 4-token quad of the chunk each
constexpr int TPW = C / NKW; // tokens per key wave
constexpr int NTHR = 64 * (NKW + 4);  // and 4 value waves, 16 value columns each
// LDS layouts.  A matrix-core operand read has lane (l16, g4) fetch 16 bytes from row r0 + l16 at
// 16-byte column block b0 + g4.  Measured on gfx950, such reads run at the full 256 B/clock per CU
// when token-major [C][DK] rows are padded to 288 bytes (272 or 320 bytes run ~1.8x slower), and
// when 64-byte rows of the [rows][C] tiles store column block b at b ^ ((row >> 1) & 3) (unpadded
// or 80-byte rows run ~1.8x slower).
constexpr int LDK = DK + 16; // padded row (16-bit elements) of token-major [C][DK] tiles
constexpr int LDT = C;       // row of the [rows][C] tiles (channel-major [D][C], and [C][C]), swizzled
constexpr int LDA = C;
constexpr int LDF = C + 4;  // [C][C] float tiles
constexpr int LDQ = 2 * NKW + 4;  // padded row of the quad-sum table (16-byte reads hit distinct banks)

// Matrix-core operand order.  A 16x16x32 product takes, in lane group g (lanes 16g..16g+15), the
// eight contraction indices 8g..8g+7.  Accumulator registers hold rows 4g..4g+3 of a 16-row block,
// so to feed accumulators back in as operands the contraction index j of a 32-long sum is mapped to
// {4g + r} (j < 16) and {16 + 4g + r} (j >= 16).  Tiles read as operands store their contraction
// index permuted, position 8g + 4h + r for j = 16h + 4g + r, so that each lane's eight elements are
// contiguous and one 16-byte LDS read fetches them.
__device__ __forceinline__ constexpr int tperm(int j) { return ((j >> 2) & 3) * 8 + (j >> 4) * 4 + (j & 3); }
// the same within each 32-channel block of a 128-channel row
__device__ __forceinline__ constexpr int cperm(int c) { return (c & ~31) + tperm(c & 31); }
// column position of element (row, col) of a [rows][C] tile: 16-byte blocks XOR-swizzled by row
__device__ __forceinline__ constexpr int sw(int row, int col) { return col ^ (((row >> 1) & 3) << 3); }

struct alignas(16) KeyTiles {                // written and read by the key waves within one step
    uint16_t qmh[C][LDK], qml[C][LDK];       // Q * exp(b - b_15)       split bf16
    uint16_t km[C][LDK];                     // K * exp(b - b_15)       bf16
    uint16_t khh[C][LDK], khl[C][LDK];       // K * exp(b_15 - b)       split bf16
    float tot[DK / 2][LDQ];                  // per-quad sums of g (log decay): row = channel pair,
                                             // element 2*quad + (channel & 1)
};
struct alignas(16) Handoff2 {                // key -> value, double buffered by chunk parity
    uint16_t qg[C][LDK];                     // Q * Gamma                 f16, channels cperm'd
    uint16_t kgn[C][LDK];                    // -(K * Gamma)              f16, channels cperm'd
    uint16_t kbh[DK][LDT], kbl[DK][LDT];     // (K * exp(b_last - b))^T   split bf16 (HP), else f16 in kbh;
                                             //                           tokens tperm'd
    uint16_t ah[C][LDA], al[C][LDA];         // A                         split bf16, columns tperm'd
    float gamc[DK];                          // Gamma of the chunk's last token
};
struct alignas(16) Handoff1 {                // key -> value, one buffer (written after the reader is done)
    float lf[C][LDF];                        // L (strictly lower within the diagonal blocks)
    uint16_t vt[DVH][LDT];                   // V^T (this value half)     bf16, tokens tperm'd
    float beta[C];
};
struct alignas(16) ValueTiles {              // value waves only (the key waves write L(1,0) here)
    uint16_t th[C][LDA], tl[C][LDA];         // T split bf16, columns tperm'd; block (1,0) holds L(1,0)
};
struct alignas(16) Smem {
    KeyTiles key;
    Handoff2 h2[2];
    Handoff1 h1;
    ValueTiles val;
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// Lane M of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + M, 0xf, 0xf, true));
}
// Low 16-bit halves of a and b as one word (a's in the low half); likewise the high halves.
__device__ __forceinline__ uint32_t perm_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t perm_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// One key thread's share of one chunk of input, as loaded.  bf16 inputs: q, k, v as packed pairs;
// float32 inputs: q, k as float pairs, and v is read by the value waves themselves.
template <bool IN_F32>
struct Raw;
template <>
struct Raw<false> {
    uint32_t q[TPW], k[TPW], v[TPW];
    f32x2 g[TPW];
    float beta;
};
template <>
struct Raw<true> {
    f32x2 q[TPW], k[TPW];
    f32x2 g[TPW];
    float beta;
};
__device__ __forceinline__ f32x2 unpack_q(uint32_t w) { return f32x2{bf16lo_to_f(w), bf16hi_to_f(w)}; }
__device__ __forceinline__ f32x2 unpack_q(f32x2 w) { return w; }

// Per-thread constants of the key waves' chunk loads (byte offsets within a chunk).
struct KeyLoad {
    uint32_t off[TPW];   // token TPW*kw + i, key channels 2*lane, 2*lane+1 of q/k (g: twice this)
    uint32_t voff[TPW];  // token TPW*kw + i, value columns half*64 + 2*(lane & 31) (+1)
    uint32_t boff;       // beta of token TPW*kw + (lane % TPW)
    uint32_t lane_b, vlane_b, tok_b;  // for the clamped tail loads
    int kw, lane;
};

// A global-memory pointer every lane agrees on, held in scalar registers, so that loads and stores
// use a scalar base plus a 32-bit per-lane offset.
typedef __attribute__((address_space(1))) char gchar;
__device__ __forceinline__ gchar* uniform_gptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (gchar*)(((uint64_t)hi << 32) | lo);
}
template <typename Tv>
__device__ __forceinline__ Tv gload(const gchar* base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(1))) Tv*>(base + off);
}
template <typename Tv>
__device__ __forceinline__ void gstore(gchar* base, uint32_t off, Tv v) {
    *reinterpret_cast<__attribute__((address_space(1))) Tv*>(base + off) = v;
}

// Tokens t0 + TPW*kw + i: key channels 2*lane, 2*lane+1; value columns half*64 + 2*(lane & 31) (+1);
// beta of token t0 + TPW*kw + (lane % TPW).  Tokens past the end read the last valid row; mask_tail()
// zeroes them when the chunk is consumed.  Nothing here uses the loaded values, so the loads stay
// in flight until their first use in the next step.  Requires T >= 1 and t0 < T.
// PART selects what is loaded: LOAD_ALL, LOAD_GVB (decays, values, beta) or LOAD_QK (queries, keys).
// Every step issues the same loads whatever the chunk (past the last one, the last chunk is read
// again and ignored): with no load under a condition the compiler can count the loads issued since
// any register's own, and wait for exactly that one instead of for all of them.
enum { LOAD_ALL = 3, LOAD_GVB = 1, LOAD_QK = 2 };
template <int PART, bool IN_F32>
__device__ __forceinline__ void load_chunk(Raw<IN_F32>& r, const Params& p, const KeyLoad& kl, size_t row0, int t0) {
    constexpr bool LG = PART & LOAD_GVB, LQ = PART & LOAD_QK;
    const size_t ce = (row0 + (size_t)t0 * p.H) * DK;  // element offset of the chunk's first row
    constexpr uint32_t qs = IN_F32 ? 2 : 1;            // q/k byte offsets scale with the element size
    const gchar* qc = uniform_gptr((const char*)p.q + ce * 2 * qs);
    const gchar* kc = uniform_gptr((const char*)p.k + ce * 2 * qs);
    const gchar* gc = uniform_gptr(p.g + ce);
    // v == NULL stands for v = 0 (the transition-matrix run of the in-device context parallelism): the
    // value loads then read the chunk's g instead (a valid address at every value offset, g having
    // twice v's row size) and the reader substitutes zeros
    const gchar* vc = uniform_gptr(p.v ? (const void*)((const uint16_t*)p.v + ce) : (const void*)(p.g + ce));
    const gchar* bc = uniform_gptr(p.beta + row0 + (size_t)t0 * p.H);
    using QT = typename std::conditional<IN_F32, f32x2, uint32_t>::type;
    if (t0 + C <= p.T) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if constexpr (LQ) r.q[i] = gload<QT>(qc, qs * kl.off[i]);
            if constexpr (LQ) r.k[i] = gload<QT>(kc, qs * kl.off[i]);
            if constexpr (LG) r.g[i] = gload<f32x2>(gc, 2 * kl.off[i]);
            if constexpr (LG && !IN_F32) r.v[i] = gload<uint32_t>(vc, kl.voff[i]);
        }
        if constexpr (LG) r.beta = gload<float>(bc, kl.boff);
    } else {
        const int lim = p.T - 1 - t0;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const uint32_t tb = (uint32_t)min(TPW * kl.kw + i, lim) * kl.tok_b;
            const uint32_t o = tb + kl.lane_b, ov = tb + kl.vlane_b;  // both non-negative, < 2^31
            if constexpr (LQ) r.q[i] = gload<QT>(qc, qs * o);
            if constexpr (LQ) r.k[i] = gload<QT>(kc, qs * o);
            if constexpr (LG) r.g[i] = gload<f32x2>(gc, 2 * o);
            if constexpr (LG && !IN_F32) r.v[i] = gload<uint32_t>(vc, ov);
        }
        if constexpr (LG) r.beta = gload<float>(bc, (uint32_t)min(TPW * kl.kw + (kl.lane % TPW), lim) * 4u * p.H);
    }
}

// Zero the tokens at or past T (k = v = 0, beta = 0, g = 0 leaves the state unchanged).
template <bool IN_F32>
__device__ __forceinline__ void mask_tail(Raw<IN_F32>& r, int T, int t0, int kw, int lane) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        if (t0 + TPW * kw + i >= T) {
            r.q[i] = {};
            r.k[i] = {};
            if constexpr (!IN_F32) r.v[i] = 0u;
            r.g[i] = f32x2{0.f, 0.f};
        }
    }
    if (t0 + TPW * kw + (lane % TPW) >= T) r.beta = 0.f;
}

// Factors of the previous chunk that the value-side tiles are made from, kept in registers from
// part 2 of one step to part 1 of the next (the value waves read those tiles only a step later).
struct Carry {
    float qm[TPW][2], km[TPW][2], kh[TPW][2];  // Q, K times exp(b - b_15); K times exp(b_15 - b)
    float eP[2], eC[2], gam[2];                // exp(b_15), exp(b_31 - b_15), exp(b_31)
};

// ------------------------------------------------------------------------------------------------
// key waves: one step = chunk n (nothing when n == nchunk); three barriers
// ------------------------------------------------------------------------------------------------
template <bool IN_F32, bool HP>
__device__ __forceinline__ void key_step(Smem& sm, const Params& p, const KeyLoad& kl, size_t row0, int n,
                                         int nchunk, Raw<IN_F32>& cur, Raw<IN_F32>& nxt, Carry& cy) {
    const int kw = kl.kw, lane = kl.lane;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int c0 = 2 * lane;   // key channels c0, c0 + 1
    const bool work = n < nchunk;
    const int t0 = n * C;
    const int tn = min(t0 + C, (nchunk - 1) * C);  // the chunk prefetched this step (see load_chunk)
    Handoff2& H = sm.h2[n & 1];  // A of chunk n (part 3); its other tiles are written next step

    // ---------------- part 1: decay sums over the quad; prefetch of the next chunk; the previous
    // chunk's value-side tiles (Q*Gamma, -(K*Gamma), Kbar^T, Gamma_last), which its value step reads
    if (work) {
        if (t0 + C > p.T) mask_tail(cur, p.T, t0, kw, lane);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < TPW; ++i) { a0 += cur.g[i][0]; a1 += cur.g[i][1]; }
        *reinterpret_cast<float2*>(&sm.key.tot[lane][2 * kw]) = make_float2(a0, a1);
    }
    load_chunk<LOAD_GVB>(nxt, p, kl, row0, tn);  // part of the next chunk
    if (n >= 1) {
        Handoff2& Hp = sm.h2[(n - 1) & 1];
        const int pc0 = cperm(c0);  // c0 even: c0 + 1 follows it
        const int tq = TPW * kw;
        uint32_t kb[TPW], kl8[TPW], wqg[TPW], wkg[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            wqg[i] = pack_f16(cy.qm[i][0] * cy.eP[0], cy.qm[i][1] * cy.eP[1]);
            wkg[i] = pack_f16(-(cy.km[i][0] * cy.eP[0]), -(cy.km[i][1] * cy.eP[1]));
            if constexpr (HP)
                split_bf16(cy.kh[i][0] * cy.eC[0], cy.kh[i][1] * cy.eC[1], kb[i], kl8[i]);
            else
                kb[i] = pack_f16(cy.kh[i][0] * cy.eC[0], cy.kh[i][1] * cy.eC[1]);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hp.qg[tq + i][pc0]) = wqg[i];
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hp.kgn[tq + i][pc0]) = wkg[i];
        // token pairs of channel c0 (low halves) and of channel c0 + 1 (high halves); the quad's
        // four tokens are contiguous after tperm
        const int pt = tperm(tq);
        auto put_t = [&](uint16_t (*dst)[LDT], const uint32_t* w) {
            *reinterpret_cast<u32x2*>(&dst[c0][sw(c0, pt)]) = u32x2{perm_lo(w[0], w[1]), perm_lo(w[2], w[3])};
            *reinterpret_cast<u32x2*>(&dst[c0 + 1][sw(c0 + 1, pt)]) = u32x2{perm_hi(w[0], w[1]), perm_hi(w[2], w[3])};
        };
        put_t(Hp.kbh, kb);
        if constexpr (HP) put_t(Hp.kbl, kl8);
        if (kw == 0) *reinterpret_cast<float2*>(&Hp.gamc[c0]) = make_float2(cy.gam[0], cy.gam[1]);
    }
    lds_barrier();  // ---- barrier 1

    // ---------------- part 2: all decay factors, relative to the cumulative decay at token 15
    if (work) {
        float tt0[NKW], tt1[NKW];
#pragma unroll
        for (int o = 0; o < NKW; o += 2) {
            const f32x4 t = *reinterpret_cast<const f32x4*>(&sm.key.tot[lane][2 * o]);
            tt0[o] = t[0]; tt1[o] = t[1]; tt0[o + 1] = t[2]; tt1[o + 1] = t[3];
        }
        // p = b at token 15 (the reference), q = b at token 31 minus p, and o = b at the token before
        // this quad minus p, from pair sums of the quad totals (kw is wave-uniform: no divergence)
        const float s01a = tt0[0] + tt0[1], s23a = tt0[2] + tt0[3], s45a = tt0[4] + tt0[5], s67a = tt0[6] + tt0[7];
        const float s01b = tt1[0] + tt1[1], s23b = tt1[2] + tt1[3], s45b = tt1[4] + tt1[5], s67b = tt1[6] + tt1[7];
        const float p0 = s01a + s23a, p1 = s01b + s23b, q0 = s45a + s67a, q1 = s45b + s67b;
        float o0, o1;
        static_assert(NKW == 8, "pair sums below assume eight quads");
        switch (kw) {
            case 0: o0 = -p0; o1 = -p1; break;
            case 1: o0 = -(tt0[1] + s23a); o1 = -(tt1[1] + s23b); break;
            case 2: o0 = -s23a; o1 = -s23b; break;
            case 3: o0 = -tt0[3]; o1 = -tt1[3]; break;
            case 4: o0 = 0.f; o1 = 0.f; break;
            case 5: o0 = tt0[4]; o1 = tt1[4]; break;
            case 6: o0 = s45a; o1 = s45b; break;
            default: o0 = s45a + tt0[6]; o1 = s45b + tt1[6]; break;
        }
        o0 *= kLog2e; o1 *= kLog2e;
        cy.eP[0] = fexp(p0); cy.eP[1] = fexp(p1);
        cy.eC[0] = fexp(q0); cy.eC[1] = fexp(q1);
        cy.gam[0] = cy.eP[0] * cy.eC[0]; cy.gam[1] = cy.eP[1] * cy.eC[1];
        uint32_t wqh[TPW], wql[TPW], wkm[TPW], wkh[TPW], wkl[TPW];
        float y0 = o0, y1 = o1;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            y0 = __builtin_fmaf(cur.g[i][0], kLog2e, y0);  // (b_t - b_15) log2(e)
            y1 = __builtin_fmaf(cur.g[i][1], kLog2e, y1);
            const float e0 = __builtin_amdgcn_exp2f(y0), e1 = __builtin_amdgcn_exp2f(y1);
            const float f0 = __builtin_amdgcn_exp2f(-y0), f1 = __builtin_amdgcn_exp2f(-y1);
            const f32x2 qq = unpack_q(cur.q[i]), kk = unpack_q(cur.k[i]);
            cy.qm[i][0] = qq[0] * e0; cy.qm[i][1] = qq[1] * e1;
            cy.km[i][0] = kk[0] * e0; cy.km[i][1] = kk[1] * e1;
            cy.kh[i][0] = kk[0] * f0; cy.kh[i][1] = kk[1] * f1;
            split_bf16(cy.qm[i][0], cy.qm[i][1], wqh[i], wql[i]);
            wkm[i] = pack_bf16(cy.km[i][0], cy.km[i][1]);
            split_bf16(cy.kh[i][0], cy.kh[i][1], wkh[i], wkl[i]);
        }
        // one array at a time, so that stores of neighbouring tokens pair up
        const int tq = TPW * kw;
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.qmh[tq + i][c0]) = wqh[i];
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.qml[tq + i][c0]) = wql[i];
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.km[tq + i][c0]) = wkm[i];
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khh[tq + i][c0]) = wkh[i];
#pragma unroll
        for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khl[tq + i][c0]) = wkl[i];
        // beta of this chunk (the value waves read the previous chunk's before barrier 1)
        if (lane < TPW) sm.h1.beta[TPW * kw + lane] = cur.beta;
    }
    lds_barrier();  // ---- barrier 2

    // ---------------- part 3: Gram products, and the inputs the value waves read next step
    // the rest of the next chunk (first read in part 2 of the next step), issued here so that the
    // loads are spread over the step rather than queued all at once
    load_chunk<LOAD_QK>(nxt, p, kl, row0, tn);
    if (work) {
        if (kw < 3) {
            // A(0,0), A(1,0), A(1,1): split bf16 with three independent accumulators
            const int R = kw == 0 ? 0 : 1, S = kw == 2 ? 1 : 0;
            const uint16_t(*rh)[LDK] = sm.key.khh + SUB * S;
            const uint16_t(*rl)[LDK] = sm.key.khl + SUB * S;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;  // two chains over alternate channel blocks
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kc = 32 * m + 8 * g4;
                const u32x4 aH = ld16(&sm.key.qmh[SUB * R + l16][kc]);
                const u32x4 aL = ld16(&sm.key.qml[SUB * R + l16][kc]);
                const u32x4 bH = ld16(&rh[l16][kc]);
                const u32x4 bL = ld16(&rl[l16][kc]);
                f32x4& a = (m & 1) ? a1 : a0;
                a = mfma_bf16(aH, bH, a);
                a = mfma_bf16(aH, bL, a);
                a = mfma_bf16(aL, bH, a);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g4 + r;
                float v = a0[r] + a1[r];
                if (R == S && l16 > i) v = 0.f;  // lower triangle including the diagonal
                const uint32_t hi = pack_bf16(v, 0.f);
                const int ac = sw(SUB * R + i, tperm(SUB * S + l16));
                H.ah[SUB * R + i][ac] = hi & 0xffffu;
                H.al[SUB * R + i][ac] = pack_bf16(v - bf16lo_to_f(hi), 0.f) & 0xffffu;
            }
        } else if (kw == 3) {
            // L(0,0), L(1,0), L(1,1): bf16 Km against K/Gamma (split bf16 when HP, else its high part)
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kc = 32 * m + 8 * g4;
                const u32x4 a0 = ld16(&sm.key.km[l16][kc]);
                const u32x4 a1 = ld16(&sm.key.km[SUB + l16][kc]);
                acc0 = mfma_bf16(a0, ld16(&sm.key.khh[l16][kc]), acc0);
                acc1 = mfma_bf16(a1, ld16(&sm.key.khh[l16][kc]), acc1);
                acc2 = mfma_bf16(a1, ld16(&sm.key.khh[SUB + l16][kc]), acc2);
                if constexpr (HP) {
                    acc0 = mfma_bf16(a0, ld16(&sm.key.khl[l16][kc]), acc0);
                    acc1 = mfma_bf16(a1, ld16(&sm.key.khl[l16][kc]), acc1);
                    acc2 = mfma_bf16(a1, ld16(&sm.key.khl[SUB + l16][kc]), acc2);
                }
            }
            // the diagonal blocks as -Diag(beta) L, the form the substitution uses
            const f32x4 nb0 = -*reinterpret_cast<const f32x4*>(&sm.h1.beta[4 * g4]);
            const f32x4 nb1 = -*reinterpret_cast<const f32x4*>(&sm.h1.beta[SUB + 4 * g4]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g4 + r;
                sm.h1.lf[i][l16] = (l16 >= i) ? 0.f : nb0[r] * acc0[r];  // strictly lower
                sm.h1.lf[SUB + i][SUB + l16] = (l16 >= i) ? 0.f : nb1[r] * acc2[r];
                // L(1,0) as a split-bf16 operand, in the block of the T tile that T itself leaves unused
                const uint32_t hi = pack_bf16(acc1[r], 0.f);
                sm.val.th[SUB + i][sw(SUB + i, tperm(l16))] = hi & 0xffffu;
                sm.val.tl[SUB + i][sw(SUB + i, tperm(l16))] = pack_bf16(acc1[r] - bf16lo_to_f(hi), 0.f) & 0xffffu;
            }
        }
        // V^T and beta of this chunk (the value waves are done with the previous ones)
        if constexpr (!IN_F32) {
            if (lane < 32) {  // V^T for value columns 2*lane, 2*lane+1 of this half
                uint32_t v[TPW];
#pragma unroll
                for (int i = 0; i < TPW; ++i) v[i] = p.v ? cur.v[i] : 0u;  // v == NULL: v = 0
                const int pt = tperm(TPW * kw);
                *reinterpret_cast<u32x2*>(&sm.h1.vt[2 * lane][sw(2 * lane, pt)]) = u32x2{perm_lo(v[0], v[1]), perm_lo(v[2], v[3])};
                *reinterpret_cast<u32x2*>(&sm.h1.vt[2 * lane + 1][sw(2 * lane + 1, pt)]) = u32x2{perm_hi(v[0], v[1]), perm_hi(v[2], v[3])};
            }
        }
    }
    lds_barrier();  // ---- barrier 3
}

template <bool IN_F32, bool HP>
__device__ void key_waves(Smem& sm, const Params& p, size_t row0, int half, int kw, int lane, int nchunk) {
    // A's block (0,1) is zero in both buffers; no chunk writes it
    for (int e = 64 * kw + lane; e < 2 * SUB * SUB; e += 64 * NKW) {
        Handoff2& Hz = sm.h2[e >> 8];
        const int r = (e >> 4) & 15, c = tperm(SUB + (e & 15));
        Hz.ah[r][sw(r, c)] = 0; Hz.al[r][sw(r, c)] = 0;
    }
    KeyLoad kl;
    kl.kw = kw;
    kl.lane = lane;
    kl.tok_b = (uint32_t)p.H * DK * 2;
    kl.lane_b = 4 * lane;
    kl.vlane_b = 2 * (half * DVH + 2 * (lane & 31));
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        kl.off[i] = (uint32_t)(TPW * kw + i) * kl.tok_b + kl.lane_b;
        kl.voff[i] = (uint32_t)(TPW * kw + i) * kl.tok_b + kl.vlane_b;
    }
    kl.boff = (uint32_t)(TPW * kw + (lane % TPW)) * 4u * p.H;
    Raw<IN_F32> ra, rb;
    Carry cy;
    load_chunk<LOAD_ALL>(ra, p, kl, row0, 0);
    // two steps per iteration so the prefetch target alternates between two register sets
    for (int n = 0; n <= nchunk; n += 2) {
        key_step<IN_F32, HP>(sm, p, kl, row0, n, nchunk, ra, rb, cy);
        if (n + 1 <= nchunk) key_step<IN_F32, HP>(sm, p, kl, row0, n + 1, nchunk, rb, ra, cy);
    }
}

// ------------------------------------------------------------------------------------------------
// value waves: one step = chunk n-1 (nothing when n == 0); three barriers
// ------------------------------------------------------------------------------------------------
template <bool OUT_F32, bool IN_F32, bool HP, bool CKPT>
__device__ void value_waves(Smem& sm, const Params& p, int bh, size_t row0, int half, int vw, int lane, int nchunk) {
    const int l16 = lane & 15, g4 = lane >> 4;
    ValueTiles& V = sm.val;

    // state: st[cb][r] = S[16*cb + 4*g4 + r][col]
    const int col = half * DVH + 16 * vw + l16;
    f32x4 st[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = 16 * cb + 4 * g4 + r;
            st[cb][r] = p.S0 ? p.S0[((size_t)bh * DK + c) * DV + col] : 0.f;
        }
    }
    // state as f16 operands of the channel contraction, K-step m over channels 32m..32m+31 in the
    // order {32m + 4*g4 + r} then {32m + 16 + 4*g4 + r}; as an A operand it is S^T
    u32x4 sb[4];
    auto make_sb = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m)
            sb[m] = u32x4{pack_f16(st[2 * m][0], st[2 * m][1]), pack_f16(st[2 * m][2], st[2 * m][3]),
                          pack_f16(st[2 * m + 1][0], st[2 * m + 1][1]), pack_f16(st[2 * m + 1][2], st[2 * m + 1][3])};
    };
    make_sb();
    // byte offsets of this lane's output (token 16R + l16 of a chunk, value columns 4*g4..4*g4+3)
    uint32_t ooff[2];
#pragma unroll
    for (int R = 0; R < 2; ++R)
        ooff[R] = ((uint32_t)(SUB * R + l16) * (uint32_t)p.H * DV + half * DVH + 16 * vw + 4 * g4) * (OUT_F32 ? 4u : 2u);

    // float32 inputs: this lane's V values (tokens 16R + 4*g4 + r of a chunk, column col), read one
    // step ahead; rows past T read the last valid row (their U rows come out zero: beta = 0 there)
    f32x4 vnext[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // (v == NULL stands for v = 0: the rows of g, which have v's float32 layout, are read and zeroed)
    auto load_v = [&](int tc0) {
        const size_t e0 = (row0 + (size_t)tc0 * p.H) * DV;
        const gchar* vb = uniform_gptr(p.v ? (const void*)((const float*)p.v + e0) : (const void*)(p.g + e0));
        const int lim = p.T - 1 - tc0;
#pragma unroll
        for (int R = 0; R < 2; ++R)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                vnext[R][r] = gload<float>(vb, ((uint32_t)min(SUB * R + 4 * g4 + r, lim) * (uint32_t)p.H * DV + col) * 4u);
    };
    if constexpr (IN_F32) load_v(0);

    for (int n = 0; n <= nchunk; ++n) {
        const bool work = n >= 1;  // this step handles chunk n-1
        const int t0 = (n - 1) * C;
        const Handoff2& H = sm.h2[(n - 1) & 1];
        // ---------------- part 1: UT inverse of the two diagonal blocks, spread over the value waves
        // Wave vw solves two columns ja, jb of block vw >> 1 of (I + Diag(beta) L) X = I per 16-lane row
        // g4: ja = g4, jb = 12 + g4 (even vw) or ja = 4 + g4, jb = 8 + g4 (odd vw); lane l16 holds matrix
        // row i = l16 of N = -Diag(beta) L.  With x_i = [i == j] + y_i, forward substitution reads
        // y = N e_j + N y: y starts as column j of N, and at step m row m's (final) y_m is broadcast along
        // the 16-lane row and rows below take y_i += N[i][m] y_m.  Rows at or above j keep y = 0, so
        // column j needs steps m > j only, which the column pairing balances.
        if (work) {
            const float* beta = sm.h1.beta;
            const bool odd = vw & 1;
            const int o = SUB * (vw >> 1), i = l16, ja = (odd ? 4 : 0) + g4, jb = (odd ? 8 : 12) + g4;
            float Nr[SUB];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(&sm.h1.lf[o + i][o + 4 * q4]);
                Nr[4 * q4] = t[0]; Nr[4 * q4 + 1] = t[1]; Nr[4 * q4 + 2] = t[2]; Nr[4 * q4 + 3] = t[3];
            }
            float ya = sm.h1.lf[o + i][o + ja], yb = sm.h1.lf[o + i][o + jb];
#define KDA_STEP_A(m) ya = __builtin_fmaf(Nr[m], row_bcast<m>(ya), ya);
#define KDA_STEP_AB(m)                                                                           \
            {                                                                                    \
                const float xa = row_bcast<m>(ya), xb = row_bcast<m>(yb);                        \
                ya = __builtin_fmaf(Nr[m], xa, ya);                                              \
                yb = __builtin_fmaf(Nr[m], xb, yb);                                              \
            }
            if (!odd) {  // columns 0-3 from step 1, columns 12-15 from step 13
                KDA_STEP_A(1) KDA_STEP_A(2) KDA_STEP_A(3) KDA_STEP_A(4) KDA_STEP_A(5) KDA_STEP_A(6)
                KDA_STEP_A(7) KDA_STEP_A(8) KDA_STEP_A(9) KDA_STEP_A(10) KDA_STEP_A(11) KDA_STEP_A(12)
                KDA_STEP_AB(13) KDA_STEP_AB(14)
            } else {     // columns 4-7 from step 5, columns 8-11 from step 9
                KDA_STEP_A(5) KDA_STEP_A(6) KDA_STEP_A(7) KDA_STEP_A(8)
                KDA_STEP_AB(9) KDA_STEP_AB(10) KDA_STEP_AB(11) KDA_STEP_AB(12) KDA_STEP_AB(13) KDA_STEP_AB(14)
            }
#undef KDA_STEP_A
#undef KDA_STEP_AB
            // T = X Diag(beta), as split bf16 in the tperm'd columns of T's tile
            const float ta = ((i == ja ? 1.f : 0.f) + ya) * beta[o + ja];
            const float tb = ((i == jb ? 1.f : 0.f) + yb) * beta[o + jb];
            uint32_t hi, lo;
            split_bf16(ta, tb, hi, lo);
            const int ca = sw(o + i, tperm(o + ja)), cb = sw(o + i, tperm(o + jb));
            V.th[o + i][ca] = hi & 0xffffu;
            V.th[o + i][cb] = hi >> 16;
            V.tl[o + i][ca] = lo & 0xffffu;
            V.tl[o + i][cb] = lo >> 16;
        }
        lds_barrier();  // ---- barrier 1

        // ---------------- part 2: U = T (V - (K*Gamma) S), and (Q*Gamma) S
        f32x4 oacc[2];
        u32x4 uf, uh, ul;
        if (work) {
            // X = V - (K*Gamma) S, started from V in accumulator layout
            f32x4 xr[2];
            if constexpr (IN_F32) {
                xr[0] = p.v ? vnext[0] : f32x4{0.f, 0.f, 0.f, 0.f};
                xr[1] = p.v ? vnext[1] : f32x4{0.f, 0.f, 0.f, 0.f};
                load_v(min(n, nchunk - 1) * C);  // V of the chunk handled next step (unconditionally, as above)
            } else {
                const u32x4 vv = ld16(&sm.h1.vt[16 * vw + l16][sw(l16, 8 * g4)]);  // tokens 4g4+r, then 16+4g4+r
                xr[0] = f32x4{bf16lo_to_f(vv.x), bf16hi_to_f(vv.x), bf16lo_to_f(vv.y), bf16hi_to_f(vv.y)};
                xr[1] = f32x4{bf16lo_to_f(vv.z), bf16hi_to_f(vv.z), bf16lo_to_f(vv.w), bf16hi_to_f(vv.w)};
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int R = 0; R < 2; ++R)
                    xr[R] = mfma_f16(ld16(&H.kgn[SUB * R + l16][32 * m + 8 * g4]), sb[m], xr[R]);
            }
            // (Q*Gamma) S as O^T: lane (token l16, group g4) gets value columns 4*g4..4*g4+3
#pragma unroll
            for (int R = 0; R < 2; ++R) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < 4; ++m) acc = mfma_f16(sb[m], ld16(&H.qg[SUB * R + l16][32 * m + 8 * g4]), acc);
                oacc[R] = acc;
            }
            // U by block forward substitution over the two sub-tiles (T is block lower triangular):
            //   U0 = T00 X0,   U1 = T11 (X1 - L10 U0),
            // as split-bf16 16x16x16 products whose contraction index is token 4*g4 + r of a sub-tile
            auto split4 = [](const f32x4 x, u32x2& h, u32x2& l) {
                uint32_t h0, h1, l0, l1;
                split_bf16(x[0], x[1], h0, l0);
                split_bf16(x[2], x[3], h1, l1);
                h = u32x2{h0, h1};
                l = u32x2{l0, l1};
            };
            auto prod3 = [](u32x2 aH, u32x2 aL, u32x2 bH, u32x2 bL) {
                f32x4 a = mfma_bf16_k16(aH, bH, f32x4{0.f, 0.f, 0.f, 0.f});
                a = mfma_bf16_k16(aH, bL, a);
                return mfma_bf16_k16(aL, bH, a);
            };
            auto ld8 = [](const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); };
            f32x4 u[2];
            u32x2 bh, bl;
            split4(xr[0], bh, bl);
            const int c0s = sw(l16, 8 * g4);  // (rows l16 and SUB + l16 share the swizzle)
            u[0] = prod3(ld8(&V.th[l16][c0s]), ld8(&V.tl[l16][c0s]), bh, bl);
            split4(u[0], bh, bl);
            const f32x4 lu = prod3(ld8(&V.th[SUB + l16][c0s]), ld8(&V.tl[SUB + l16][c0s]), bh, bl);
            split4(xr[1] - lu, bh, bl);
            u[1] = prod3(ld8(&V.th[SUB + l16][c0s + 4]), ld8(&V.tl[SUB + l16][c0s + 4]), bh, bl);
            if constexpr (!HP)
                uf = u32x4{pack_f16(u[0][0], u[0][1]), pack_f16(u[0][2], u[0][3]), pack_f16(u[1][0], u[1][1]),
                           pack_f16(u[1][2], u[1][3])};
            uint32_t uh0, uh1, uh2, uh3, ul0, ul1, ul2, ul3;
            split_bf16(u[0][0], u[0][1], uh0, ul0);
            split_bf16(u[0][2], u[0][3], uh1, ul1);
            split_bf16(u[1][0], u[1][1], uh2, ul2);
            split_bf16(u[1][2], u[1][3], uh3, ul3);
            uh = u32x4{uh0, uh1, uh2, uh3};
            ul = u32x4{ul0, ul1, ul2, ul3};
        }
        lds_barrier();  // ---- barrier 2

        // ---------------- part 3: O += A U, output; S <- Diag(Gamma_last) S + Kbar^T U
        if (work) {
            if (p.o) {  // (o == NULL: a state-only run of the in-device context parallelism)
                gchar* ob = (gchar*)uniform_gptr((const char*)p.o + ((row0 + (size_t)t0 * p.H) * DV) * (OUT_F32 ? 4 : 2));
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const u32x4 aH = ld16(&H.ah[SUB * R + l16][sw(l16, 8 * g4)]);
                    const u32x4 aL = ld16(&H.al[SUB * R + l16][sw(l16, 8 * g4)]);
                    f32x4 acc = mfma_bf16(uh, aH, oacc[R]);
                    acc = mfma_bf16(ul, aH, acc);
                    acc = mfma_bf16(uh, aL, acc);
                    if (p.scale != 1.f) acc *= p.scale;
                    if (t0 + SUB * R + l16 < p.T) {
                        if constexpr (OUT_F32)
                            gstore<f32x4>(ob, ooff[R], acc);
                        else
                            gstore<u32x2>(ob, ooff[R], u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])});
                    }
                }
            }
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(&H.gamc[16 * cb + 4 * g4]);
                const u32x4 aH = ld16(&H.kbh[16 * cb + l16][sw(l16, 8 * g4)]);
                if constexpr (HP) {
                    const u32x4 aL = ld16(&H.kbl[16 * cb + l16][sw(l16, 8 * g4)]);
                    f32x4 acc = mfma_bf16(aH, uh, st[cb] * gm);
                    acc = mfma_bf16(aH, ul, acc);
                    st[cb] = mfma_bf16(aL, uh, acc);
                } else {
                    st[cb] = mfma_f16(aH, uf, st[cb] * gm);
                }
            }
            make_sb();
            if (CKPT && n % p.ckpt_chunks == 0 && n / p.ckpt_chunks <= p.n_ckpt) {
                // the state after tokens [0, n*C): checkpoint n / ckpt_chunks - 1
                float* dst = p.S_ckpt + ((size_t)bh * p.n_ckpt + (n / p.ckpt_chunks - 1)) * DK * DV;
#pragma unroll
                for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(16 * cb + 4 * g4 + r) * DV + col] = st[cb][r];
            }
        }
        lds_barrier();  // ---- barrier 3
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

// CKPT: S_ckpt is set (a separate instantiation keeps the plain forward free of the checkpoint code)
template <bool OUT_F32, bool IN_F32, bool HP, bool CKPT>
__global__ void __launch_bounds__(NTHR, 1) kda_fwd_bf16_kernel(Params p) {
    __shared__ Smem sm;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

    // workgroup -> (batch*head, value half); both halves of a head land on the same XCD
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
    const size_t row0 = (size_t)b * p.tstride * p.H + h;  // row of token 0: (b*tstride + t)*H + h = row0 + t*H
    const int nchunk = (p.T + C - 1) / C;
    if (nchunk == 0) return;  // (the host runs the state copy instead; every wave leaves here alike)

    if (wave < NKW)
        key_waves<IN_F32, HP>(sm, p, row0, half, wave, lane, nchunk);
    else
        value_waves<OUT_F32, IN_F32, HP, CKPT>(sm, p, bh, row0, half, wave - NKW, lane, nchunk);
}

}  // namespace bf16path

namespace bf16path {
template <bool CKPT>
void launch_bf16_io(const Params& p, hipStream_t stream, dim3 grid, dim3 block) {
    if (p.o_f32 && p.precise)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, false, true, CKPT>), grid, block, 0, stream, p);
    else if (p.o_f32)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, false, false, CKPT>), grid, block, 0, stream, p);
    else if (p.precise)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, true, CKPT>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, false, CKPT>), grid, block, 0, stream, p);
}
}  // namespace bf16path

hipError_t launch_fwd_bf16(const Params& p, hipStream_t stream) {
    using namespace bf16path;
    if (p.T == 0) return launch_state_copy(p, stream);
    const dim3 grid(2 * p.B * p.H), block(NTHR);
    if (p.in_f32)  // the layer's variant (it records no checkpoints)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, true, true, false>), grid, block, 0, stream, p);
    else if (p.S_ckpt)
        launch_bf16_io<true>(p, stream, grid, block);
    else
        launch_bf16_io<false>(p, stream, grid, block);
    return hipGetLastError();
}

}  // namespace kda
