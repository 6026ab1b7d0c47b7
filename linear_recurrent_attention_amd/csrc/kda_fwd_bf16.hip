// Chunkwise KDA forward for bf16 (or float32) q/k/v, float32 g/beta/state, d_k = d_v = 128, on gfx950.
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
//
// Decay factors.  Every factor is taken relative to the cumulative decay at the chunk's token 15:
// Qm = Q*exp(b - b_15), Km = K*exp(b - b_15), Kh = K*exp(b_15 - b).  With the lower bound g >= -5
// of sections 3.1-3.2 each factor lies in [e^-80, e^80], inside the normal range of float32 and
// bf16; the products that enter L and A (t >= s) are at most 1.  The inter-chunk products reuse
// the same tiles by moving exp(b_15) onto the state: (K*Gamma) S = Km (Diag(exp(b_15)) S), and
// likewise for Q.  The value waves keep the state in that row-scaled frame for the whole run,
// R = -2^(64 + kappa) S per row, with kappa = round(b_15 log2 e) an integer: the power of two is exact,
// and the rest of exp(b_15), 2^delta with |delta| <= 1/2, is carried by the factor tiles (Qm, Km and
// Kh take 2^(+-delta); the Gram products do not see it).  R itself is the state operand, so no
// per-row scaling is applied when it is split into matrix-core operands.  With the factor 2^64 both R
// (>= 2^-52 |S|) and every product Km R (<= 2^64 |S|) stay normal for any state with
// 2^-75 <= |S| < 2^60, so the result does not depend on the scale of v and S0 (the recurrence is
// linear in them).  The rest of the value path carries the matching powers of two, all exact:
//   X~ = 2^64 V + Km R              = 2^64 (V - (K*Gamma) S)
//   T' = 2^-64 T,  L10' = 2^64 L10  so U = T' X~ comes out unscaled (block forward substitution
//                                   over the two 16-token sub-tiles: U0 = T'00 X~0,
//                                   U1 = T'11 (X~1 - L10' U0))
//   A'' = -2^64 A,                  O = -2^-64 (Qm R + A'' U)
//   R <- Diag(rho) R + Kbar'^T U    rho = 2^(kappa' - kappa) exp(b_31),  Kbar' = -2^(64 + kappa') K exp(b_31 - b)
// with kappa' that of the next chunk (0 after the last one, which leaves R = -2^64 S_T).  S0 enters as
// Diag(-2^(64 + kappa)) S0 and checkpoints leave as R times the exact reciprocal of that power of two,
// so a run resumed from a checkpoint or cut at a chunk boundary reproduces the uncut run bit for bit.
//
// Mapping.  One workgroup per (batch, head, value half): the 128 value columns are split over two
// workgroups that both compute the key-side products, so 2*B*H workgroups fill the chip; the two
// halves of a head are placed on the same XCD so their common reads of q, k, g share its L2.
// Each workgroup runs 16 waves, four per SIMD, in three roles:
//   key waves 0-7     wave kw owns tokens 4kw..4kw+3 of a chunk (two key channels per lane): decay
//                     sums, exponentials and operand tiles, two chunks ahead of the value waves;
//                     Kbar^T one chunk ahead;
//   value waves 8-11  wave 8+w owns 16 value columns of the float32 state (all 128 rows) in
//                     matrix-core accumulator layout for the whole run: the products with the state,
//                     U, the output and the state update of one chunk per step;
//   helper waves 12-15  the L Gram products (waves 12, 13) and the A Gram half-sums (14, 15), the UT
//                     inverse and A from its half-sums, one chunk ahead;
//                     the v loads of the value waves (staged through LDS).
// A step has three parts separated by workgroup barriers.  A single wave issues at most one vector
// instruction every ~9 clocks on gfx950, while a SIMD shared by four waves issues one every ~2.5;
// the parts are laid out so that each SIMD always has its four waves' work to interleave, and the
// value waves, which carry the serial chain, issue at the highest priority (the helper waves next).
// Tiles pass between roles through LDS, double buffered by chunk parity (the state scalings by chunk
// index mod 3).

// Matrix-core operands (v_mfma_f32_16x16x32_bf16 and 16x16x16, float32 accumulate; "split" is
// hi = bf16(x), lo = bf16(x - hi), products hi*hi + hi*lo + lo*hi):
//   L = Km Kh^T         bf16 (PRECISE: Kh split)       A = Qm Kh^T        split
//   X~ = 2^64 V + Km R  Km bf16, R split                Qm R               split
//   U = T' X~           split                          A'' U              split
//   Kbar^T U            split
// The inverse solves the two 16x16 diagonal blocks of (I + Diag(beta) L) by forward substitution
// in float32, one matrix row per lane, spread over the four helper waves.
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
constexpr int NVW = 4;      // value waves, 16 value columns (all 128 state rows) each
constexpr int NHW = 4;      // helper waves
constexpr int NTHR = 64 * (NKW + NVW + NHW);
constexpr float kUp = 18446744073709551616.f;     // 2^64
constexpr float kDown = 5.42101086242752217e-20f;  // 2^-64
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
// Physical row of channel r in the Kbar^T tiles.  A key wave stores one 8-byte quarter-row of 64
// channels 2 apart in one instruction; with rows in channel order those stores fall on 8 of the 16
// reachable 8-byte bank positions of a 256-byte LDS line (row bit 1 repeats the swizzle's bit), and
// row bits 3-4 folded into bits 0-1 of the row spread them over all 16.  The reads of a 16-row slab
// touch the same rows in another order.  (The float32-input variant keeps channel order: it has no
// VGPRs to spare for the permuted addresses.)
template <bool IN_F32>
__device__ __forceinline__ constexpr int kbrow(int r) { return IN_F32 ? r : r ^ ((r >> 3) & 3); }

// Token-major tiles store channels in cperm order, so that a 16-byte read of a row gives the eight
// channels a lane contracts over in the state products (whose operand comes straight from the
// accumulator layout of the state); the Gram products see the same order on both sides.
struct alignas(16) KeyTiles {                // key waves (written in part 3, read in part 2 of the next step)
    uint16_t khh[C][LDK], khl[C][LDK];       // K * exp(b_15 - b)         split bf16
    float tot[DK / 2][LDQ];                  // per-quad sums of g (log decay): row = channel pair,
                                             // element 2*quad + (channel & 1)
};
struct alignas(16) ChunkTiles {              // between roles, double buffered by chunk parity
    uint16_t qmh[C][LDK], qml[C][LDK];       // Q * exp(b - b_15)         split bf16
    uint16_t km[C][LDK];                     // K * exp(b - b_15)         bf16
    uint16_t kbh[DK][LDT], kbl[DK][LDT];     // Kbar'^T split bf16, tokens tperm'd, rows kbrow(channel)
    uint16_t ah[C][LDA], al[C][LDA];         // -2^64 A                   split bf16, columns tperm'd
    uint16_t th[C][LDA], tl[C][LDA];         // 2^-64 T split bf16, columns tperm'd; block (1,0) holds
                                             // 2^64 L(1,0)
    float beta[C];
};
struct alignas(16) Scalings {                // state scalings of one chunk, by chunk index mod 3
    float ep[DK];                            // -2^(64 + kappa)           row scale R = ep S of the state entering
                                             //                           the chunk (kappa = round(b_15 log2 e))
    float gam[DK];                           // rho = 2^(kappa' - kappa) exp(b_31), kappa' the next chunk's
};
struct alignas(16) VStage {                  // 2^64 v of one chunk, loaded by the helper waves for the value
    float x[NVW][2][64][4];                  // waves: [value wave][R][lane][r] = token 16R + 4*g4 + r of the
                                             // lane's column (zero past T, or when v == NULL); each 16-byte
                                             // access of a wave covers 1 KB contiguously (no bank conflicts)
};
struct alignas(16) Single {                  // written and read within one step
    float lf[C][LDF];                        // -Diag(beta) L on the two diagonal blocks
    float apart[6][4][64];                   // A: partial sums over channels 0-63 / 64-127 of its three
                                             // 16x16 blocks, in accumulator layout [block, half][r][lane]
};
struct alignas(16) Smem {
    KeyTiles key;
    ChunkTiles ch[2];
    Scalings sc[3];
    VStage vs[2];                            // by chunk parity
    Single s;
};

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
// Lane M of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + M, 0xf, 0xf, true));
}

// One key thread's share of one chunk of input, as loaded: q, k as packed bf16 pairs (float pairs
// for float32 inputs), g as float pairs, and one beta.
template <bool IN_F32>
struct Raw {
    using QT = typename std::conditional<IN_F32, f32x2, uint32_t>::type;
    QT q[TPW], k[TPW];
    f32x2 g[TPW];
    float beta;
};
__device__ __forceinline__ f32x2 unpack_q(uint32_t w) { return f32x2{bf16lo_to_f(w), bf16hi_to_f(w)}; }
__device__ __forceinline__ f32x2 unpack_q(f32x2 w) { return w; }

// Per-thread constants of the key waves' chunk loads (byte offsets within a chunk).
struct KeyLoad {
    uint32_t off[TPW];   // token TPW*kw + i, key channels 2*lane, 2*lane+1 of bf16 q/k
    uint32_t goff[TPW];  // the same for float32 g (and float32 q/k): twice off
    uint32_t boff;       // beta of token TPW*kw + (lane % TPW)
    uint32_t lane_b, tok_b;  // for the clamped tail loads
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

// Tokens t0 + TPW*kw + i: key channels 2*lane, 2*lane+1; beta of token t0 + TPW*kw + (lane % TPW).
// Tokens past the end read the last valid row; mask_tail() zeroes them when the chunk is consumed.
// Nothing here uses the loaded values, so the loads stay in flight until their first use in the
// next step.  Requires T >= 1 and t0 < T.
// PART selects what is loaded: LOAD_ALL, LOAD_GB (decays, beta) or LOAD_QK (queries, keys).
// Every step issues the same loads whatever the chunk (past the last one, the last chunk is read
// again and ignored): with no load under a condition the compiler can count the loads issued since
// any register's own, and wait for exactly that one instead of for all of them.
enum { LOAD_ALL = 3, LOAD_GB = 1, LOAD_QK = 2 };
template <int PART, bool IN_F32>
__device__ __forceinline__ void load_chunk(Raw<IN_F32>& r, const Params& p, const KeyLoad& kl, size_t row0, int t0) {
    constexpr bool LG = PART & LOAD_GB, LQ = PART & LOAD_QK;
    const size_t ce = (row0 + (size_t)t0 * p.H) * DK;  // element offset of the chunk's first row
    constexpr uint32_t qs = IN_F32 ? 2 : 1;            // q/k byte offsets scale with the element size
    const gchar* qc = uniform_gptr((const char*)p.q + ce * 2 * qs);
    const gchar* kc = uniform_gptr((const char*)p.k + ce * 2 * qs);
    const gchar* gc = uniform_gptr(p.g + ce);
    const gchar* bc = uniform_gptr(p.beta + row0 + (size_t)t0 * p.H);
    using QT = typename Raw<IN_F32>::QT;
    // Offsets grow with the token, so tokens past the end are clamped to the last valid one by a min on
    // the byte offset (no clamp at all for a full chunk: a bound of ~0).
    const bool full = t0 + C <= p.T;
    const uint32_t lim = (uint32_t)(p.T - 1 - t0);
    const uint32_t lq = full ? ~0u : lim * kl.tok_b + kl.lane_b;  // bf16 q/k bound
    const uint32_t lg = full ? ~0u : 2u * (lim * kl.tok_b + kl.lane_b);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const uint32_t oq = IN_F32 ? min(kl.goff[i], lg) : min(kl.off[i], lq);
        if constexpr (LQ) r.q[i] = gload<QT>(qc, oq);
        if constexpr (LQ) r.k[i] = gload<QT>(kc, oq);
        if constexpr (LG) r.g[i] = gload<f32x2>(gc, min(kl.goff[i], lg));
    }
    if constexpr (LG) r.beta = gload<float>(bc, min(kl.boff, full ? ~0u : lim * 4u * (uint32_t)p.H));
}

// Zero the tokens at or past T (k = v = 0, beta = 0, g = 0 leaves the state unchanged; the value
// waves zero their v rows there themselves).
template <bool IN_F32>
__device__ __forceinline__ void mask_tail(Raw<IN_F32>& r, int T, int t0, int kw, int lane) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        if (t0 + TPW * kw + i >= T) {
            r.q[i] = {};
            r.k[i] = {};
            r.g[i] = f32x2{0.f, 0.f};
        }
    }
    if (t0 + TPW * kw + (lane % TPW) >= T) r.beta = 0.f;
}

// Values of one chunk kept in registers across parts and steps by a key wave: the exponentials of
// part 2 (used in part 3), and the factors its Kbar^T tile is made from (used in part 1 of the next
// step).
struct Carry {
    float e[TPW][2], f[TPW][2];  // 2^(y + delta), 2^-(y + delta) with y = (b - b_15) log2(e)
    float kh[TPW][2];            // K times 2^-(y + delta)
    float eC[2];                 // 2^((b_31 - b_15) log2(e) + delta)
    float a[2];                  // b_31 log2(e) - kappa (key wave 0: the row decay of the next step)
};

// Split x into bf16 hi + lo, packing the pair (a, b) into one word of each (a in the low half).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) { split_bf16(a, b, hi, lo); }

// ------------------------------------------------------------------------------------------------
// key waves.  Step n forms the factors of chunk n+1 and the Kbar^T tile of
// chunk n.  Three barriers per step; steps n = -1 .. nchunk.
// ------------------------------------------------------------------------------------------------
template <bool IN_F32, bool SO>
__device__ __forceinline__ void key_step(Smem& sm, const Params& p, const KeyLoad& kl, size_t row0, int n,
                                         int nchunk, Raw<IN_F32>& cur, Raw<IN_F32>& nxt, Carry& cy) {
    const int kw = kl.kw, lane = kl.lane;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int c0 = 2 * lane;   // key channels c0, c0 + 1
    const int pc0 = cperm(c0); // (c0 even: c0 + 1 follows it)
    const int tq = TPW * kw;
    const int nf = n + 1;                     // chunk whose factors this step forms
    const bool fwork = nf < nchunk;
    const bool gwork = n >= 0 && n < nchunk;  // chunk n: Kbar^T
    const int t0 = nf * C;
    const int tn = min(t0 + C, (nchunk - 1) * C);  // the chunk prefetched this step (see load_chunk)
    ChunkTiles& Hf = sm.ch[nf & 1];
    ChunkTiles& Hg = sm.ch[n & 1];

    // ---------------- part 1: decay sums of chunk n+1 over the quad; prefetch
    if (fwork) {
        if (t0 + C > p.T) mask_tail(cur, p.T, t0, kw, lane);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int i = 0; i < TPW; ++i) { a0 += cur.g[i][0]; a1 += cur.g[i][1]; }
        *reinterpret_cast<float2*>(&sm.key.tot[lane][2 * kw]) = make_float2(a0, a1);
    }
    load_chunk<LOAD_GB>(nxt, p, kl, row0, tn);  // part of the chunk after
    lds_barrier();  // ---- barrier 1

    // ---------------- part 2: decays, row scales and exponentials of chunk n+1; the row decay and the
    // Kbar^T tile of chunk n (the Gram products of chunk n are the helper waves')
    float kap0 = 0.f, kap1 = 0.f;  // kappa of chunk n+1 (0 past the last chunk: the state leaves unscaled)
    float eCn0 = 0.f, eCn1 = 0.f, an0 = 0.f, an1 = 0.f;
    if (fwork) {
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
        // b_15 log2(e) = kappa + delta, kappa an integer, |delta| <= 1/2: the state carries 2^kappa of
        // exp(b_15) (exactly, as a power of two) and the factors carry 2^delta
        const float lp0 = p0 * kLog2e, lp1 = p1 * kLog2e;
        kap0 = __builtin_rintf(lp0); kap1 = __builtin_rintf(lp1);
        const float d0 = lp0 - kap0, d1 = lp1 - kap1;
        o0 = __builtin_fmaf(o0, kLog2e, d0); o1 = __builtin_fmaf(o1, kLog2e, d1);
        eCn0 = __builtin_amdgcn_exp2f(__builtin_fmaf(q0, kLog2e, d0));
        eCn1 = __builtin_amdgcn_exp2f(__builtin_fmaf(q1, kLog2e, d1));
        an0 = __builtin_fmaf(p0 + q0, kLog2e, -kap0); an1 = __builtin_fmaf(p1 + q1, kLog2e, -kap1);
        if (kw == 0) {  // the row scale -2^(64 + kappa) of chunk n+1 (the state's entry scaling, checkpoints)
            Scalings& Sf = sm.sc[nf % 3];
            *reinterpret_cast<float2*>(&Sf.ep[c0]) =
                make_float2(__builtin_amdgcn_ldexpf(-1.f, 64 + (int)kap0), __builtin_amdgcn_ldexpf(-1.f, 64 + (int)kap1));
        }
        float y0 = o0, y1 = o1;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            y0 = __builtin_fmaf(cur.g[i][0], kLog2e, y0);  // (b_t - b_15) log2(e)
            y1 = __builtin_fmaf(cur.g[i][1], kLog2e, y1);
            cy.e[i][0] = __builtin_amdgcn_exp2f(y0); cy.e[i][1] = __builtin_amdgcn_exp2f(y1);
            cy.f[i][0] = __builtin_amdgcn_exp2f(-y0); cy.f[i][1] = __builtin_amdgcn_exp2f(-y1);
        }
        if (lane < TPW) Hf.beta[TPW * kw + lane] = cur.beta;
    }
    if (gwork) {
        // chunk n, in the state's row-scaled frame R = -2^(64 + kappa) S: R <- rho R + Kbar'^T U with
        //   rho   = 2^(kappa_{n+1} - kappa_n) exp(b_31)          = 2^kappa_{n+1} 2^(b_31 log2(e) - kappa_n)
        //   Kbar' = -2^(64 + kappa_{n+1}) K exp(b_31 - b)        = -2^(64 + kappa_{n+1}) Kh eC
        // (the powers of two applied last, exactly, so that a run cut at a chunk boundary and resumed from
        // its unscaled state reproduces the uncut run bit for bit)
        if (kw == 0) {
            Scalings& Sg = sm.sc[n % 3];
            *reinterpret_cast<float2*>(&Sg.gam[c0]) =
                make_float2(__builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(cy.a[0]), (int)kap0),
                            __builtin_amdgcn_ldexpf(__builtin_amdgcn_exp2f(cy.a[1]), (int)kap1));
        }
        // per channel, token pairs (0,1) and (2,3) of the quad, contiguous after tperm
        const int s0 = 64 + (int)kap0, s1 = 64 + (int)kap1;
        uint32_t h[2][2], l[2][2];
        float x[2][TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            x[0][i] = __builtin_amdgcn_ldexpf(-(cy.kh[i][0] * cy.eC[0]), s0);
            x[1][i] = __builtin_amdgcn_ldexpf(-(cy.kh[i][1] * cy.eC[1]), s1);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            split2(x[c][0], x[c][1], h[c][0], l[c][0]);
            split2(x[c][2], x[c][3], h[c][1], l[c][1]);
        }
        const int pt = tperm(tq);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            *reinterpret_cast<u32x2*>(&Hg.kbh[kbrow<IN_F32>(c0 + c)][sw(c0 + c, pt)]) = u32x2{h[c][0], h[c][1]};
            *reinterpret_cast<u32x2*>(&Hg.kbl[kbrow<IN_F32>(c0 + c)][sw(c0 + c, pt)]) = u32x2{l[c][0], l[c][1]};
        }
    }
    if (fwork) {
        cy.eC[0] = eCn0; cy.eC[1] = eCn1;
        cy.a[0] = an0; cy.a[1] = an1;
    }
    lds_barrier();  // ---- barrier 2

    // ---------------- part 3: operand tiles of chunk n+1
    // the rest of the chunk after (first read in part 3 of the next step), issued here so that the
    // loads are spread over the step rather than queued all at once
    load_chunk<LOAD_QK>(nxt, p, kl, row0, tn);
    if (fwork) {
        // Layer by layer across the quad (unpack and products, hi, remainders, lo), with scheduling
        // barriers between layers: each layer is a set of independent instructions, so a wave
        // issues them back to back instead of waiting on each result in turn.
        // Qm serves only the output (Qm P and A): the state-only instantiation forms the key tiles alone.
        if constexpr (!SO) {
            uint32_t wqh[TPW], wql[TPW], wkm[TPW], wkh[TPW], wkl[TPW];
            f32x2 qe[TPW], ke[TPW], kf[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const f32x2 qq = unpack_q(cur.q[i]), kk = unpack_q(cur.k[i]);
                qe[i] = f32x2{qq[0] * cy.e[i][0], qq[1] * cy.e[i][1]};
                ke[i] = f32x2{kk[0] * cy.e[i][0], kk[1] * cy.e[i][1]};
                cy.kh[i][0] = kk[0] * cy.f[i][0]; cy.kh[i][1] = kk[1] * cy.f[i][1];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                wqh[i] = pack_bf16(qe[i][0], qe[i][1]);
                wkm[i] = pack_bf16(ke[i][0], ke[i][1]);
                wkh[i] = pack_bf16(cy.kh[i][0], cy.kh[i][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                qe[i] = f32x2{remainder_lo(wqh[i], qe[i][0]), remainder_hi(wqh[i], qe[i][1])};
                kf[i] = f32x2{remainder_lo(wkh[i], cy.kh[i][0]), remainder_hi(wkh[i], cy.kh[i][1])};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                wql[i] = pack_bf16(qe[i][0], qe[i][1]);
                wkl[i] = pack_bf16(kf[i][0], kf[i][1]);
            }
            // one array at a time, so that stores of neighbouring tokens pair up
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hf.qmh[tq + i][pc0]) = wqh[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hf.qml[tq + i][pc0]) = wql[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hf.km[tq + i][pc0]) = wkm[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khh[tq + i][pc0]) = wkh[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khl[tq + i][pc0]) = wkl[i];
        } else {
            uint32_t wkm[TPW], wkh[TPW], wkl[TPW];
            f32x2 ke[TPW], kf[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const f32x2 kk = unpack_q(cur.k[i]);
                ke[i] = f32x2{kk[0] * cy.e[i][0], kk[1] * cy.e[i][1]};
                cy.kh[i][0] = kk[0] * cy.f[i][0]; cy.kh[i][1] = kk[1] * cy.f[i][1];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                wkm[i] = pack_bf16(ke[i][0], ke[i][1]);
                wkh[i] = pack_bf16(cy.kh[i][0], cy.kh[i][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) kf[i] = f32x2{remainder_lo(wkh[i], cy.kh[i][0]), remainder_hi(wkh[i], cy.kh[i][1])};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TPW; ++i) wkl[i] = pack_bf16(kf[i][0], kf[i][1]);
            // one array at a time, so that stores of neighbouring tokens pair up
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&Hf.km[tq + i][pc0]) = wkm[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khh[tq + i][pc0]) = wkh[i];
#pragma unroll
            for (int i = 0; i < TPW; ++i) *reinterpret_cast<uint32_t*>(&sm.key.khl[tq + i][pc0]) = wkl[i];
        }
    }
    lds_barrier();  // ---- barrier 3
}

template <bool IN_F32, bool SO>
__device__ __forceinline__ void key_waves(Smem& sm, const Params& p, size_t row0, int kw, int lane, int nchunk) {
    KeyLoad kl;
    kl.kw = kw;
    kl.lane = lane;
    kl.tok_b = (uint32_t)p.H * DK * 2;
    kl.lane_b = 4 * lane;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        kl.off[i] = (uint32_t)(TPW * kw + i) * kl.tok_b + kl.lane_b;
        kl.goff[i] = 2u * kl.off[i];
    }
    kl.boff = (uint32_t)(TPW * kw + (lane % TPW)) * 4u * p.H;
    Raw<IN_F32> ra, rb;
    Carry cy;
    load_chunk<LOAD_ALL>(ra, p, kl, row0, 0);
    // two steps per iteration so the prefetch target alternates between two register sets
    for (int n = -1; n <= nchunk; n += 2) {
        key_step<IN_F32, SO>(sm, p, kl, row0, n, nchunk, ra, rb, cy);
        if (n + 1 <= nchunk) key_step<IN_F32, SO>(sm, p, kl, row0, n + 1, nchunk, rb, ra, cy);
    }
}

// ------------------------------------------------------------------------------------------------
// helper waves.  Step n: the L Gram products (part 2), then the UT inverse and A (part 3) of chunk n.
// ------------------------------------------------------------------------------------------------
template <bool IN_F32, bool HP, bool SO>
__device__ __forceinline__ void helper_waves(Smem& sm, const Params& p, size_t row0, int half, int hw, int lane, int nchunk) {
    const int l16 = lane & 15, g4 = lane >> 4;
    // v for value wave hw: this lane's values are tokens 16R + 4*g4 + r of a chunk, column col, read one
    // step ahead into registers and staged in LDS a step before their use.  Rows past T read the last
    // valid row and are zeroed when staged.  v == NULL stands for v = 0: the rows of g are read instead
    // (valid at every offset v would use).  These waves store nothing to global memory, so waiting for
    // their loads never waits for a store.
    using VT = typename std::conditional<IN_F32, float, uint16_t>::type;
    const int col = half * DVH + 16 * hw + l16;
    const uint32_t vrow = (uint32_t)p.H * DV * (uint32_t)sizeof(VT);  // bytes between tokens
    const uint32_t vcol = (uint32_t)col * (uint32_t)sizeof(VT);
    VT vr[2][4];
    uint32_t voff[2][4];  // byte offsets of this lane's values within a chunk
#pragma unroll
    for (int R = 0; R < 2; ++R)
#pragma unroll
        for (int r = 0; r < 4; ++r) voff[R][r] = (uint32_t)(SUB * R + 4 * g4 + r) * vrow + vcol;
    auto load_v = [&](int tc0) {
        const size_t e0 = (row0 + (size_t)tc0 * p.H) * DV;
        const gchar* vb = uniform_gptr(p.v ? (const void*)((const VT*)p.v + e0) : (const void*)(p.g + e0));
        // offsets grow with the row, so a row past T is clamped to row T-1 by a min on the offset
        const uint32_t last = tc0 + C <= p.T ? 0xffffffffu : (uint32_t)(p.T - 1 - tc0) * vrow + vcol;
#pragma unroll
        for (int R = 0; R < 2; ++R)
#pragma unroll
            for (int r = 0; r < 4; ++r) vr[R][r] = gload<VT>(vb, min(voff[R][r], last));
    };
    load_v(0);
    // A's block (0,1) is zero in both buffers; no chunk writes it
    for (int e = 64 * hw + lane; e < 2 * SUB * SUB; e += 64 * NHW) {
        ChunkTiles& Hz = sm.ch[e >> 8];
        const int r = (e >> 4) & 15, c = tperm(SUB + (e & 15));
        Hz.ah[r][sw(r, c)] = 0; Hz.al[r][sw(r, c)] = 0;
    }
    // A from its half-sums: elements e = 256 hw' + ... of the 768 in blocks (0,0), (1,0), (1,1); each lane
    // takes three, at fixed places (hoisted out of the loop: source index and destination column)
    int asrc[3], adst[3];
    bool azero[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int e = 256 * k + 64 * hw + lane;  // block k, element (r, ln) = ((e >> 6) & 3, e & 63)
        const int r = (e >> 6) & 3, ln = e & 63;
        const int R = k == 0 ? 0 : 1, S = k == 2 ? 1 : 0;
        const int i = 4 * (ln >> 4) + r, jj = ln & 15;
        asrc[k] = (r * 64 + ln);                                  // within apart[2k] / apart[2k+1]
        adst[k] = (SUB * R + i) * LDA + sw(SUB * R + i, tperm(SUB * S + jj));
        azero[k] = R == S && jj > i;                              // above the diagonal of a diagonal block
    }
    __builtin_amdgcn_s_setprio(2);  // the substitution is a chain of dependent steps: issue it early
    for (int n = -1; n <= nchunk; ++n) {
        const bool gwork = n >= 0 && n < nchunk;
        ChunkTiles& H = sm.ch[n & 1];
        // ---------------- part 1: 2^64 v of chunk n to LDS (the value waves use it in the next step)
        if (gwork) {
            float x[8];
            const int t0 = n * C;
            // (rows past T and v == NULL, where the loads read g, are replaced by 0; full chunks of v, the
            // common case, take no per-lane test)
#pragma unroll
            for (int R = 0; R < 2; ++R)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (IN_F32) x[4 * R + r] = vr[R][r];
                    else x[4 * R + r] = __uint_as_float((uint32_t)vr[R][r] << 16);
                }
            if (p.v && t0 + C <= p.T) {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] *= kUp;
            } else {
#pragma unroll
                for (int R = 0; R < 2; ++R)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[4 * R + r] = (p.v && t0 + SUB * R + 4 * g4 + r < p.T) ? kUp * x[4 * R + r] : 0.f;
            }
            *reinterpret_cast<f32x4*>(&sm.vs[n & 1].x[hw][0][lane][0]) = f32x4{x[0], x[1], x[2], x[3]};
            *reinterpret_cast<f32x4*>(&sm.vs[n & 1].x[hw][1][lane][0]) = f32x4{x[4], x[5], x[6], x[7]};
        }
        load_v(min(n + 1, nchunk - 1) * C);  // v of the chunk after (unconditionally, as in load_chunk)
        lds_barrier();  // ---- barrier 1
        // ---------------- part 2: L(0,0), L(1,1) (wave 0) and 2^64 L(1,0) (wave 1) of chunk n
        if (gwork && hw < 2) {
            const int Ra = hw == 0 ? 0 : 1;   // L(0,0) or L(1,0)
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;  // acc1: L(1,1) (wave 0)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int kc = 32 * m + 8 * g4;
                const u32x4 a0 = ld16(&H.km[SUB * Ra + l16][kc]);
                acc0 = mfma_bf16(a0, ld16(&sm.key.khh[l16][kc]), acc0);
                if constexpr (HP) acc0 = mfma_bf16(a0, ld16(&sm.key.khl[l16][kc]), acc0);
                if (hw == 0) {
                    const u32x4 a1 = ld16(&H.km[SUB + l16][kc]);
                    acc1 = mfma_bf16(a1, ld16(&sm.key.khh[SUB + l16][kc]), acc1);
                    if constexpr (HP) acc1 = mfma_bf16(a1, ld16(&sm.key.khl[SUB + l16][kc]), acc1);
                }
            }
            if (hw == 0) {  // the diagonal blocks as -Diag(beta) L (strictly lower), the form the substitution uses
                const f32x4 nb0 = -*reinterpret_cast<const f32x4*>(&H.beta[4 * g4]);
                const f32x4 nb1 = -*reinterpret_cast<const f32x4*>(&H.beta[SUB + 4 * g4]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * g4 + r;
                    sm.s.lf[i][l16] = (l16 >= i) ? 0.f : nb0[r] * acc0[r];
                    sm.s.lf[SUB + i][SUB + l16] = (l16 >= i) ? 0.f : nb1[r] * acc1[r];
                }
            } else {        // 2^64 L(1,0) as a split-bf16 operand, in the block (1,0) of T's tile
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 4 * g4 + r;
                    uint32_t hi, lo;
                    split2(kUp * acc0[r], 0.f, hi, lo);
                    H.th[SUB + i][sw(SUB + i, tperm(l16))] = hi & 0xffffu;
                    H.tl[SUB + i][sw(SUB + i, tperm(l16))] = lo & 0xffffu;
                }
            }
        }
        // ---------------- part 2: the A Gram half-sums of chunk n (waves 2, 3): blocks (R,S) = (0,0),
        // (1,0), (1,1) of Qm Kh^T over channels 0-63 (wave 2) or 64-127 (wave 3), split bf16; the
        // float32 half-sums go to apart, which part 3 adds (A serves only the output: not in a state-only run)
        if (!SO && gwork && hw >= 2) {
            const int mh = hw - 2;
#pragma unroll
            for (int blk = 0; blk < 3; ++blk) {
                const int R = blk == 0 ? 0 : 1, S = blk == 2 ? 1 : 0;
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mm = 0; mm < 2; ++mm) {
                    const int kc = 32 * (2 * mh + mm) + 8 * g4;
                    const u32x4 aH = ld16(&H.qmh[SUB * R + l16][kc]);
                    const u32x4 aL = ld16(&H.qml[SUB * R + l16][kc]);
                    const u32x4 bH = ld16(&sm.key.khh[SUB * S + l16][kc]);
                    const u32x4 bL = ld16(&sm.key.khl[SUB * S + l16][kc]);
                    a = mfma_bf16(aH, bH, a);
                    a = mfma_bf16(aH, bL, a);
                    a = mfma_bf16(aL, bH, a);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.s.apart[2 * blk + mh][r][lane] = a[r];
            }
        }
        lds_barrier();  // ---- barrier 2
        // ---------------- part 3: UT inverse of the two diagonal blocks; A'' = -2^64 A
        if (gwork) {
            // Wave hw solves two columns ja, jb of block hw >> 1 of (I + Diag(beta) L) X = I per 16-lane row
            // g4: ja = g4, jb = 12 + g4 (even hw) or ja = 4 + g4, jb = 8 + g4 (odd hw); lane l16 holds matrix
            // row i = l16 of N = -Diag(beta) L.  With x_i = [i == j] + y_i, forward substitution reads
            // y = N e_j + N y: y starts as column j of N, and at step m row m's (final) y_m is broadcast along
            // the 16-lane row and rows below take y_i += N[i][m] y_m.  Rows at or above j keep y = 0, so
            // column j needs steps m > j only, which the column pairing balances.
            const bool odd = hw & 1;
            const int o = SUB * (hw >> 1), i = l16, ja = (odd ? 4 : 0) + g4, jb = (odd ? 8 : 12) + g4;
            float Nr[SUB];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(&sm.s.lf[o + i][o + 4 * q4]);
                Nr[4 * q4] = t[0]; Nr[4 * q4 + 1] = t[1]; Nr[4 * q4 + 2] = t[2]; Nr[4 * q4 + 3] = t[3];
            }
            float ya = sm.s.lf[o + i][o + ja], yb = sm.s.lf[o + i][o + jb];
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
            // T' = 2^-64 X Diag(beta), as split bf16 in the tperm'd columns of T's tile
            const float ta = ((i == ja ? 1.f : 0.f) + ya) * (H.beta[o + ja] * kDown);
            const float tb = ((i == jb ? 1.f : 0.f) + yb) * (H.beta[o + jb] * kDown);
            uint32_t hi, lo;
            split2(ta, tb, hi, lo);
            const int ca = sw(o + i, tperm(o + ja)), cb = sw(o + i, tperm(o + jb));
            H.th[o + i][ca] = hi & 0xffffu;
            H.th[o + i][cb] = hi >> 16;
            H.tl[o + i][ca] = lo & 0xffffu;
            H.tl[o + i][cb] = lo >> 16;
            // A'' = -2^64 A from the two channel-half sums (lower triangle on the diagonal blocks); only
            // with an output
            if constexpr (!SO) {
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const float* ap = &sm.s.apart[2 * k][0][0];
                    float v = -kUp * (ap[asrc[k]] + ap[256 + asrc[k]]);
                    if (azero[k]) v = 0.f;
                    uint32_t h2, l2;
                    split2(v, 0.f, h2, l2);
                    (&H.ah[0][0])[adst[k]] = h2 & 0xffffu;
                    (&H.al[0][0])[adst[k]] = l2 & 0xffffu;
                }
            }
        }
        lds_barrier();  // ---- barrier 3
    }
}

// ------------------------------------------------------------------------------------------------
// value waves.  Step n handles chunk n-1 (nothing for n < 1); three barriers per step.
// ------------------------------------------------------------------------------------------------
template <bool OUT_F32, bool IN_F32, bool CKPT, bool SO>
__device__ __forceinline__ void value_waves(Smem& sm, const Params& p, int bh, size_t row0, int half, int vw, int lane, int nchunk) {
    const int l16 = lane & 15, g4 = lane >> 4;

    // state: st[cb][r] = S[16*cb + 4*g4 + r][col]
    const int col = half * DVH + 16 * vw + l16;
    // byte offset of state element (16*cb + 4*g4 + r, col) within a head's [DK][DV] float32 state
    const uint32_t soff = (uint32_t)(4 * g4 * DV + col) * 4u;
    auto sidx = [&](int cb, int r) { return soff + (uint32_t)((16 * cb + r) * DV * 4); };
    f32x4 st[8];
    {
        const gchar* s0 = uniform_gptr(p.S0 ? (const void*)(p.S0 + (size_t)bh * DK * DV) : nullptr);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[cb][r] = p.S0 ? gload<float>(s0, sidx(cb, r)) : 0.f;
    }
    // byte offsets of this lane's output (token 16R + l16 of a chunk, value columns 4*g4..4*g4+3)
    uint32_t ooff[2];
#pragma unroll
    for (int R = 0; R < 2; ++R)
        ooff[R] = ((uint32_t)(SUB * R + l16) * (uint32_t)p.H * DV + half * DVH + 16 * vw + 4 * g4) * (OUT_F32 ? 4u : 2u);
    const float oscale = -kDown * p.scale;

    __builtin_amdgcn_s_setprio(3);  // the value waves carry the serial chain: issue them first

    // steps -1 and 0 have no chunk yet (the first chunk's tiles are being formed)
    for (int n = -1; n <= 0; ++n) {
        lds_barrier();
        lds_barrier();
        lds_barrier();
    }
    // the state enters the row-scaled frame R = Diag(ep) S of chunk 0 (exact: powers of two)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) st[cb] *= *reinterpret_cast<const f32x4*>(&sm.sc[0].ep[16 * cb + 4 * g4]);

    for (int n = 1; n <= nchunk; ++n) {
        constexpr bool work = true;  // step n handles chunk n-1
        const int c = n - 1;
        const int t0 = c * C;
        const ChunkTiles& H = sm.ch[c & 1];
        const Scalings& Sc = sm.sc[c % 3];
        u32x4 ph[4];
        f32x4 oacc[2];
        // ---------------- part 1: the state operand P = R as split-bf16 operands; Qm P
        // (the two row blocks' chains alternate, so consecutive matrix instructions are independent; each
        // chain accumulates in place, which the matrix core forwards without a vector add).  A state-only
        // run needs P_hi alone (for X~).
        if (SO && work) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 a = st[2 * m], b = st[2 * m + 1];
                ph[m] = u32x4{pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]), pack_bf16(b[2], b[3])};
            }
        }
        if (!SO && work) {
            // K-step m over channels 32m..32m+31 in the order {32m + 4*g4 + r} then {32m + 16 + 4*g4 + r};
            // as an A operand it is P^T.  Qm P as O^T: lane (token l16, group g4) gets columns 4*g4..4*g4+3
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 a = st[2 * m], b = st[2 * m + 1];
                uint32_t h0, h1, h2, h3, q0, q1, q2, q3;
                split2(a[0], a[1], h0, q0);
                split2(a[2], a[3], h1, q1);
                split2(b[0], b[1], h2, q2);
                split2(b[2], b[3], h3, q3);
                ph[m] = u32x4{h0, h1, h2, h3};
                const u32x4 pl = u32x4{q0, q1, q2, q3};
                const u32x4 bH0 = ld16(&H.qmh[l16][32 * m + 8 * g4]), bL0 = ld16(&H.qml[l16][32 * m + 8 * g4]);
                const u32x4 bH1 = ld16(&H.qmh[SUB + l16][32 * m + 8 * g4]), bL1 = ld16(&H.qml[SUB + l16][32 * m + 8 * g4]);
                oacc[0] = mfma_bf16(ph[m], bH0, m ? oacc[0] : f32x4{0.f, 0.f, 0.f, 0.f});
                oacc[1] = mfma_bf16(ph[m], bH1, m ? oacc[1] : f32x4{0.f, 0.f, 0.f, 0.f});
                oacc[0] = mfma_bf16(pl, bH0, oacc[0]);
                oacc[1] = mfma_bf16(pl, bH1, oacc[1]);
                oacc[0] = mfma_bf16(ph[m], bL0, oacc[0]);
                oacc[1] = mfma_bf16(ph[m], bL1, oacc[1]);
            }
        }
        lds_barrier();  // ---- barrier 1

        // ---------------- part 2: X~ = 2^64 V + Km P; U
        u32x4 uh, ul;
        if (work) {
            // 2^64 V in accumulator layout (tokens 16R + 4*g4 + r, column col), staged by a helper wave
            f32x4 xr[2] = {*reinterpret_cast<const f32x4*>(&sm.vs[c & 1].x[vw][0][lane][0]),
                           *reinterpret_cast<const f32x4*>(&sm.vs[c & 1].x[vw][1][lane][0])};
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int R = 0; R < 2; ++R)
                    xr[R] = mfma_bf16(ld16(&H.km[SUB * R + l16][32 * m + 8 * g4]), ph[m], xr[R]);
            // U by block forward substitution over the two sub-tiles (T is block lower triangular):
            //   U0 = T'00 X~0,   U1 = T'11 (X~1 - L'10 U0),
            // as split-bf16 16x16x16 products whose contraction index is token 4*g4 + r of a sub-tile
            auto split4 = [](const f32x4 x, u32x2& h, u32x2& l) {
                uint32_t h0, h1, l0, l1;
                split2(x[0], x[1], h0, l0);
                split2(x[2], x[3], h1, l1);
                h = u32x2{h0, h1};
                l = u32x2{l0, l1};
            };
            auto prod3 = [](u32x2 aH, u32x2 aL, u32x2 bH, u32x2 bL) {
                f32x4 a = mfma_bf16_k16(aH, bH, f32x4{0.f, 0.f, 0.f, 0.f});
                a = mfma_bf16_k16(aH, bL, a);
                return mfma_bf16_k16(aL, bH, a);
            };
            auto ld8 = [](const uint16_t* q) { return *reinterpret_cast<const u32x2*>(q); };
            f32x4 u[2];
            u32x2 sh, sl;
            split4(xr[0], sh, sl);
            const int c0s = sw(l16, 8 * g4);  // (rows l16 and SUB + l16 share the swizzle)
            u[0] = prod3(ld8(&H.th[l16][c0s]), ld8(&H.tl[l16][c0s]), sh, sl);
            split4(u[0], sh, sl);
            const f32x4 lu = prod3(ld8(&H.th[SUB + l16][c0s]), ld8(&H.tl[SUB + l16][c0s]), sh, sl);
            split4(xr[1] - lu, sh, sl);
            u[1] = prod3(ld8(&H.th[SUB + l16][c0s + 4]), ld8(&H.tl[SUB + l16][c0s + 4]), sh, sl);
            uint32_t uh0, uh1, uh2, uh3, ul0, ul1, ul2, ul3;
            split2(u[0][0], u[0][1], uh0, ul0);
            split2(u[0][2], u[0][3], uh1, ul1);
            split2(u[1][0], u[1][1], uh2, ul2);
            split2(u[1][2], u[1][3], uh3, ul3);
            uh = u32x4{uh0, uh1, uh2, uh3};
            ul = u32x4{ul0, ul1, ul2, ul3};
        }
        lds_barrier();  // ---- barrier 2

        // ---------------- part 3: O = -2^-64 (Qm P + A'' U), output; R <- Diag(rho) R + Kbar'^T U
        if (work) {
            if (!SO && p.o) {  // (o == NULL: a state-only run of the in-device context parallelism)
                gchar* ob = (gchar*)uniform_gptr((const char*)p.o + ((row0 + (size_t)t0 * p.H) * DV) * (OUT_F32 ? 4 : 2));
                u32x4 aH[2], aL[2];
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    aH[R] = ld16(&H.ah[SUB * R + l16][sw(l16, 8 * g4)]);
                    aL[R] = ld16(&H.al[SUB * R + l16][sw(l16, 8 * g4)]);
                }
                f32x4 oc[2];
#pragma unroll
                for (int R = 0; R < 2; ++R) oc[R] = mfma_bf16(uh, aH[R], oacc[R]);
#pragma unroll
                for (int R = 0; R < 2; ++R) oc[R] = mfma_bf16(ul, aH[R], oc[R]);
#pragma unroll
                for (int R = 0; R < 2; ++R) oc[R] = mfma_bf16(uh, aL[R], oc[R]);
#pragma unroll
                for (int R = 0; R < 2; ++R) {
                    const f32x4 acc = oc[R] * oscale;
                    if (t0 + SUB * R + l16 < p.T) {
                        if constexpr (OUT_F32)
                            gstore<f32x4>(ob, ooff[R], acc);
                        else
                            gstore<u32x2>(ob, ooff[R], u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])});
                    }
                }
            }
            // kbrow(16 cb + l16) = 16 cb + (lr ^ 2 (cb & 1)): two lane offsets, the rest immediate
            constexpr int kodd = IN_F32 ? 0 : 2;
            const int lr = IN_F32 ? l16 : l16 ^ (l16 >> 3), kcol = sw(l16, 8 * g4);
#pragma unroll
            for (int c4 = 0; c4 < 8; c4 += 4) {  // four row blocks at a time, term by term
                u32x4 aH[4], aL[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cb = c4 + j;
                    aH[j] = ld16(&H.kbh[16 * cb + (lr ^ ((cb & 1) * kodd))][kcol]);
                    aL[j] = ld16(&H.kbl[16 * cb + (lr ^ ((cb & 1) * kodd))][kcol]);
                    if constexpr (!IN_F32) {
                        // rho of rows 16cb + 4g4 + r: lane r of each 16-lane row reads it, and the multiply
                        // takes it by row broadcast (a quarter of the LDS bytes of a 16-byte read per lane)
                        const float rh = Sc.gam[16 * cb + 4 * g4 + (l16 & 3)];
                        st[cb][0] *= row_bcast<0>(rh);
                        st[cb][1] *= row_bcast<1>(rh);
                        st[cb][2] *= row_bcast<2>(rh);
                        st[cb][3] *= row_bcast<3>(rh);
                    } else {  // (the float32-input variant has no registers to spare for it)
                        st[cb] *= *reinterpret_cast<const f32x4*>(&Sc.gam[16 * cb + 4 * g4]);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) st[c4 + j] = mfma_bf16(aH[j], uh, st[c4 + j]);
#pragma unroll
                for (int j = 0; j < 4; ++j) st[c4 + j] = mfma_bf16(aH[j], ul, st[c4 + j]);
#pragma unroll
                for (int j = 0; j < 4; ++j) st[c4 + j] = mfma_bf16(aL[j], uh, st[c4 + j]);
            }
            if (CKPT && n % p.ckpt_chunks == 0 && n / p.ckpt_chunks <= p.n_ckpt) {
                // the state after tokens [0, n*C): checkpoint n / ckpt_chunks - 1
                gchar* dst = uniform_gptr(p.S_ckpt + ((size_t)bh * p.n_ckpt + (n / p.ckpt_chunks - 1)) * DK * DV);
                uint32_t o = soff;
                asm volatile("" : "+v"(o));  // formed here: offsets held across the loop would spill
                // S = R / ep with ep = -2^(64 + kappa) of chunk n (-2^64 past the last chunk): the exact
                // reciprocal of a power of two, by its exponent field
                const Scalings& Sn = sm.sc[n % 3];
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    f32x4 ie = f32x4{-kDown, -kDown, -kDown, -kDown};
                    if (n < nchunk) {
                        const f32x4 e = *reinterpret_cast<const f32x4*>(&Sn.ep[16 * cb + 4 * g4]);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            ie[r] = __int_as_float((int)(0xff000000u - ((uint32_t)__float_as_int(e[r]) & 0x7f800000u)));
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) gstore<float>(dst, o + (uint32_t)((16 * cb + r) * DV * 4), st[cb][r] * ie[r]);
                }
            }
        }
        lds_barrier();  // ---- barrier 3
    }

    if (p.S_T) {  // the last chunk left R = -2^64 S
        gchar* sT = uniform_gptr(p.S_T + (size_t)bh * DK * DV);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) gstore<float>(sT, sidx(cb, r), st[cb][r] * -kDown);
    }
}

// CKPT: S_ckpt is set (a separate instantiation keeps the plain forward free of the checkpoint code)
// SO: a state-only run (o == NULL): the output and everything only it needs (Qm, A, Qm P) is skipped
template <bool OUT_F32, bool IN_F32, bool HP, bool CKPT, bool SO>
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
    int b = bh / p.H;
    const int h = bh - b * p.H;
    Params q = p;  // this workgroup's view (wave-uniform)
    if (p.alt_b0 > 0 && b >= p.alt_b0) {  // the second row set of a merged launch (see Params)
        b -= p.alt_b0;
        q.v = nullptr;
        q.S0 = p.alt_S0;
        q.S_T = p.alt_ST;
        q.seg_lo = p.alt_seg_lo;
        q.seg_cnt = p.alt_seg_cnt;
    }
    if (q.seg_cnt > 0)  // a subset of the batch rows (see Params)
        b = (b / q.seg_cnt) * q.seg_n + q.seg_lo + b % q.seg_cnt;
    bh = b * p.H + h;
    size_t row0;  // row of token 0: (first token + t)*H + h = row0 + t*H
    if (p.seg_T > 0) {  // row b = segment b % seg_n of sequence b / seg_n; the last segment runs to seg_T
        const int s = b % p.seg_n;
        row0 = ((size_t)(b / p.seg_n) * p.seg_T + (size_t)s * p.tstride) * p.H + h;
        q.T = s == p.seg_n - 1 ? p.seg_T - (p.seg_n - 1) * p.tstride : p.tstride;
    } else {
        row0 = (size_t)b * p.tstride * p.H + h;
    }
    const int nchunk = (q.T + C - 1) / C;
    if (nchunk == 0) return;  // (the host runs the state copy instead; every wave leaves here alike)

    if (wave < NKW)
        key_waves<IN_F32, SO>(sm, q, row0, wave, lane, nchunk);
    else if (wave < NKW + NVW)
        value_waves<OUT_F32, IN_F32, CKPT, SO>(sm, q, bh, row0, half, wave - NKW, lane, nchunk);
    else
        helper_waves<IN_F32, HP, SO>(sm, q, row0, half, wave - NKW - NVW, lane, nchunk);
}

}  // namespace bf16path

namespace bf16path {
template <bool CKPT>
void launch_bf16_io(const Params& p, hipStream_t stream, dim3 grid, dim3 block) {
    if (!p.o && p.precise)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, true, CKPT, true>), grid, block, 0, stream, p);
    else if (!p.o)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, false, CKPT, true>), grid, block, 0, stream, p);
    else if (p.o_f32 && p.precise)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, false, true, CKPT, false>), grid, block, 0, stream, p);
    else if (p.o_f32)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, false, false, CKPT, false>), grid, block, 0, stream, p);
    else if (p.precise)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, true, CKPT, false>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, false, false, CKPT, false>), grid, block, 0, stream, p);
}
}  // namespace bf16path

hipError_t launch_fwd_bf16(const Params& p, hipStream_t stream) {
    using namespace bf16path;
    if (p.T == 0) return launch_state_copy(p, stream);
    const dim3 grid(2 * p.B * p.H), block(NTHR);
    if (p.in_f32 && !p.o)  // the layer's variant (it records no checkpoints)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<false, true, true, false, true>), grid, block, 0, stream, p);
    else if (p.in_f32)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<true, true, true, false, false>), grid, block, 0, stream, p);
    else if (p.S_ckpt)
        launch_bf16_io<true>(p, stream, grid, block);
    else
        launch_bf16_io<false>(p, stream, grid, block);
    return hipGetLastError();
}

}  // namespace kda
