// Backward pass of the chunkwise KDA forward, on gfx950.
//
// The forward is the gated delta rule of the explainer page "Kimi K3：开放前沿智能", section 2.2
// (paper Eq. 1), read out after the update (section 2.4), in the chunkwise form of section 2.5
// (paper Eq. 4).  The pages give no backward formulas; these kernels apply the chain rule to each
// line of the chunkwise forward in reverse.  Per chunk of CS = 16 tokens, with the forward
// quantities (Q scaled; b the cumulative log-decay from the chunk start, Gamma = exp(b))
//   Qg = Q*Gamma, Kg = K*Gamma, Kh = K/Gamma, Kb = K*exp(b_last - b), gam = Gamma_last,
//   L = tril(Kg Kh^T, -1), A = tril(Qg Kh^T), N = (I + Diag(beta) L)^{-1}, Tm = N Diag(beta),
//   X = V - Kg S, U = Tm X, O = Qg S + A U, S' = Diag(gam) S + Kb^T U,
// and the gradient dS of the state after the chunk, dO of its outputs:
//   dU = Kb dS + A^T dO;  dX = Tm^T dU (= dV);  dS_in = Diag(gam) dS + Qg^T dO - Kg^T dX
//   dKb = U dS^T;  dgam = rowsum(dS * S);  dQg = dO S^T + dA Kh;  dA = tril(dO U^T)
//   dTm = dU X^T;  dKg = -dX S^T + dL Kh;  dKh = dL^T Kg + dA^T Qg
//   dbeta = colsum(N * dTm) + rowsum(dM * L);  dM = -N^T (dTm Diag(beta)) N^T;  dL = tril(Diag(beta) dM, -1)
//   dq = dQg*scale*Gamma;  dk = dKg*Gamma + dKh/Gamma + dKb*exp(b_last - b)
//   db = dQg*Qg + dKg*Kg - dKh*Kh - dKb*Kb (+ sum_t dKb*Kb + dgam*gam on the last row);  dg = reverse cumsum of db.
// Under the g >= -5 bound of section 3.2 the factors of a 16-token chunk stay within [e^-80, e^80].
//
// Three launches (float32 arithmetic throughout):
//   1. the forward kernel with checkpoints: the state at every interval boundary (32 tokens on the
//      matrix-core path, 16 on the float32 path), no output;
//   2. kda_bwd_state_kernel, one workgroup per (sequence, value half), sequential in reverse over
//      chunks: the state gradient dS at every interval boundary (its update needs no state); half
//      the waves carry dS while the other half prepare the next chunk's factors; it also zeroes the
//      outputs step 3 accumulates into;
//   3. kda_bwd_chunk_kernel, one work item per (sequence, interval, value half), all independent,
//      taken in turn by one persistent workgroup per CU: every input gradient of the interval, from
//      the interval's start state and end gradient (a 32-token interval first steps its state
//      through the first 16-token chunk).
// Every gradient is linear in (dO, dS), so each value half computes the contributions of its own
// value columns; the two halves' contributions to dq, dk, dg and dbeta are added with float32
// atomics onto zeroed outputs (exactly two addends per element: the sum does not depend on order).
#include "kda_common.h"
#include "kda_internal.h"

#include <algorithm>
#include <type_traits>

namespace kda {
namespace bwd {

constexpr int CS = 16;   // tokens per chunk
constexpr int NT = 512;  // threads per workgroup (8 waves)
static_assert(NT >= CS * CS, "one thread per chunk-matrix entry");

// Element i of a bf16 or float32 array as raw bits: for bf16 the aligned 32-bit word holding it
// (its half is selected when the value is used, cvt with odd = i & 1), for float32 the element.
// Prefetched inputs stay raw until used: any conversion right after the load (a 16-bit load's
// zero extension included) would make the load wait there.
template <bool BF16>
__device__ __forceinline__ uint32_t ldr(const void* p, size_t i) {
    return reinterpret_cast<const uint32_t*>(p)[BF16 ? i >> 1 : i];
}
template <bool BF16>
__device__ __forceinline__ float cvt(uint32_t x, bool odd) {
    return __uint_as_float(BF16 ? (odd ? x & 0xffff0000u : x << 16) : x);
}

// Four consecutive entries of an LDS tile: along row r from column c (16-byte aligned: c and the row
// pitch multiples of 4), or down column c from row r.
template <int W>
__device__ __forceinline__ f32x4 row4(const float (*t)[W], int r, int c) {
    static_assert(W % 4 == 0, "row pitch");
    return *reinterpret_cast<const f32x4*>(&t[r][c]);
}
template <int W>
__device__ __forceinline__ f32x4 col4(const float (*t)[W], int r, int c) {
    return f32x4{t[r][c], t[r + 1][c], t[r + 2][c], t[r + 3][c]};
}

// acc += sum_k A(m, k) B(k, n) for this lane's row m and column n (see mgemm for the index order).
template <int K, typename FA, typename FB>
__device__ __forceinline__ void tile_product(FA a, FB b, int m, int n, int g, f32x4& acc) {
#pragma unroll
    for (int q = 0; q < K / 16; ++q) {
        const int k = 16 * q + 4 * g;
        const f32x4 av = a(m, k), bv = b(k, n);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[r], bv[r], acc, 0, 0, 0);
    }
}

// out(m, n) = sum_k a(m, k) b(k, n) for m < M, n < N on the matrix cores: float32
// v_mfma_f32_16x16x4_f32 (exact float32 products, float32 accumulation), one 16 x 16 output tile per
// wave at a time; f(m, n, v) receives the result.  Operand layout of that instruction: A(m, k_g) in
// lane m + 16 g, B(k_g, n) in lane n + 16 g, result (4 g + r, n) in lane n + 16 g, register r; one
// instruction adds the four products of lane groups g = 0..3.  Each lane group takes the contraction
// indices 16 q + 4 g + r (q = 0 .. K/16 - 1, r = 0..3), four consecutive ones per 16-index block, so
// that a(m, k) and b(k, n) return four consecutive indices k..k+3 at once (f32x4): one 16-byte LDS
// read where the tile stores them contiguously (row4), four reads one row apart otherwise (col4).
// Tile t goes to wave (first_wave + t) mod 8, so that small products issued back to back without a
// barrier between them can run on different waves.
template <int M, int N, int K, typename FA, typename FB, typename F>
__device__ __forceinline__ void mgemm(FA a, FB b, F f, int first_wave = 0) {
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0, "tile shape");
    constexpr int TN = N / 16, NW = NT / 64;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;
    for (int tile = (wave + NW - first_wave) % NW; tile < (M / 16) * TN; tile += NW) {
        const int m0 = (tile / TN) * 16, n0 = (tile % TN) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_product<K>(a, b, m0 + l16, n0 + l16, g, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) f(m0 + 4 * g + r, n0 + l16, acc[r]);
    }
}

// Factors of one chunk, its beta, and the value-half columns of dO (and V in X when wanted).
// Row pitches (floats): key-side [CS][D] tiles D + KP, value-half tiles DH + VP, chunk-square tiles
// CS + SP, all multiples of 4 for 16-byte reads.  Measured on gfx950 with eight waves per CU, 16-byte
// reads of 16 rows at one column block run at ~5.3 clocks per instruction when the pitch is 8 mod 64
// floats (~9 at 4 mod 64), and column reads of rows 16 q + 4 g + r at ~4.4 (~3 at 4 mod 64).
constexpr int KP = 8;
constexpr int VP = 8;
constexpr int SP = 4;

template <int D>
struct alignas(16) Chunk {
    static constexpr int DH = D / 2;
    float Qg[CS][D + KP], Kg[CS][D + KP], Kh[CS][D + KP], Kb[CS][D + KP], Gam[CS][D + KP];
    float gam[D];
    float X[CS][DH + VP], U[CS][DH + VP], dO[CS][DH + VP], dU[CS][DH + VP], dX[CS][DH + VP];
    float L[CS][CS + SP], A[CS][CS + SP], N[CS][CS + SP], Tm[CS][CS + SP];
    float beta[CS];
};

// One chunk's inputs as thread tid holds them: channel tid % D's g over the chunk's tokens and q,
// k over its share of them, tokens TS*(tid/D) .. TS*(tid/D + 1) - 1 (the NT threads split each
// channel's tokens into NT/D shares), beta of token tid (tid < CS), and dO / V entries tid + NT*k
// of the value half.
template <int D>
struct Raw {
    static constexpr int PV = CS * (D / 2) / NT;
    static constexpr int TS = CS * D / NT;  // tokens per thread (4 for D = 128, 2 for D = 64)
    uint32_t q[TS], k[TS];  // raw (see ldr)
    float g[CS];
    float beta;
    uint32_t dO[PV], v[PV];
    int n;  // valid tokens
};

// f(std::integral_constant<int, s>) for the wave-uniform share index sh < NS (a compile-time
// token offset per share keeps register arrays indexed by constants).
template <int NS, typename F>
__device__ __forceinline__ void for_share(int sh, F f) {
    if constexpr (NS > 0) {
        if (sh == NS - 1)
            f(std::integral_constant<int, NS - 1>{});
        else
            for_share<NS - 1>(sh, f);
    }
}

template <int D, bool IN_BF16, bool DO_BF16>
__device__ __forceinline__ void fetch_chunk(Raw<D>& w, const BwdParams& p, int b, int h, int c0, int half, bool want_v) {
    constexpr int DH = D / 2;
    const int tid = threadIdx.x;
    const int n = min(CS, p.T - c0);  // valid tokens (>= 1); rows past them read the last valid one
    w.n = n;
    // the chunk's first row (b, c0, h) as wave-uniform base pointers; rows r as 32-bit element offsets
    const size_t rb = ((size_t)b * p.T + c0) * p.H + h;
    const uint32_t rs = (uint32_t)p.H * D;
    auto roff = [&](int r) { return (uint32_t)min(r, n - 1) * rs; };
    constexpr size_t ie = IN_BF16 ? 2 : 4, oe = DO_BF16 ? 2 : 4;
    {
        constexpr int TS = Raw<D>::TS;
        const int ch = tid % D, r0 = TS * (tid / D);
        const float* gb = p.g + rb * D;
        const void* qb = (const char*)p.q + rb * D * ie;
        const void* kb = (const char*)p.k + rb * D * ie;
#pragma unroll
        for (int r = 0; r < CS; ++r) w.g[r] = gb[roff(r) + ch];  // (every share needs the cumulative sums)
#pragma unroll
        for (int r = 0; r < TS; ++r) {
            w.q[r] = ldr<IN_BF16>(qb, roff(r0 + r) + ch);
            w.k[r] = ldr<IN_BF16>(kb, roff(r0 + r) + ch);
        }
    }
    if (tid < CS) w.beta = p.beta[rb + (size_t)min(tid, n - 1) * p.H];
    // (branches around whole groups of loads: a select per loaded value would make each load wait)
    if (p.dO) {
        const void* ob = (const char*)p.dO + (rb * D + half * DH) * oe;
#pragma unroll
        for (int k = 0; k < Raw<D>::PV; ++k) {
            const int e = tid + NT * k, r = e / DH, j = e % DH;
            w.dO[k] = ldr<DO_BF16>(ob, roff(r) + j);
        }
    } else {  // dO == NULL: zero (never dereferenced)
#pragma unroll
        for (int k = 0; k < Raw<D>::PV; ++k) w.dO[k] = 0u;
    }
    if (want_v) {
        const void* vb = (const char*)p.v + (rb * D + half * DH) * ie;
#pragma unroll
        for (int k = 0; k < Raw<D>::PV; ++k) {
            const int e = tid + NT * k, r = e / DH, j = e % DH;
            w.v[k] = ldr<IN_BF16>(vb, roff(r) + j);
        }
    }
}

// The chunk's factors from the fetched inputs (tokens past the valid ones are zeroed: k = q = v = 0,
// g = 0, beta = 0, dO = 0).
template <int D, bool IN_BF16, bool DO_BF16>
__device__ __forceinline__ void build_chunk(Chunk<D>& c, const Raw<D>& w, float scale, bool want_v) {
    constexpr int DH = D / 2;
    const int tid = threadIdx.x;
    const int n = w.n;
    {
        constexpr int TS = Raw<D>::TS;
        const int ch = tid % D, sh = tid / D;
        float bc[CS];
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            s += r < n ? w.g[r] : 0.f;
            bc[r] = s;
        }
        const float last = bc[CS - 1], gl = fexp(last);
        if (sh == 0) c.gam[ch] = gl;
        for_share<CS / TS>(sh, [&](auto shc) {
            constexpr int R0 = TS * decltype(shc)::value;
#pragma unroll
            for (int r = 0; r < TS; ++r) {
                const int t = R0 + r;
                const float q = t < n ? cvt<IN_BF16>(w.q[r], ch & 1) * scale : 0.f;
                const float k = t < n ? cvt<IN_BF16>(w.k[r], ch & 1) : 0.f;
                const float e = fexp(bc[t]), f = fexp(-bc[t]);  // exp(b), exp(-b), both within [e^-80, e^80]
                c.Gam[t][ch] = e;
                c.Qg[t][ch] = q * e;
                c.Kg[t][ch] = k * e;
                c.Kh[t][ch] = k * f;
                c.Kb[t][ch] = k * (gl * f);  // exp(b_last - b)
            }
        });
    }
    if (tid < CS) c.beta[tid] = tid < n ? w.beta : 0.f;
#pragma unroll
    for (int k = 0; k < Raw<D>::PV; ++k) {
        const int e = tid + NT * k, r = e / DH, j = e % DH;
        c.dO[r][j] = r < n ? cvt<DO_BF16>(w.dO[k], j & 1) : 0.f;
        if (want_v) c.X[r][j] = r < n ? cvt<IN_BF16>(w.v[k], j & 1) : 0.f;
    }
}

// Lane m of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int M>
__device__ __forceinline__ float row_bcast_c(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + M, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_bcast(float x, int m) {
    switch (m) {
        case 0: return row_bcast_c<0>(x);   case 1: return row_bcast_c<1>(x);   case 2: return row_bcast_c<2>(x);
        case 3: return row_bcast_c<3>(x);   case 4: return row_bcast_c<4>(x);   case 5: return row_bcast_c<5>(x);
        case 6: return row_bcast_c<6>(x);   case 7: return row_bcast_c<7>(x);   case 8: return row_bcast_c<8>(x);
        case 9: return row_bcast_c<9>(x);   case 10: return row_bcast_c<10>(x); case 11: return row_bcast_c<11>(x);
        case 12: return row_bcast_c<12>(x); case 13: return row_bcast_c<13>(x); case 14: return row_bcast_c<14>(x);
        default: return row_bcast_c<15>(x);
    }
}

// out(m, n) = sum_k a(m, k) b(k, n) as in mgemm, on waves W0 .. W0 + NWU - 1 only (tile t on wave
// W0 + t mod NWU); the other waves return at once.
template <int M, int N, int K, int W0, int NWU, typename FA, typename FB, typename F>
__device__ __forceinline__ void mgemm_w(FA a, FB b, F f) {
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 16 == 0, "tile shape");
    constexpr int TN = N / 16;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave < W0 || wave >= W0 + NWU) return;
    const int l16 = lane & 15, g = lane >> 4;
    for (int tile = wave - W0; tile < (M / 16) * TN; tile += NWU) {
        const int m0 = (tile / TN) * 16, n0 = (tile % TN) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        tile_product<K>(a, b, m0 + l16, n0 + l16, g, acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) f(m0 + 4 * g + r, n0 + l16, acc[r]);
    }
}

// dst(m, n) = gam(m) src(m, n) + (Qg^T dO)(m, n) - (Kg^T dX)(m, n) for the D x DH state-gradient tile
// (the gradient of the state before a chunk), on all waves: wave w takes value-column block w mod
// (DH / 16) and every (NT / 64) / (DH / 16)-th channel block, so each wave reads its column block of
// dO and dX once.  Rounding as two products applied one after the other.  dst may be src.
// SPLIT (the bf16-input path): the products as split bf16 on 16x16x16 matrix-core instructions
// (hi*hi + hi*lo + lo*hi of x = hi + lo, each part a bf16, ~16 significant bits per operand), three
// instructions of ~17 clocks in place of four float32 ones of ~33.
template <int D, bool SPLIT, typename TQ, typename TO, typename TX, typename TS>
__device__ __forceinline__ void state_grad_step(const TQ& Qg, const TQ& Kg, const TO& dO, const TX& dX,
                                                const float* gam, const TS& src, TS& dst) {
    static_assert(CS == 16, "one block of four contraction indices per lane group");
    constexpr int DH = D / 2, TN = DH / 16, NW = NT / 64, TM = D / 16;
    static_assert(NW % TN == 0, "column blocks per wave");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4, k = 4 * g, n0 = 16 * (wave % TN);
    const f32x4 bo = col4(dO, k, n0 + l16), bx = col4(dX, k, n0 + l16);
    auto split4 = [](const f32x4 x, u32x2& h, u32x2& l) {
        uint32_t h0, h1, l0, l1;
        split_bf16(x[0], x[1], h0, l0);
        split_bf16(x[2], x[3], h1, l1);
        h = u32x2{h0, h1};
        l = u32x2{l0, l1};
    };
    u32x2 boh, bol, bxh, bxl;
    if constexpr (SPLIT) {
        split4(bo, boh, bol);
        split4(bx, bxh, bxl);
    }
    for (int mb = wave / TN; mb < TM; mb += NW / TN) {
        const int m0 = 16 * mb;
        const f32x4 aq = col4(Qg, k, m0 + l16), ak = col4(Kg, k, m0 + l16);
        f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pk = pq;
        if constexpr (SPLIT) {
            u32x2 aqh, aql, akh, akl;
            split4(aq, aqh, aql);
            split4(ak, akh, akl);
            pq = mfma_bf16_k16(aqh, boh, pq);
            pk = mfma_bf16_k16(akh, bxh, pk);
            pq = mfma_bf16_k16(aqh, bol, pq);
            pk = mfma_bf16_k16(akh, bxl, pk);
            pq = mfma_bf16_k16(aql, boh, pq);
            pk = mfma_bf16_k16(akl, bxh, pk);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pq = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[r], bo[r], pq, 0, 0, 0);
                pk = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bx[r], pk, 0, 0, 0);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * g + r, n = n0 + l16;
            dst[m][n] = __builtin_fmaf(gam[m], src[m][n], pq[r]) - pk[r];
        }
    }
}

// dst(m, n) = gam(m) src(m, n) + (Kb^T U)(m, n): the state after a chunk from the state before it, in
// the same tile order and (SPLIT) the same split-bf16 products as state_grad_step.
template <int D, bool SPLIT, typename TK, typename TU, typename TS>
__device__ __forceinline__ void state_fwd_step(const TK& Kb, const TU& U, const float* gam, const TS& src, TS& dst) {
    static_assert(CS == 16, "one block of four contraction indices per lane group");
    constexpr int DH = D / 2, TN = DH / 16, NW = NT / 64, TM = D / 16;
    static_assert(NW % TN == 0, "column blocks per wave");
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4, k = 4 * g, n0 = 16 * (wave % TN);
    const f32x4 bu = col4(U, k, n0 + l16);
    u32x2 buh, bul;
    if constexpr (SPLIT) {
        uint32_t h0, h1, l0, l1;
        split_bf16(bu[0], bu[1], h0, l0);
        split_bf16(bu[2], bu[3], h1, l1);
        buh = u32x2{h0, h1};
        bul = u32x2{l0, l1};
    }
    for (int mb = wave / TN; mb < TM; mb += NW / TN) {
        const int m0 = 16 * mb;
        const f32x4 ak = col4(Kb, k, m0 + l16);
        f32x4 pu = {0.f, 0.f, 0.f, 0.f};
        if constexpr (SPLIT) {
            uint32_t h0, h1, l0, l1;
            split_bf16(ak[0], ak[1], h0, l0);
            split_bf16(ak[2], ak[3], h1, l1);
            const u32x2 akh{h0, h1}, akl{l0, l1};
            pu = mfma_bf16_k16(akh, buh, pu);
            pu = mfma_bf16_k16(akh, bul, pu);
            pu = mfma_bf16_k16(akl, buh, pu);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) pu = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[r], bu[r], pu, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * g + r, n = n0 + l16;
            dst[m][n] = __builtin_fmaf(gam[m], src[m][n], pu[r]);
        }
    }
}

// L = tril(Kg Kh^T, -1) on wave W and A = tril(Qg Kh^T) on wave W + 1 (one 16 x 16 tile each).
template <int D, int W, typename CT>
__device__ __forceinline__ void gram_products(CT& c) {
    mgemm_w<CS, CS, D, W, 1>([&](int m, int k) { return row4(c.Kg, m, k); }, [&](int k, int n) { return row4(c.Kh, n, k); },
                             [&](int m, int n, float v) { c.L[m][n] = n < m ? v : 0.f; });
    mgemm_w<CS, CS, D, W + 1, 1>([&](int m, int k) { return row4(c.Qg, m, k); }, [&](int k, int n) { return row4(c.Kh, n, k); },
                                 [&](int m, int n, float v) { c.A[m][n] = n <= m ? v : 0.f; });
}

// N = (I + Diag(beta) L)^{-1} and Tm = N Diag(beta) by forward substitution on the last CS*CS
// threads, one matrix entry per lane: column j of N per 16-lane row, lane i holding row i of
// -Diag(beta) L.  With x_i = [i == j] + y_i the substitution is y = (-Diag(beta) L)(e_j + y); at
// step m row m's final y_m is broadcast along the 16 lanes (DPP row_newbcast) for the rows below.
template <typename CT>
__device__ __forceinline__ void unit_inverse(CT& c) {
    const int te = (int)threadIdx.x - (NT - CS * CS);
    if (te < 0) return;
    const int j = te / CS, i = te % CS;
    const float nb = -c.beta[i];
    float nr[CS];
#pragma unroll
    for (int m = 0; m < CS; ++m) nr[m] = nb * c.L[i][m];
    float y = nb * c.L[i][j];
#pragma unroll
    for (int m = 0; m < CS - 1; ++m) y = __builtin_fmaf(nr[m], row_bcast(y, m), y);
    const float x = (i == j ? 1.f : 0.f) + y;
    c.N[i][j] = x;
    c.Tm[i][j] = x * c.beta[j];
}

// ------------------------------------------------------------------------------------------------
// 2. state gradients at interval boundaries, sequential in reverse
// ------------------------------------------------------------------------------------------------
// What the state pass keeps of a chunk (two of these: the chunk being processed and the next one).
template <int D>
struct alignas(16) SChunk {
    static constexpr int DH = D / 2;
    float Qg[CS][D + KP], Kg[CS][D + KP], Kh[CS][D + KP], Kb[CS][D + KP];
    float gam[D];
    float dO[CS][DH + VP];
    float L[CS][CS + SP], A[CS][CS + SP], N[CS][CS + SP], Tm[CS][CS + SP];
    float beta[CS];
};

// One chunk's inputs as the state pass's factor waves (4-7, thread u = tid - NT/2) hold them:
// channel u % D's g over the chunk's tokens and q, k over its share of them, tokens
// TS*(u/D) .. TS*(u/D + 1) - 1 (the NT/2 threads split each channel's tokens into NT/2 / D shares),
// beta of token u (u < CS), dO entries u + (NT/2)*k of the value half.
constexpr int NTH = NT / 2;  // threads of the factor waves
template <int D>
struct SRaw {
    static constexpr int PV = CS * (D / 2) / NTH;
    static constexpr int TS = CS * D / NTH;  // tokens per thread (8 for D = 128, 4 for D = 64)
    uint32_t q[TS], k[TS];  // raw (see ldr)
    float g[CS];
    float beta;
    uint32_t dO[PV];
    int n;  // valid tokens
};

template <int D, bool IN_BF16, bool DO_BF16>
__device__ __forceinline__ void fetch_s(SRaw<D>& w, const BwdParams& p, int b, int h, int c0, int half) {
    constexpr int DH = D / 2;
    const int u = threadIdx.x - NTH;
    const int n = min(CS, p.T - c0);  // valid tokens (>= 1); rows past them read the last valid one
    w.n = n;
    // the chunk's first row (b, c0, h) as wave-uniform base pointers; rows r as 32-bit element offsets
    const size_t rb = ((size_t)b * p.T + c0) * p.H + h;
    const uint32_t rs = (uint32_t)p.H * D;
    auto roff = [&](int r) { return (uint32_t)min(r, n - 1) * rs; };
    const float* gb = p.g + rb * D;
    const void* qb = (const char*)p.q + rb * D * (IN_BF16 ? 2 : 4);
    const void* kb = (const char*)p.k + rb * D * (IN_BF16 ? 2 : 4);
    {
        constexpr int TS = SRaw<D>::TS;
        const int ch = u % D, r0 = TS * (u / D);
#pragma unroll
        for (int r = 0; r < CS; ++r) w.g[r] = gb[roff(r) + ch];  // (every share needs the cumulative sums)
#pragma unroll
        for (int r = 0; r < TS; ++r) {
            w.q[r] = ldr<IN_BF16>(qb, roff(r0 + r) + ch);
            w.k[r] = ldr<IN_BF16>(kb, roff(r0 + r) + ch);
        }
    }
    if (u < CS) w.beta = p.beta[rb + (size_t)min(u, n - 1) * p.H];
    if (p.dO) {  // (one branch around the loads: a select per loaded value would make each load wait)
        const void* ob = (const char*)p.dO + (rb * D + half * DH) * (DO_BF16 ? 2 : 4);
#pragma unroll
        for (int k = 0; k < SRaw<D>::PV; ++k) {
            const int e = u + NTH * k, r = e / DH, j = e % DH;
            w.dO[k] = ldr<DO_BF16>(ob, roff(r) + j);
        }
    } else {  // dO == NULL: zero (never dereferenced)
#pragma unroll
        for (int k = 0; k < SRaw<D>::PV; ++k) w.dO[k] = 0u;
    }
}

// The chunk's factors (tokens past the valid ones are zeroed: k = q = 0, g = 0, beta = 0, dO = 0).
template <int D, bool IN_BF16, bool DO_BF16>
__device__ __forceinline__ void build_s(SChunk<D>& c, const SRaw<D>& w, float scale) {
    constexpr int DH = D / 2;
    const int u = threadIdx.x - NTH;
    const int n = w.n;
    {
        constexpr int TS = SRaw<D>::TS;
        const int ch = u % D, r0 = TS * (u / D);
        float bc[CS];
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < CS; ++r) {
            s += r < n ? w.g[r] : 0.f;
            bc[r] = s;
        }
        const float last = bc[CS - 1], gl = fexp(last);
        if (r0 == 0) c.gam[ch] = gl;
        // this thread's share of tokens (a compile-time offset per branch keeps bc in registers)
        auto share = [&](auto r0c) {
            constexpr int R0 = decltype(r0c)::value;
#pragma unroll
            for (int r = 0; r < TS; ++r) {
                const int t = R0 + r;
                const float q = t < n ? cvt<IN_BF16>(w.q[r], ch & 1) * scale : 0.f;
                const float k = t < n ? cvt<IN_BF16>(w.k[r], ch & 1) : 0.f;
                const float e = fexp(bc[t]), f = fexp(-bc[t]);  // exp(b), exp(-b), both within [e^-80, e^80]
                c.Qg[t][ch] = q * e;
                c.Kg[t][ch] = k * e;
                c.Kh[t][ch] = k * f;
                c.Kb[t][ch] = k * (gl * f);  // exp(b_last - b)
            }
        };
        static_assert(CS / TS <= 4, "up to four shares per channel");
        switch (r0 / TS) {  // wave-uniform
            case 0: share(std::integral_constant<int, 0>{}); break;
            case 1: if constexpr (CS / TS > 1) share(std::integral_constant<int, TS>{}); break;
            case 2: if constexpr (CS / TS > 2) share(std::integral_constant<int, 2 * TS>{}); break;
            default: if constexpr (CS / TS > 3) share(std::integral_constant<int, 3 * TS>{}); break;
        }
    }
    if (u < CS) c.beta[u] = u < n ? w.beta : 0.f;
#pragma unroll
    for (int k = 0; k < SRaw<D>::PV; ++k) {
        const int e = u + NTH * k, r = e / DH, j = e % DH;
        c.dO[r][j] = r < n ? cvt<DO_BF16>(w.dO[k], j & 1) : 0.f;
    }
}

// One workgroup per (sequence, value half), reverse over 16-token chunks, as a two-stage pipeline:
// waves 0-3 carry dS through chunk j (dU = Kb dS + A^T dO, dX = Tm^T dU), while waves 4-7 build
// chunk j-1's factors, its Gram products L and A and its inverse, and fetch chunk j-3's inputs;
// then all waves update dS <- Diag(gam) dS + Qg^T dO - Kg^T dX.  Three barriers per chunk.
template <int D, int CK, bool IN_BF16, bool DO_BF16>
__global__ void __launch_bounds__(NT) kda_bwd_state_kernel(BwdParams p) {
    constexpr int DH = D / 2;
    static_assert(NT - CS * CS >= NTH && D <= NTH && CS <= NTH, "the factor waves own the inverse and the build");
    __shared__ SChunk<D> sc[2];
    __shared__ __attribute__((aligned(16))) float dU[CS][DH + VP], dX[CS][DH + VP];
    __shared__ __attribute__((aligned(16))) float dS[D][DH + VP];
    const int tid = threadIdx.x;
    const bool chain = tid < NTH;  // waves 0-3
    const int bh = blockIdx.x >> 1, half = blockIdx.x & 1;
    const int b = bh / p.H, h = bh - b * p.H;
    const int nint = p.nint;
    auto at = [&](int i) { return ((size_t)bh * nint + i) * D * D + half * DH; };  // [bh][i][row][half*DH + col]

    for (int e = tid; e < D * DH; e += NT) {
        const int r = e / DH, j = e % DH;
        const float v = p.dST ? p.dST[(size_t)bh * D * D + (size_t)r * D + half * DH + j] : 0.f;
        dS[r][j] = v;
        p.dSb[at(nint - 1) + (size_t)r * D + j] = v;
    }
    const int nch = (p.T + CS - 1) / CS;
    constexpr int SPI = CK / CS;  // chunks per interval
    // the last chunk's factors; the next two chunks' inputs in flight (iteration k of the loop below
    // builds chunk nch-2-k from register set k & 1 and refills that set with chunk nch-4-k; chunk
    // indices below 0 read chunk 0 again, unused)
    SRaw<D> wa, wb;
    if (!chain) {
        fetch_s<D, IN_BF16, DO_BF16>(wb, p, b, h, (nch - 1) * CS, half);
        build_s<D, IN_BF16, DO_BF16>(sc[(nch - 1) & 1], wb, p.scale);
        fetch_s<D, IN_BF16, DO_BF16>(wa, p, b, h, max(nch - 2, 0) * CS, half);
        fetch_s<D, IN_BF16, DO_BF16>(wb, p, b, h, max(nch - 3, 0) * CS, half);
    }
    __syncthreads();
    {
        SChunk<D>& c = sc[(nch - 1) & 1];
        gram_products<D, 4>(c);
        __syncthreads();
        unit_inverse(c);
        __syncthreads();
    }
    // Zeroing of the outputs the input-gradient kernel accumulates into (when zero_in_state): dbeta
    // here, and this workgroup's share of dq, dk and dg a few 16-byte stores per chain thread per
    // step, in the chain waves' idle time of the first phase.
    const size_t nz4 = p.zero_in_state ? (size_t)p.B * p.T * p.H * D / 4 : 0;
    const size_t z0 = nz4 * blockIdx.x / gridDim.x, z1 = nz4 * (blockIdx.x + 1) / gridDim.x;
    const size_t zps = (z1 - z0 + (size_t)nch * NTH - 1) / ((size_t)nch * NTH);  // per chain thread and step
    if (p.zero_in_state && p.dbeta) {
        const size_t nb = (size_t)p.B * p.T * p.H;
        for (size_t e = nb * blockIdx.x / gridDim.x + tid; e < nb * (blockIdx.x + 1) / gridDim.x; e += NT) p.dbeta[e] = 0.f;
    }
    auto step = [&](const int cj, SRaw<D>& w) {
        SChunk<D>& c = sc[cj & 1];         // this chunk
        SChunk<D>& cn = sc[(cj - 1) & 1];  // the next one (chunk cj - 1)
        const bool next = cj >= 1;
        // dU = Kb dS + A^T dO  |  the next chunk's factors; its successor's inputs
        mgemm_w<CS, DH, D, 0, 4>([&](int m, int k) { return row4(c.Kb, m, k); }, [&](int k, int n) { return col4(dS, k, n); },
                                 [&](int m, int n, float v) { dU[m][n] = v; });
        mgemm_w<CS, DH, CS, 0, 4>([&](int m, int k) { return col4(c.A, k, m); }, [&](int k, int n) { return col4(c.dO, k, n); },
                                  [&](int m, int n, float v) { dU[m][n] += v; });
        if (!chain && next) {
            build_s<D, IN_BF16, DO_BF16>(cn, w, p.scale);
            fetch_s<D, IN_BF16, DO_BF16>(w, p, b, h, max(cj - 3, 0) * CS, half);
        }
        // the chain waves, done with dU long before the build: their share of the zeroing, and the
        // gradient of the state at the start of chunk cj + 1 when an interval starts there (dS
        // changes only in the last phase)
        if (chain && zps > 0) {
            const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
            const size_t zb = z0 + (size_t)(nch - 1 - cj) * zps * NTH + tid;
            for (size_t j = 0; j < zps; ++j) {
                const size_t z = zb + j * NTH;
                if (z < z1) {
                    if (p.dq) reinterpret_cast<float4*>(p.dq)[z] = zero;
                    if (p.dk) reinterpret_cast<float4*>(p.dk)[z] = zero;
                    if (p.dg) reinterpret_cast<float4*>(p.dg)[z] = zero;
                }
            }
        }
        if (chain && (cj + 1) % SPI == 0 && cj + 1 < nch) {
            for (int e = tid; e < D * DH; e += NTH) {
                const int r = e / DH, j = e % DH;
                p.dSb[at((cj + 1) / SPI - 1) + (size_t)r * D + j] = dS[r][j];
            }
        }
        __syncthreads();
        // dX = Tm^T dU  |  the next chunk's L and A
        mgemm_w<CS, DH, CS, 0, 4>([&](int m, int k) { return col4(c.Tm, k, m); }, [&](int k, int n) { return col4(dU, k, n); },
                                  [&](int m, int n, float v) { dX[m][n] = v; });
        if (next) gram_products<D, 4>(cn);
        __syncthreads();
        // the next inverse (waves 4-7), then on all waves
        // dS <- Diag(gam) dS + Qg^T dO - Kg^T dX   (each entry read and written by its own thread)
        if (next) unit_inverse(cn);
        state_grad_step<D, IN_BF16>(c.Qg, c.Kg, c.dO, dX, c.gam, dS, dS);
        __syncthreads();
    };
    for (int cj = nch - 1; cj >= 0; cj -= 2) {
        step(cj, wa);
        if (cj >= 1) step(cj - 1, wb);
    }
    if (p.dS0) {
        for (int e = tid; e < D * DH; e += NT) {
            const int r = e / DH, j = e % DH;
            p.dS0[(size_t)bh * D * D + (size_t)r * D + half * DH + j] = dS[r][j];
        }
    }
}

// ------------------------------------------------------------------------------------------------
// 3. input gradients, one interval per workgroup (value half)
// ------------------------------------------------------------------------------------------------
template <int D>
struct alignas(16) Grad {
    static constexpr int DH = D / 2;
    float G[CS][D + KP];      // one key-side gradient at a time (dKb, dQg, dKg, dKh), then db
    float P[D][DH + VP];       // state / state-gradient tiles of the current chunk (this value half):
    float Q[D][DH + VP];       // which is which depends on the chunk, see the kernel
    float dA[CS][CS + SP], dTm[CS][CS + SP], dM[CS][CS + SP];
    float dgam[D], dlast[D];
    float dbeta[CS];
};

// On one wave (lane 0..63): dN = dTm Diag(beta);  dbeta = colsum(N * dTm);  dM = -N^T dN N^T;
// dbeta += rowsum(dM * L);  dL = tril(Diag(beta) dM, -1), kept in dM.  In registers: the first
// product is formed transposed, T1^T = dN^T N, so that its accumulator (lane (l16, g) holds rows
// 4g..4g+3 of column l16) is the B operand of the second, dM^T = -N T1^T, whose accumulator then holds
// row l16 of dM, columns 4g..4g+3; the row and column sums reduce over the four lane groups.
template <int D>
__device__ __forceinline__ void dl_chain(Chunk<D>& c, Grad<D>& gr, int lane) {
    static_assert(CS == 16, "one 16 x 16 tile");
    const int l16 = lane & 15, g = lane >> 4, k = 4 * g;
    const f32x4 dtm = col4(gr.dTm, k, l16), nc = col4(c.N, k, l16);  // rows 4g.. of column l16
    const float bl = c.beta[l16];
    f32x4 t = {0.f, 0.f, 0.f, 0.f}, d = t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t = __builtin_amdgcn_mfma_f32_16x16x4f32(dtm[r] * bl, nc[r], t, 0, 0, 0);
    const f32x4 nr = row4(c.N, l16, k);
#pragma unroll
    for (int r = 0; r < 4; ++r) d = __builtin_amdgcn_mfma_f32_16x16x4f32(nr[r], t[r], d, 0, 0, 0);
    // d[r] = -dM[l16][4g + r]
    const f32x4 lr = row4(c.L, l16, k);
    float cs = 0.f, rs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        cs = __builtin_fmaf(nc[r], dtm[r], cs);  // column l16 of N * dTm, rows 4g..
        rs = __builtin_fmaf(-d[r], lr[r], rs);   // row l16 of dM * L, columns 4g..
    }
    float a = cs + rs;
    a += __shfl_xor(a, 16, 64);
    a += __shfl_xor(a, 32, 64);
    if (g == 0) gr.dbeta[l16] = a;
    f32x4 dl;
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[r] = k + r < l16 ? -bl * d[r] : 0.f;
    *reinterpret_cast<f32x4*>(&gr.dM[l16][k]) = dl;
}

// This thread's entries e = tid + NT*k of the value-half tile src[r][col0 + j] (r = e / DH,
// j = e % DH) of a [D][D] float32 matrix in global memory (NULL = zeros), into registers; put_state
// writes them to an LDS tile.
template <int D>
__device__ __forceinline__ void fetch_state(float* v, const float* src, int col0) {
    constexpr int DH = D / 2;
    // (one branch around all the loads: a select per loaded value would make each load wait)
    if (src) {
#pragma unroll
        for (int k = 0; k < D * DH / NT; ++k) {
            const int e = threadIdx.x + NT * k, r = e / DH, j = e % DH;
            v[k] = src[(size_t)r * D + col0 + j];
        }
    } else {
#pragma unroll
        for (int k = 0; k < D * DH / NT; ++k) v[k] = 0.f;
    }
}
template <int D>
__device__ __forceinline__ void put_state(float (*dst)[D / 2 + VP], const float* v) {
    constexpr int DH = D / 2;
#pragma unroll
    for (int k = 0; k < D * DH / NT; ++k) {
        const int e = threadIdx.x + NT * k;
        dst[e / DH][e % DH] = v[k];
    }
}

template <int D, int CK, bool IN_BF16, bool DO_BF16>
__global__ void __launch_bounds__(NT) kda_bwd_chunk_kernel(BwdParams p) {
    constexpr int DH = D / 2;
    constexpr int PER = CS * D / NT;  // key-side tile entries per thread (e = tid + NT * k)
    __shared__ Chunk<D> c;
    __shared__ Grad<D> gr;
    const int tid = threadIdx.x;
    // Work items (interval, value half), item = 2 * (bh * nint + i) + half, taken by the workgroups in
    // turn (item = blockIdx.x + k * gridDim.x); each workgroup reads its next item's state tiles and
    // inputs while it computes the last chunk of the current one.
    const int nitems = 2 * p.B * p.H * p.nint;
    constexpr int SPT = D * DH / NT;
    float s0r[SPT], dsr[SPT];
    Raw<D> w, w1;
    // start state of the interval and the gradient of the state after it (global, full rows), and the
    // inputs of its first chunk, into registers
    auto fetch_item = [&](int item) {
        const int hf = item & 1, wj = item >> 1;
        const int bj = wj / p.nint, ij = wj - bj * p.nint;
        const int bb = bj / p.H, hh = bj - bb * p.H;
        const int ns = (min(CK, p.T - ij * CK) + CS - 1) / CS;
        const float* S0g = ij == 0 ? (p.S0 ? p.S0 + (size_t)bj * D * D : nullptr) : p.Sck + ((size_t)bj * p.nck + ij - 1) * D * D;
        fetch_state<D>(s0r, S0g, hf * DH);
        fetch_state<D>(dsr, p.dSb + ((size_t)bj * p.nint + ij) * D * D, hf * DH);
        fetch_chunk<D, IN_BF16, DO_BF16>(w, p, bb, hh, ij * CK, hf, true);
    };
    fetch_item(blockIdx.x);
    for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
        const int half = item & 1;
        const int wi = item >> 1;
        const int bh = wi / p.nint, i = wi - bh * p.nint;
        const int b = bh / p.H, h = bh - b * p.H;
        const int col0 = half * DH;
        const int nsub = (min(CK, p.T - i * CK) + CS - 1) / CS;
        // the second chunk's inputs (if any), first needed after the first chunk's state step
        fetch_chunk<D, IN_BF16, DO_BF16>(w1, p, b, h, i * CK + (nsub - 1) * CS, half, true);

        // Buffers: one chunk:  P = start state, Q = end gradient.
        // Two chunks: P = start state -> Q = state after the first chunk; second chunk: S = Q, dS = P
        // (the interval's end gradient); its start gradient goes to Q; first chunk: S = P (start state
        // again), dS = Q.
        put_state<D>(gr.P, s0r);
        if (nsub == 2) {  // Q = Diag(gam) S + Kb^T Tm (V - Kg S)
            build_chunk<D, IN_BF16, DO_BF16>(c, w, p.scale, true);
            __syncthreads();
            // L and A (waves 4, 5) beside X = V - Kg S (waves 0-3), then the inverse
            gram_products<D, 4>(c);
            mgemm_w<CS, DH, D, 0, 4>([&](int m, int k) { return row4(c.Kg, m, k); }, [&](int k, int n) { return col4(gr.P, k, n); },
                                     [&](int m, int n, float v) { c.X[m][n] -= v; });
            __syncthreads();
            unit_inverse(c);
            __syncthreads();
            mgemm<CS, DH, CS>([&](int m, int k) { return row4(c.Tm, m, k); }, [&](int k, int n) { return col4(c.X, k, n); },
                                   [&](int m, int n, float v) { c.U[m][n] = v; });
            __syncthreads();
            state_fwd_step<D, IN_BF16>(c.Kb, c.U, c.gam, gr.P, gr.Q);
            __syncthreads();
            put_state<D>(gr.P, dsr);
        } else {
            put_state<D>(gr.Q, dsr);
        }
        __syncthreads();
        // the interval's chunks in reverse (written out twice rather than looped, so that the registers
        // holding the prefetched inputs are live only where they are needed)
        auto step = [&](const int s) {
            const int c0 = i * CK + s * CS;
            float (*Sb)[DH + VP] = (nsub == 2 && s == 1) ? gr.Q : gr.P;
            float (*dSb)[DH + VP] = (nsub == 2 && s == 1) ? gr.P : gr.Q;
            if (nsub == 2 && s == 1) {
                build_chunk<D, IN_BF16, DO_BF16>(c, w1, p.scale, true);
            } else {
                build_chunk<D, IN_BF16, DO_BF16>(c, w, p.scale, true);
                // every register input of this item is used: read the next item's
                if (item + (int)gridDim.x < nitems) fetch_item(item + gridDim.x);
            }
            __syncthreads();
            // L and A (waves 4, 5) beside X = V - Kg S (waves 0-3); the inverse (waves 4-7) beside Kb dS
            gram_products<D, 4>(c);
            mgemm_w<CS, DH, D, 0, 4>([&](int m, int k) { return row4(c.Kg, m, k); }, [&](int k, int n) { return col4(Sb, k, n); },
                                     [&](int m, int n, float v) { c.X[m][n] -= v; });
            __syncthreads();
            unit_inverse(c);
            mgemm_w<CS, DH, D, 0, 4>([&](int m, int k) { return row4(c.Kb, m, k); }, [&](int k, int n) { return col4(dSb, k, n); },
                                     [&](int m, int n, float v) { c.dU[m][n] = v; });
            __syncthreads();
            // U = Tm X
            mgemm<CS, DH, CS>([&](int m, int k) { return row4(c.Tm, m, k); }, [&](int k, int n) { return col4(c.X, k, n); },
                                   [&](int m, int n, float v) { c.U[m][n] = v; });
            __syncthreads();
            // dU += A^T dO;  dKb = U dS^T;  dgam = rowsum(dS * S)
            mgemm<CS, DH, CS>([&](int m, int k) { return col4(c.A, k, m); }, [&](int k, int n) { return col4(c.dO, k, n); },
                                   [&](int m, int n, float v) { c.dU[m][n] += v; });
            mgemm<CS, D, DH>([&](int m, int k) { return row4(c.U, m, k); }, [&](int k, int n) { return row4(dSb, n, k); },
                                  [&](int m, int n, float v) { gr.G[m][n] = v; });
            {  // dgam: NT / D consecutive lanes per channel, each a slice of the columns, then a shuffle sum
                constexpr int NP = NT / D, SL = DH / NP;
                const int ch = tid / NP, pt = tid % NP;
                float a = 0.f;
    #pragma unroll
                for (int j = 0; j < SL; ++j) a = __builtin_fmaf(dSb[ch][pt * SL + j], Sb[ch][pt * SL + j], a);
    #pragma unroll
                for (int o = NP / 2; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
                if (pt == 0) gr.dgam[ch] = a;
            }
            __syncthreads();
            // fold dKb: dk = dKb exp(b_last - b);  db = -dKb Kb;  last row: sum_t dKb Kb + dgam gam
            float dKr[PER], dbr[PER];
    #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = tid + NT * k, r = e / D, ch = e % D;
                const float gk = gr.G[r][ch];
                dKr[k] = gk * (c.gam[ch] / c.Gam[r][ch]);
                dbr[k] = -gk * c.Kb[r][ch];
            }
            if (tid < D) {
                float a = gr.dgam[tid] * c.gam[tid];
                for (int r = 0; r < CS; ++r) a = __builtin_fmaf(gr.G[r][tid], c.Kb[r][tid], a);
                gr.dlast[tid] = a;
            }
            // dTm = dU X^T (wave 4);  dA = tril(dO U^T) (wave 5);  dX = Tm^T dU  (dv)
            mgemm<CS, CS, DH>([&](int m, int k) { return row4(c.dU, m, k); }, [&](int k, int n) { return row4(c.X, n, k); },
                                   [&](int m, int n, float v) { gr.dTm[m][n] = v; }, 4);
            mgemm<CS, CS, DH>([&](int m, int k) { return row4(c.dO, m, k); }, [&](int k, int n) { return row4(c.U, n, k); },
                                   [&](int m, int n, float v) { gr.dA[m][n] = n <= m ? v : 0.f; }, 5);
            mgemm<CS, DH, CS>([&](int m, int k) { return col4(c.Tm, k, m); }, [&](int k, int n) { return col4(c.dU, k, n); },
                                   [&](int m, int n, float v) { c.dX[m][n] = v; });
            __syncthreads();
            // the dTm -> dL chain on wave 7, then dQg = dO S^T + dA Kh on all waves (then
            // dq = dQg scale Gamma, Qg holding the scale, and db += dQg Qg)
            if (tid >= NT - 64) dl_chain(c, gr, tid & 63);
            mgemm<CS, D, DH>([&](int m, int k) { return row4(c.dO, m, k); }, [&](int k, int n) { return row4(Sb, n, k); },
                             [&](int m, int n, float v) { gr.G[m][n] = v; });
            mgemm<CS, D, CS>([&](int m, int k) { return row4(gr.dA, m, k); }, [&](int k, int n) { return col4(c.Kh, k, n); },
                             [&](int m, int n, float v) { gr.G[m][n] += v; });
            __syncthreads();
            const int n_ok = min(CS, p.T - c0);
            auto grow = [&](int r) { return ((size_t)b * p.T + c0 + r) * p.H + h; };
    #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = tid + NT * k, r = e / D, ch = e % D;
                const float gq = gr.G[r][ch];
                dbr[k] = __builtin_fmaf(gq, c.Qg[r][ch], dbr[k]);
                if (r < n_ok && p.dq) atomicAdd(&p.dq[grow(r) * D + ch], gq * p.scale * c.Gam[r][ch]);
            }
            __syncthreads();
            // dKg = -dX S^T + dL Kh -> dk += dKg Gamma, db += dKg Kg
            mgemm<CS, D, DH>([&](int m, int k) { return row4(c.dX, m, k); }, [&](int k, int n) { return row4(Sb, n, k); },
                                  [&](int m, int n, float v) { gr.G[m][n] = -v; });
            mgemm<CS, D, CS>([&](int m, int k) { return row4(gr.dM, m, k); }, [&](int k, int n) { return col4(c.Kh, k, n); },
                                  [&](int m, int n, float v) { gr.G[m][n] += v; });
            __syncthreads();
    #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = tid + NT * k, r = e / D, ch = e % D;
                const float gk = gr.G[r][ch];
                dKr[k] = __builtin_fmaf(gk, c.Gam[r][ch], dKr[k]);
                dbr[k] = __builtin_fmaf(gk, c.Kg[r][ch], dbr[k]);
            }
            __syncthreads();
            // dKh = dL^T Kg + dA^T Qg -> dk += dKh / Gamma, db -= dKh Kh
            mgemm<CS, D, CS>([&](int m, int k) { return col4(gr.dM, k, m); }, [&](int k, int n) { return col4(c.Kg, k, n); },
                                  [&](int m, int n, float v) { gr.G[m][n] = v; });
            mgemm<CS, D, CS>([&](int m, int k) { return col4(gr.dA, k, m); }, [&](int k, int n) { return col4(c.Qg, k, n); },
                                  [&](int m, int n, float v) { gr.G[m][n] += v; });
            __syncthreads();
    #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = tid + NT * k, r = e / D, ch = e % D;
                const float gh = gr.G[r][ch];
                dKr[k] += gh / c.Gam[r][ch];
                dbr[k] = __builtin_fmaf(-gh, c.Kh[r][ch], dbr[k]);
                if (r < n_ok && p.dk) atomicAdd(&p.dk[grow(r) * D + ch], dKr[k]);
            }
            __syncthreads();
    #pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int e = tid + NT * k;
                gr.G[e / D][e % D] = dbr[k];
            }
            // outputs of the chunk: dv, dbeta, dg (reverse cumulative sum of db)
            for (int e = tid; e < CS * DH; e += NT) {
                const int r = e / DH, j = e % DH;
                if (r < n_ok && p.dv) p.dv[grow(r) * D + col0 + j] = c.dX[r][j];
            }
            if (tid < CS && tid < n_ok && p.dbeta) atomicAdd(&p.dbeta[grow(tid)], gr.dbeta[tid]);
            __syncthreads();
            if (tid < D && p.dg) {
                float a = gr.dlast[tid];
                for (int r = CS - 1; r >= 0; --r) {
                    a += gr.G[r][tid];
                    if (r < n_ok) atomicAdd(&p.dg[grow(r) * D + tid], a);
                }
            }
            if (nsub == 2 && s == 1) {
                // the gradient of the state between the two chunks, Diag(gam) dS + Qg^T dO - Kg^T dX,
                // into Q (the state S of this chunk, no longer read); then P gets the start state back
                __syncthreads();
                state_grad_step<D, IN_BF16>(c.Qg, c.Kg, c.dO, c.dX, c.gam, gr.P, gr.Q);
                __syncthreads();
                put_state<D>(gr.P, s0r);
            }
            __syncthreads();
        };
        if (nsub == 2) step(1);
        step(0);
    }
}

// Zero the accumulated outputs.
__global__ void kda_bwd_zero_kernel(float* a, size_t na, float* b, size_t nb, float* c, size_t nc, float* d, size_t nd) {
    const size_t st = (size_t)gridDim.x * blockDim.x;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < na + nb + nc + nd; e += st) {
        if (e < na) { if (a) a[e] = 0.f; }
        else if (e < na + nb) { if (b) b[e - na] = 0.f; }
        else if (e < na + nb + nc) { if (c) c[e - na - nb] = 0.f; }
        else if (d) d[e - na - nb - nc] = 0.f;
    }
}

template <int D, int CK, bool IN_BF16, bool DO_BF16>
hipError_t launch_kernels(const BwdParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((kda_bwd_state_kernel<D, CK, IN_BF16, DO_BF16>), dim3((unsigned)(2 * p.B * p.H)), dim3(NT), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per compute unit (its LDS allows no second), each taking every gridDim-th item
    int dev = 0, ncu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const size_t nitems = 2 * (size_t)p.B * p.H * p.nint;
    hipLaunchKernelGGL((kda_bwd_chunk_kernel<D, CK, IN_BF16, DO_BF16>),
                       dim3((unsigned)std::min(nitems, (size_t)std::max(ncu, 1))), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace bwd

size_t bwd_workspace_bytes(int B, int T, int H, int D, bool in_bf16) {
    const int CK = in_bf16 ? 32 : 16;
    const size_t nint = (size_t)(T + CK - 1) / CK;
    return 2 * (size_t)B * H * nint * D * D * sizeof(float);
}

hipError_t launch_bwd(const BwdParams& p0, bool in_bf16, bool do_bf16, bool precise, float* ws, hipStream_t stream) {
    BwdParams p = p0;
    const int D = p.D;
    const int CK = in_bf16 ? 32 : 16;
    p.nint = (p.T + CK - 1) / CK;
    p.nck = p.T / CK;  // checkpoints the forward records (entry i - 1 starts interval i)
    const size_t per = (size_t)p.B * p.H * p.nint * D * D;
    p.Sck = ws;
    p.dSb = ws + per;
    // 1. the forward's states at interval boundaries (entry i = after interval i)
    Params f{};  // zero: every optional field off
    f.q = p.q; f.k = p.k; f.v = p.v; f.g = p.g; f.beta = p.beta; f.S0 = p.S0; f.o = nullptr; f.S_T = nullptr;
    f.B = p.B; f.T = p.T; f.H = p.H; f.Dk = D; f.Dv = D; f.tstride = p.T; f.scale = p.scale;
    f.precise = precise;
    f.S_ckpt = ws; f.ckpt_chunks = 1; f.n_ckpt = p.T / CK;
    hipError_t e = hipSuccess;
    if (f.n_ckpt > 0) e = in_bf16 ? launch_fwd_bf16(f, stream) : launch_fwd_f32(f, stream);
    if (e != hipSuccess) return e;
    // 2. zero the accumulated outputs: inside the state pass when the float32 outputs allow 16-byte
    // stores, else by a kernel of its own
    auto a16 = [](const float* q) { return ((uintptr_t)q & 15) == 0; };
    p.zero_in_state = a16(p.dq) && a16(p.dk) && a16(p.dg);
    if (!p.zero_in_state) {
        const size_t nk = (size_t)p.B * p.T * p.H * D;
        hipLaunchKernelGGL(bwd::kda_bwd_zero_kernel, dim3(2048), dim3(256), 0, stream, p.dq, p.dq ? nk : 0, p.dk,
                           p.dk ? nk : 0, p.dg, p.dg ? nk : 0, p.dbeta, p.dbeta ? (size_t)p.B * p.T * p.H : 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 3. state gradients, then the input gradients
    if (!in_bf16) return D == 64 ? bwd::launch_kernels<64, 16, false, false>(p, stream)
                                 : bwd::launch_kernels<128, 16, false, false>(p, stream);
    return do_bf16 ? bwd::launch_kernels<128, 32, true, true>(p, stream)   // bf16 inputs: D = 128
                   : bwd::launch_kernels<128, 32, true, false>(p, stream);
}

}  // namespace kda
