// bf16 matrix-core GEMM for the fused layer's projections, on gfx950.
//
//   C[m][n] = sum_k A[m][k] * Bt[n][k]      (A: [M][K] row-major, Bt: [N][K] row-major, float32 sums)
//
// Both operands are read along k, so their tiles go to LDS row by row and every matrix-core operand
// is one 16-byte LDS read.  The layer's weights are stored [in][out]; they are transposed into this
// form on each call (transpose_batch_kernel, all of them in one launch).
//
// Mapping.  A workgroup computes a 256 x 256 tile of C with 8 waves (2 x 4), each a 128 x 64 block
// of 8 x 4 products v_mfma_f32_16x16x32_bf16.  The operand tiles move 64 columns of k at a time
// (128-byte rows, so that every request to L2 is a whole cache line: with 64-byte rows the loads
// were bound by the requests in flight), straight from global memory into two LDS stages
// (global_load_lds_dwordx4: each lane's 16 bytes land at the stage base plus 16 * lane, so the lanes
// are given the global chunks that the XOR-swizzled layout puts there).  Tiles are numbered so that
// each XCD (the hardware deals workgroups to the eight XCDs in turn) gets one contiguous range of
// them, ordered in groups of four tile rows, so that the workgroups running together on one XCD
// share A and Bt panels in its L2.
//
// Schedule.  Waves w and w + 4 share a SIMD.  They run half a step apart ("ping-pong"): in every
// phase between two barriers one of them reads its operand fragments of a k step (32 columns) from
// LDS while the other issues its 32 products of the step before, so the matrix core of each SIMD is
// fed by one wave while the other waits on LDS.  Waves 0-3 read step u in phase 2u and multiply it
// in phase 2u + 1; waves 4-7 read it in phase 2u + 1 and multiply it in phase 2u + 2.  In the first
// step of stage s a wave issues its part of the loads of stage s + 1, into the other slot, which
// every wave finished reading before; each wave waits for its own loads (vmcnt 0) before the barrier
// that closes the last phase of stage s.  The sums are those of a plain k-ordered loop.
//
// Epilogue.  Each wave rewrites its block row-major through LDS and stores whole rows (16 lanes per
// 256-byte row segment), as nontemporal stores: every workgroup of a round stores at about the same
// time, and the store burst is HBM-bound; streaming stores shortened it by about 8% in timing runs.  The columns of C may be split into up to six segments, each written to
// its own matrix (pointer and row stride), so that one product over concatenated weights fills
// separate buffers; or the decay gate of the layer is applied on the way out (GEMM_GATE).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace gemm {

constexpr int BM = 256, BN = 256, BK = 32;  // BK: the k columns of one matrix-core step
constexpr int BK2 = 64, NST = 2;            // k columns per LDS stage, stages in the ring
constexpr int NW = 8, NTHR = 64 * NW;
constexpr int WM = 128, WN = 64;  // per wave

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void g_void;

// LDS tiles [rows][64] bf16 (128-byte rows): 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7), so that the 16 rows of a matrix-core operand read (one chunk each) fall in 16
// distinct bank groups.
__device__ __forceinline__ int swz64(int row, int chunk) { return row * BK2 + 8 * (chunk ^ ((row >> 1) & 7)); }

struct alignas(16) Smem {
    uint16_t a[NST][BM * BK2];
    uint16_t b[NST][BN * BK2];
    float qx[16 * 3 * 64 + 2 * 8 * 64];  // the q/k epilogue's halo rows and per-row partial sums
};
static_assert(sizeof(Smem) >= NW * 64 * 64 * sizeof(float), "the epilogue's staging fits in the operand ring");

// s_waitcnt with only vmcnt <= N (N < 64) constrained
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }
// execution barrier without a memory fence: the operand loads are waited for explicitly above it
__device__ __forceinline__ void exec_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)); }

// The q/k epilogue of GEMM_QKCONV, for a 256-row tile whose columns start below qk_cols.  Staged
// through LDS like the plain epilogue (64 rows of the wave's 128 x 64 block at a time); per element
// the 4-tap convolution over rows r-3..r, SiLU, then the L2 norm of the row over the head's 128
// columns: the blocks of waves 2p and 2p + 1, whose partial sums of squares meet in LDS.  The rows
// above a staged half come from halos: a wave's own rows 61-63 for its second half, and for the
// waves of rows 128-255 the last three rows of the waves above (written from the accumulators first).
// Column pairs past qk_cols (a tile straddling the end of k) are stored as plain sums.
__device__ __forceinline__ void qk_epilogue(Smem& sm, f32x4 (&acc)[8][4], const GemmOut& out, int M, int N, int m0,
                                            int n0, int wave, int lane) {
    const int l16 = lane & 15, g4 = lane >> 4, wm = wave >> 2, wn = wave & 3;
    float* stage = reinterpret_cast<float*>(&sm) + wave * (64 * 64);
    float* haloA = sm.qx;             // [wave][3][64]: raw rows 125-127 of each wave's block
    float* haloB = sm.qx + 8 * 192;   // [wave][3][64]: raw rows 61-63 of this wave's block
    float* psum = sm.qx + 16 * 192;   // [half][wave][64 rows]: sums of squares over the wave's columns
    const int colb = n0 + WN * wn;    // first column of this wave's block
    const bool fused = n0 + 128 * (wn >> 1) < out.qk_cols;
    const int tr = m0 / BM;
    const size_t qkc = (size_t)out.qk_cols;
    if (l16 >= 13) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<f32x4*>(&haloA[(wave * 3 + l16 - 13) * 64 + 16 * j + 4 * g4]) = acc[7][j];
    }
    if (fused) {  // the tile's first three and last three raw rows
        if (wm == 0 && l16 < 3) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(&out.side[((size_t)tr * 6 + l16) * qkc + colb + 16 * j + 4 * g4]) = acc[0][j];
        }
        if (wm == 1 && l16 >= 13) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(&out.side[((size_t)tr * 6 + l16 - 10) * qkc + colb + 16 * j + 4 * g4]) =
                    acc[7][j];
        }
    }
    // lane (sr, l16) takes rows 16 sr .. 16 sr + 15 of each staged half, columns c0 .. c0 + 3
    const int sr = lane >> 4, sc = 4 * (lane & 15);
    const int c0 = colb + sc;
    f32x4 tw[4] = {};  // tw[t][e]: tap t of column c0 + e
    if (fused) {
        const float* taps = c0 < out.qk_hd ? out.conv_q + (size_t)c0 * 4 : out.conv_k + (size_t)(c0 - out.qk_hd) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(taps + 4 * e);
#pragma unroll
            for (int t = 0; t < 4; ++t) tw[t][e] = w[t];
        }
    }
    int seg = 0;
#pragma unroll
    for (int t = 1; t < GemmOut::kMaxSeg; ++t) seg += (t < out.nseg && c0 >= out.start[t]) ? 1 : 0;
    const int c = c0 - out.start[seg];
    const int lim = min(min(4, N - c0), out.start[seg + 1] - c0);
    float* base = static_cast<float*>(out.ptr[seg]);
    const size_t ld = (size_t)out.ld[seg];
    const bool vec = lim == 4 && (out.ld[seg] & 3) == 0;
    wait_lgkm0();
    exec_barrier();  // every wave's halo rows are in LDS
    auto row_at = [&](const float* st, int r) {
        return *reinterpret_cast<const f32x4*>(&st[r * 64 + 4 * ((sc >> 2) ^ (r & 15))]);
    };
    // sum over the 16 lanes of a row of lanes, left in the row's last lane (DPP row shifts)
    auto row_sum = [](float v) {
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true));
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true));
        return v;
    };
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(&stage[(16 * i + l16) * 64 + 4 * ((4 * j + g4) ^ l16)]) = acc[4 * half + i][j];
        wait_lgkm0();
        f32x4 x[19];  // raw rows 16 sr - 3 .. 16 sr + 15
        if (fused) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[3 + r] = row_at(stage, 16 * sr + r);
            if (sr > 0) {
#pragma unroll
                for (int r = 0; r < 3; ++r) x[r] = row_at(stage, 16 * sr - 3 + r);
            } else if (half == 1) {
#pragma unroll
                for (int r = 0; r < 3; ++r) x[r] = *reinterpret_cast<const f32x4*>(&haloB[(wave * 3 + r) * 64 + sc]);
            } else if (wm == 1) {
#pragma unroll
                for (int r = 0; r < 3; ++r) x[r] = *reinterpret_cast<const f32x4*>(&haloA[((wave - 4) * 3 + r) * 64 + sc]);
            } else {
#pragma unroll
                for (int r = 0; r < 3; ++r) x[r] = f32x4{0.f, 0.f, 0.f, 0.f};  // tile rows 0-2: finished by the caller
            }
            if (half == 0 && sr == 3) {  // raw rows 61-63 for the second half
#pragma unroll
                for (int r = 0; r < 3; ++r) *reinterpret_cast<f32x4*>(&haloB[(wave * 3 + r) * 64 + sc]) = x[16 + r];
            }
            // convolution and SiLU in place (row r reads raw rows r .. r + 3 of x, so go from the top)
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float y = 0.f;
#pragma unroll
                    for (int t = 0; t < 4; ++t) y = __builtin_fmaf(tw[t][e], x[r + t][e], y);
                    y = y * (1.f / (1.f + __builtin_amdgcn_exp2f(-y * kLog2e)));
                    x[r + 3][e] = y;
                    ss = __builtin_fmaf(y, y, ss);
                }
                ss = row_sum(ss);
                if (l16 == 15) psum[(half * 8 + wave) * 64 + 16 * sr + r] = ss;
            }
        }
        wait_lgkm0();
        exec_barrier();  // both waves' partial sums of every row of this half
        f32x4 inv[4];
        if (fused) {
            const int pa = (half * 8 + (wave & ~1)) * 64 + 16 * sr, pb = (half * 8 + (wave | 1)) * 64 + 16 * sr;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 sa = *reinterpret_cast<const f32x4*>(&psum[pa + 4 * q4]);
                const f32x4 sb = *reinterpret_cast<const f32x4*>(&psum[pb + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) inv[q4][e] = __builtin_amdgcn_rsqf(sa[e] + sb[e] + out.eps);
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = 16 * sr + r;
            const int m = m0 + WM * wm + 64 * half + rl;
            if (m >= M || lim <= 0) continue;
            f32x4 v;
            if (fused) {
                if (half == 0 && wm == 0 && rl < 3) continue;  // tile rows 0-2
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = x[r + 3][e] * inv[r >> 2][r & 3];
            } else {
                v = row_at(stage, rl);
            }
            float* dst = base + (size_t)m * ld + c;
            if (vec) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
            else for (int e = 0; e < lim; ++e) dst[e] = v[e];
        }
        wait_lgkm0();  // the next half overwrites the staging rows
    }
}

// One tile (or one piece of a split tile) of C: rows [pm0, pm0 + 32 NI) of the tile whose first row
// is the A stage's row 0 at pm0, columns [n0, n0 + 256).  Each wave multiplies NI 16-row blocks by
// its four 16-column blocks: NI = 8 for a whole 256-row tile, 4 or 2 for a half or quarter.
template <bool OUT_F32, int EPI, int NI>
__device__ __forceinline__ void gemm_tile(Smem& sm, const uint16_t* __restrict__ A, int lda,
                                          const uint16_t* __restrict__ Bt, int ldb, const GemmOut& out, int M, int N,
                                          int K, int pm0, int n0, int wave, int lane) {
    const int l16 = lane & 15, g4 = lane >> 4;
    constexpr int WR = 16 * NI;  // rows per wave

    // loads: wave w moves rows [32w, 32w + 32) of both stages, four 1 KB instructions (8 rows of
    // 128 bytes each); lane l takes row base + l/8 at physical chunk l%8, i.e. logical chunk
    // (l%8) ^ ((row >> 1) & 7).  Rows past M (N) read row M-1 (N-1); their results are never stored.
    // A last stage of 32 k columns (K = 32 mod 64) reads its first half again in place of the second.
    const int lr = 32 * wave + (lane >> 3);
    const uint16_t* ag[4];
    const uint16_t* bg[4];
    int lch[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int row = lr + 8 * h;
        lch[h] = (lane & 7) ^ ((row >> 1) & 7);
        ag[h] = A + (size_t)min(pm0 + row, M - 1) * lda;
        bg[h] = Bt + (size_t)min(n0 + row, N - 1) * ldb;
    }
    const int nsub = K / BK, nk = (nsub + 1) / 2;  // k32 sub-steps, 64-column stages
    auto issue = [&](int kt, int st) {
        const int k0 = kt * BK2;
        const bool half = 2 * kt + 1 >= nsub;  // only the first 32 columns exist
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int row = 32 * wave + 8 * h;
            const int c = half ? (lch[h] & 3) : lch[h];
            __builtin_amdgcn_global_load_lds((g_void*)(ag[h] + k0 + 8 * c), (lds_void*)&sm.a[st][row * BK2], 16, 0, 0);
            __builtin_amdgcn_global_load_lds((g_void*)(bg[h] + k0 + 8 * c), (lds_void*)&sm.b[st][row * BK2], 16, 0, 0);
        }
    };

    const int wm = wave >> 2, wn = wave & 3;
    const bool late = wave >= 4;  // waves 4-7: half a step behind
    f32x4 acc[NI][4];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 af[NI], bf[4];
    auto frags = [&](int st, int sub) {
        const uint16_t* sa = sm.a[st];
        const uint16_t* sb = sm.b[st];
#pragma unroll
        for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const u32x4*>(&sa[swz64(WR * wm + 16 * i + l16, g4 + 4 * sub)]);
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const u32x4*>(&sb[swz64(WN * wn + 16 * j + l16, g4 + 4 * sub)]);
        wait_lgkm0();
    };
    // Bt as the first operand: lane (l16, g4) gets row m = l16 of the block, columns 4*g4 .. 4*g4+3
    auto mma = [&]() {
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(bf[j], af[i], acc[i][j]);
    };

    // phases as before, one per k32 sub-step and group; stage st + 1 is issued in the first sub-step
    // of stage st (into the other slot, whose stage every wave finished reading before) and waited
    // for (vmcnt 0: nothing later is in flight) before the barrier that closes stage st's last phase
    issue(0, 0);
    wait_vm<0>();
    exec_barrier();
    if (late) exec_barrier();  // waves 4-7 sit out phase 0 (and waves 0-3 the last phase)
    for (int u = 0; u < nsub; ++u) {
        const int st = u >> 1, sub = u & 1;
        if (sub == 0 && st + 1 < nk) issue(st + 1, (st + 1) & 1);
        frags(st & 1, sub);
        const bool last_of_stage = sub == 1 || u + 1 == nsub;
        if (late && last_of_stage && st + 1 < nk) wait_vm<0>();
        exec_barrier();
        mma();
        if (!late && last_of_stage && st + 1 < nk) wait_vm<0>();
        if (!late || u + 1 < nsub) exec_barrier();
    }

    if constexpr (EPI == GEMM_QKCONV && NI == 8) {
        if (n0 < out.qk_cols) {  // (workgroup-uniform)
            qk_epilogue(sm, acc, out, M, N, pm0, n0, wave, lane);
            return;
        }
    }

    // epilogue through LDS: each wave rewrites its block row-major in its own 16 KB of the ring (64
    // rows at a time, 16-byte blocks XOR-swizzled by row), then stores whole rows: lane (sr, l16)
    // stores columns 4*l16 .. 4*l16+3 of row 4*r4 + sr.  Every operand read and load finished before
    // the last barrier, so no wave waits for the others here.
    float* stage = reinterpret_cast<float*>(&sm) + wave * (64 * 64);
    const int sr = lane >> 4, sc = 4 * (lane & 15);
    const int nb = n0 + WN * wn + sc;  // this lane's first column
    int seg = 0;
#pragma unroll
    for (int t = 1; t < GemmOut::kMaxSeg; ++t) seg += (t < out.nseg && nb >= out.start[t]) ? 1 : 0;
    const int c = nb - out.start[seg];
    const int lim = min(min(4, N - nb), out.start[seg + 1] - nb);  // segments start on multiples of 4
    char* base = static_cast<char*>(out.ptr[seg]);
    const size_t ld = (size_t)out.ld[seg];
    const bool vec = lim == 4 && (out.ld[seg] & 3) == 0;  // (segment bases are 16-byte aligned)
    const bool split = OUT_F32 && ((out.split_segs >> seg) & 1);  // (lim == 4 there: checked at launch)
    const int split_w = out.start[seg + 1] - out.start[seg];
    f32x4 gb = {0.f, 0.f, 0.f, 0.f};
    float ga = 0.f;
    if constexpr (EPI == GEMM_GATE) {  // log decay -5 sigmoid(exp(A_h) (z + b)), head h = column / 128
        if (lim > 0) {
            for (int e = 0; e < lim; ++e) gb[e] = out.bias[nb + e];
            ga = __builtin_amdgcn_exp2f(out.head_scale[nb >> 7] * kLog2e);
        }
    }
#pragma unroll
    for (int half = 0; half < (NI + 3) / 4; ++half) {
        constexpr int NH = NI < 4 ? NI : 4;  // 16-row blocks per staged half
#pragma unroll
        for (int i = 0; i < NH; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(&stage[(16 * i + l16) * 64 + 4 * ((4 * j + g4) ^ l16)]) = acc[4 * half + i][j];
        wait_lgkm0();
#pragma unroll
        for (int r4 = 0; r4 < 4 * NH; ++r4) {
            const int rl = 4 * r4 + sr;
            f32x4 v = *reinterpret_cast<const f32x4*>(&stage[rl * 64 + 4 * ((sc >> 2) ^ (rl & 15))]);
            const int m = pm0 + WR * wm + 64 * half + rl;
            if (m >= M || lim <= 0) continue;
            if constexpr (EPI == GEMM_GATE) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = -5.f * sigmoid_f(ga * (v[e] + gb[e]));
            }
            if constexpr (OUT_F32) {
                if (split) {  // bf16 hi in columns [0, W), the remainder in [W, 2W) of the row
                    uint16_t* dst = reinterpret_cast<uint16_t*>(base) + (size_t)m * ld + c;
                    uint32_t h01, l01, h23, l23;
                    split_bf16(v[0], v[1], h01, l01);
                    split_bf16(v[2], v[3], h23, l23);
                    *reinterpret_cast<u32x2*>(dst) = u32x2{h01, h23};
                    *reinterpret_cast<u32x2*>(dst + split_w) = u32x2{l01, l23};
                    continue;
                }
                float* dst = reinterpret_cast<float*>(base) + (size_t)m * ld + c;
                if (vec) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
                else for (int e = 0; e < lim; ++e) dst[e] = v[e];
            } else {
                uint16_t* dst = reinterpret_cast<uint16_t*>(base) + (size_t)m * ld + c;
                if (vec) __builtin_nontemporal_store(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, reinterpret_cast<u32x2*>(dst));
                else for (int e = 0; e < lim; ++e) dst[e] = (uint16_t)(pack_bf16(v[e], 0.f) & 0xffffu);
            }
        }
        wait_lgkm0();  // the next half overwrites the staging rows
    }
}

// Tiles are numbered so that each XCD gets a contiguous range of them (see the header).  When the
// tile count leaves a partial last round (at most half of the 256 compute units busy), that round's
// tiles are split along M into sf = 4 (or 2) pieces of 64 (128) rows, each a workgroup of its own on
// the XCD of its tile; on each XCD up to 16 pieces run first, then the whole tiles, then the rest.
template <bool OUT_F32, int EPI>
__global__ void __launch_bounds__(NTHR, 1) gemm_nt_kernel(const uint16_t* __restrict__ A, int lda,
                                                          const uint16_t* __restrict__ Bt, int ldb, GemmOut out,
                                                          int M, int N, int K, int nfull, int sf) {
    __shared__ Smem sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN, total = tm * tn;
    const int xcd = blockIdx.x & 7, q = total >> 3, rem = total & 7;
    const int first = xcd * q + min(xcd, rem);  // this XCD's first tile
    int pid, piece = -1;
    if (sf == 1) {  // whole tiles only (nfull = the tile count)
        if ((int)blockIdx.x >= nfull) return;
        pid = first + (blockIdx.x >> 3);
    } else {
        // nfull (a multiple of 256) whole tiles, then the pieces.  w: ordinal on this XCD in the order
        // [whole tiles][pieces]; the first half of the XCD's compute units start with one piece each
        // and the others with whole tiles, so the two halves run a quarter tile apart and their
        // epilogue stores do not all reach HBM at once.
        const int F = nfull / 8, cnt = q + (xcd < rem ? 1 : 0) - F;  // whole and split tiles of this XCD
        const int v = blockIdx.x >> 3, hs = min(16, sf * cnt);
        const int w = v < hs ? F + v : v < hs + F ? v - hs : v;
        if (w < F) {
            pid = first + w;
        } else {
            const int t = (w - F) / sf;
            if (t >= cnt) return;  // (the whole workgroup)
            pid = first + F + t;
            piece = (w - F) % sf;
        }
    }
    constexpr int GM = 4;
    const int in_group = GM * tn, first_m = (pid / in_group) * GM, gsize = min(tm - first_m, GM);
    const int im = first_m + (pid % in_group) % gsize, jn = (pid % in_group) / gsize;
    const int m0 = im * BM, n0 = jn * BN;
    if (piece < 0)
        gemm_tile<OUT_F32, EPI, 8>(sm, A, lda, Bt, ldb, out, M, N, K, m0, n0, wave, lane);
    else if (sf == 2)
        gemm_tile<OUT_F32, EPI, 4>(sm, A, lda, Bt, ldb, out, M, N, K, m0 + 128 * piece, n0, wave, lane);
    else
        gemm_tile<OUT_F32, EPI, 2>(sm, A, lda, Bt, ldb, out, M, N, K, m0 + 64 * piece, n0, wave, lane);
}

// Batched transpose: job j writes dst[n * ldd + k] = src[k * lds + n] for k < K, n < N (bf16), one
// 64 x 64 tile per workgroup, every job of a call in one launch (the layer's weights are a handful
// of small matrices, so separate launches would cost more than their bytes).  A job's rows are
// moved as 16-byte chunks when both matrices allow it (vec).
__global__ void __launch_bounds__(256) transpose_batch_kernel(TransposeBatch batch) {
    __shared__ uint16_t t[64][72];  // [k][n], rows padded by 16 bytes
    TransposeJob J = batch.job[0];
#pragma unroll
    for (int i = 1; i < TransposeBatch::kMax; ++i)
        if (i < batch.njobs && (int)blockIdx.x >= batch.job[i].first) J = batch.job[i];
    const int local = (int)blockIdx.x - J.first;
    const int k0 = (local / J.tiles_n) * 64, n0 = (local % J.tiles_n) * 64;
    const int K = J.K, N = J.N;
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
        const int r = e >> 3, c8 = 8 * (e & 7);  // k row, first n of the chunk
        const int k = k0 + r, n = n0 + c8;
        if (J.vec && k < K && n + 8 <= N) {
            *reinterpret_cast<u32x4*>(&t[r][c8]) = *reinterpret_cast<const u32x4*>(J.src + (size_t)k * J.lds + n);
        } else {
            for (int x = 0; x < 8; ++x)
                t[r][c8 + x] = (k < K && n + x < N) ? J.src[(size_t)k * J.lds + n + x] : (uint16_t)0;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 8; e += 256) {
        const int r = e >> 3, c8 = 8 * (e & 7);  // n row, first k of the chunk
        const int n = n0 + r, k = k0 + c8;
        if (n >= N) continue;
        uint16_t v[8];
        for (int x = 0; x < 8; ++x) v[x] = t[c8 + x][r];
        if (J.vec && k + 8 <= K) {
            u32x4 w;
            for (int x = 0; x < 4; ++x) w[x] = (uint32_t)v[2 * x] | ((uint32_t)v[2 * x + 1] << 16);
            *reinterpret_cast<u32x4*>(J.dst + (size_t)n * J.ldd + k) = w;
        } else {
            for (int x = 0; x < 8; ++x)
                if (k + x < K) J.dst[(size_t)n * J.ldd + k + x] = v[x];
        }
    }
}


}  // namespace gemm

hipError_t launch_gemm_nt(const uint16_t* A, int lda, const uint16_t* Bt, int ldb, const GemmOut& out, bool out_f32,
                          int M, int N, int K, hipStream_t stream) {
    using namespace gemm;
    if (M <= 0 || N <= 0 || K <= 0 || K % BK || lda % 8 || ldb % 8 || out.nseg < 1 || out.nseg > GemmOut::kMaxSeg)
        return hipErrorInvalidValue;
    if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(Bt) & 15)) return hipErrorInvalidValue;
    for (int s = 0; s < out.nseg; ++s)
        if (out.start[s] % 4 || out.start[s + 1] <= out.start[s] || !out.ptr[s] || out.ld[s] < 1 ||
            (reinterpret_cast<uintptr_t>(out.ptr[s]) & 15))
            return hipErrorInvalidValue;
    if (out.start[0] != 0 || out.start[out.nseg] < N) return hipErrorInvalidValue;
    if (out.epi == GEMM_GATE && (out.nseg != 1 || !out_f32 || !out.bias || !out.head_scale)) return hipErrorInvalidValue;
    for (int s = 0; s < out.nseg; ++s)  // hi + lo segments: whole 4-column groups inside N, room for both halves
        if (((out.split_segs >> s) & 1) &&
            (!out_f32 || out.start[s + 1] > N || out.ld[s] < 2 * (out.start[s + 1] - out.start[s]) || out.ld[s] % 4 ||
             (out.epi == GEMM_QKCONV && out.start[s] < out.qk_cols)))
            return hipErrorInvalidValue;
    if (out.split_segs >> out.nseg) return hipErrorInvalidValue;
    if (out.epi == GEMM_QKCONV &&
        (!out_f32 || M % BM || out.qk_cols < 128 || out.qk_cols % 128 || out.qk_hd % 128 || out.qk_hd > out.qk_cols ||
         out.qk_cols > N || !out.conv_q || !out.conv_k || !out.side || (reinterpret_cast<uintptr_t>(out.side) & 15)))
        return hipErrorInvalidValue;
    const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles > (1L << 30)) return hipErrorInvalidValue;
    // a partial last round of at most 64 (128) tiles runs as 64-row (128-row) pieces (not when one of
    // them holds q/k columns of GEMM_QKCONV, whose epilogue needs whole tiles)
    const long nfull = tiles / 256 * 256, tail = tiles - nfull;
    int sf = (nfull > 0 && tail > 0) ? (tail <= 64 ? 4 : tail <= 128 ? 2 : 1) : 1;
    if (sf > 1 && out.epi == GEMM_QKCONV) {
        const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN, in_group = 4 * tn;
        for (long pid = nfull; pid < tiles; ++pid) {  // the tail tiles, numbered as in the kernel
            const int first_m = (int)(pid / in_group) * 4, gsize = min(tm - first_m, 4);
            const int jn = (int)(pid % in_group) / gsize;
            if (jn * BN < out.qk_cols) sf = 1;
        }
    }
    long nwg = tiles;
    if (sf > 1) nwg = nfull + 8L * sf * ((tiles / 8 - nfull / 8) + (tiles % 8 ? 1 : 0));
    const int nf = sf > 1 ? (int)nfull : (int)tiles;
    const dim3 grid((unsigned)nwg), block(NTHR);
    if (out.epi == GEMM_GATE)
        hipLaunchKernelGGL((gemm_nt_kernel<true, GEMM_GATE>), grid, block, 0, stream, A, lda, Bt, ldb, out, M, N, K,
                           nf, sf);
    else if (out.epi == GEMM_QKCONV)
        hipLaunchKernelGGL((gemm_nt_kernel<true, GEMM_QKCONV>), grid, block, 0, stream, A, lda, Bt, ldb, out, M, N, K,
                           nf, sf);
    else if (out_f32)
        hipLaunchKernelGGL((gemm_nt_kernel<true, GEMM_STORE>), grid, block, 0, stream, A, lda, Bt, ldb, out, M, N, K,
                           nf, sf);
    else
        hipLaunchKernelGGL((gemm_nt_kernel<false, GEMM_STORE>), grid, block, 0, stream, A, lda, Bt, ldb, out, M, N, K,
                           nf, sf);
    return hipGetLastError();
}

hipError_t launch_transpose_batch(TransposeBatch& b, hipStream_t stream) {
    if (b.njobs < 1 || b.njobs > TransposeBatch::kMax) return hipErrorInvalidValue;
    long total = 0;
    for (int i = 0; i < b.njobs; ++i) {
        TransposeJob& J = b.job[i];
        if (J.K < 1 || J.N < 1 || !J.src || !J.dst) return hipErrorInvalidValue;
        J.tiles_n = (J.N + 63) / 64;
        J.first = (int)total;
        J.vec = J.lds % 8 == 0 && J.ldd % 8 == 0 && (reinterpret_cast<uintptr_t>(J.src) & 15) == 0 &&
                (reinterpret_cast<uintptr_t>(J.dst) & 15) == 0;
        total += (long)J.tiles_n * ((J.K + 63) / 64);
        if (total > (1L << 30)) return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(gemm::transpose_batch_kernel, dim3((unsigned)total), dim3(256), 0, stream, b);
    return hipGetLastError();
}


}  // namespace kda
