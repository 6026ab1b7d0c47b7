// In-device context parallelism for long sequences, on gfx950.
//
// The explainer page "Kimi K3：开放前沿智能", section 13.3.1, splits one long sequence into segments
// evaluated side by side on one device, then merges them to recover each segment's initial state;
// section 13.3.2 states the decomposition that makes the merge possible: the state after segment i
// is M_i S_start(i) + S_hat_i, with M_i the segment's accumulated transition and S_hat_i its local
// state estimate (the segment run from a zero state).  Here, for nseg segments of Ls tokens:
//   1. S_hat_i: the chunkwise kernel from S = 0 (no output), for segments 1..nseg-2; segment 0 runs
//               from the call's S0 instead, which gives S_start(1) itself;
//      M_i:     the same kernel with v = 0 and S = I (no output), for segments 1..nseg-2: the gated
//               delta rule is linear in (S, v), so with v = 0 it maps the initial state through the
//               segment, and from I it yields the transition matrix itself;
//      (the last segment needs neither, and segment 0 no transition);
//   2. the scan S_start(0) = S0, S_start(1) = the first pass's segment 0,
//      S_start(i+1) = M_i S_start(i) + S_hat_i, in float32;
//   3. the chunkwise kernel over every segment at once from S_start(i), writing o and the segment's
//      final state; the last segment's is S_T.
// Both first-pass launches run only the segments they need (the kernel's batch-row subset) and use
// its state-only instantiation.
// A sequence too short for B*H*nseg to matter, or T not a multiple of nseg*32, is handled by running
// the whole multiple of nseg*32 this way and the remaining tail with the plain kernel from the last
// segment's state.  This is three passes of work in exchange for nseg times more workgroups: worth it
// when 2*B*H workgroups leave most of the 256 compute units idle.
#include <mutex>

#include "kda.h"
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace cp {

constexpr int D = 128;
constexpr int SCOLS = 16;  // state columns per scan workgroup
constexpr int NTHR = 256;  // 16 row groups of 8 rows x 16 columns

// Scan over segments for one (batch, head) and 16 state columns.  Shat, M: [B][nseg][H][D][D];
// S0: [B][H][D][D] or NULL; Sst (out): [B][nseg][H][D][D], entry i = S_start(i).
__global__ void __launch_bounds__(NTHR) kda_cp_scan_kernel(const float* __restrict__ Shat, const float* __restrict__ M,
                                                           const float* __restrict__ S0, float* __restrict__ Sst,
                                                           int nseg, int H) {
    __shared__ float Ms[D][D + 1];  // M_i; the odd pitch puts rows 8 apart in different banks
    __shared__ float Sc[D][SCOLS];  // the current S_start(i), these columns
    const int tid = threadIdx.x, c = tid & (SCOLS - 1), rg = tid / SCOLS;
    const int ncb = D / SCOLS;
    const int bh = blockIdx.x / ncb, cb = blockIdx.x - bh * ncb;
    const int b = bh / H, h = bh - b * H;
    const int col = cb * SCOLS + c;
    auto at = [&](int i) { return ((size_t)(b * nseg + i) * H + h) * D * D; };

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = rg * 8 + i;
        Sst[at(0) + (size_t)row * D + col] = S0 ? S0[(size_t)bh * D * D + (size_t)row * D + col] : 0.f;
    }
    // S_start(1): segment 0's final state, which the first pass computed from S0 (nseg >= 2 here)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = rg * 8 + i;
        acc[i] = Shat[at(0) + (size_t)row * D + col];
        Sc[row][c] = acc[i];
        Sst[at(1) + (size_t)row * D + col] = acc[i];
    }
    for (int s = 1; s + 1 < nseg; ++s) {
        __syncthreads();  // Sc holds S_start(s); the previous step is done with Ms
        const float4* src = reinterpret_cast<const float4*>(M + at(s));
        for (int e = tid; e < D * D / 4; e += NTHR) {
            const float4 m = src[e];
            const int row = (4 * e) / D, cm = (4 * e) % D;
            Ms[row][cm] = m.x; Ms[row][cm + 1] = m.y; Ms[row][cm + 2] = m.z; Ms[row][cm + 3] = m.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = Shat[at(s) + (size_t)(rg * 8 + i) * D + col];
        __syncthreads();
        for (int k = 0; k < D; ++k) {
            const float sk = Sc[k][c];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(Ms[rg * 8 + i][k], sk, acc[i]);
        }
        __syncthreads();  // every read of Sc is done
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = rg * 8 + i;
            Sc[row][c] = acc[i];
            Sst[at(s + 1) + (size_t)row * D + col] = acc[i];
        }
    }
}

size_t seg_floats(int Bg, int nseg, int H) { return (size_t)Bg * nseg * H * D * D; }

// Initial states of the first pass: S0 (or 0) for segment 0 of each of Bg sequences, 0 for the others.
// Sst: [Bg][nseg][H][D][D]; S0: [Bg][H][D][D] or NULL.
__global__ void kda_cp_seed_kernel(const float* __restrict__ S0, float* __restrict__ Sst, int Bg, int nseg, int H) {
    const size_t mat = (size_t)D * D, n = (size_t)Bg * nseg * H * mat;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t m = e / mat, w = e - m * mat;  // m = (b * nseg + s) * H + h
        const int h = (int)(m % H), s = (int)((m / H) % nseg), b = (int)(m / ((size_t)H * nseg));
        Sst[e] = (s == 0 && S0) ? S0[((size_t)b * H + h) * mat + w] : 0.f;
    }
}

// n D x D identity matrices, back to back.
__global__ void kda_cp_identity_kernel(float* __restrict__ S, size_t n) {
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n * D * D; e += (size_t)gridDim.x * blockDim.x) {
        const int w = (int)(e % ((size_t)D * D));
        S[e] = (w / D == w % D) ? 1.f : 0.f;
    }
}

// Params of the chunkwise kernel over the nseg segments of Bg batches starting at batch b0: each
// segment is a batch row of its own (row stride Ls tokens), which matches the [B, T, H, D] layout
// when the group's sequences are exactly nseg * Ls tokens long, or when the group is one sequence.
Params seg_params(const Params& u, int b0, int Bg, int nseg, int Ls) {
    Params p = u;
    const size_t tok = (size_t)b0 * u.T * u.H;  // first row of batch b0
    const size_t esz = u.in_f32 ? 4 : 2;        // q, k, v element size
    p.q = (const char*)u.q + tok * D * esz;
    p.k = (const char*)u.k + tok * D * esz;
    p.v = (const char*)u.v + tok * D * esz;
    p.g = u.g + tok * D;
    p.beta = u.beta + tok;
    p.o = u.o ? (char*)u.o + tok * D * (u.o_f32 ? 4 : 2) : nullptr;
    p.B = Bg * nseg;
    p.T = Ls;
    p.tstride = Ls;
    p.S_ckpt = nullptr; p.ckpt_chunks = 1; p.n_ckpt = 0;
    return p;
}

}  // namespace cp

// Number of segments the orchestration below will use, and the tokens per segment (0: plain run).
void cp_plan(int B, int T, int H, int nseg_req, int& nseg, int& Ls) {
    nseg = nseg_req;
    if (nseg == 0) {  // enough segments for about one workgroup per compute unit, each >= 1024 tokens
        nseg = 1;
        while (2 * B * H * nseg * 2 <= 256 && T / (nseg * 2) >= 1024) nseg *= 2;
    }
    Ls = nseg >= 2 ? (T / (nseg * 32)) * 32 : 0;
    if (Ls == 0) nseg = 1;
}

size_t cp_workspace_bytes(int B, int T, int H, int nseg_req) {
    int nseg, Ls;
    cp_plan(B, T, H, nseg_req, nseg, Ls);
    if (nseg == 1) return 0;
    const int Bg = (nseg * Ls == T) ? B : 1;
    return 3 * cp::seg_floats(Bg, nseg, H) * sizeof(float);
}

hipError_t launch_fwd_cp(const Params& u, int nseg_req, float* ws, hipStream_t stream) {
    int nseg, Ls;
    cp_plan(u.B, u.T, u.H, nseg_req, nseg, Ls);
    if (nseg == 1) return launch_fwd_bf16(u, stream);
    const int Tm = nseg * Ls;
    const int Bg = (Tm == u.T) ? u.B : 1;  // a ragged tail is run per sequence
    const size_t n = cp::seg_floats(Bg, nseg, u.H);
    float* Shat = ws;
    float* M = ws + n;
    float* Sst = ws + 2 * n;
    hipError_t e = hipSuccess;
    for (int b0 = 0; b0 < u.B && e == hipSuccess; b0 += Bg) {
        const float* S0 = u.S0 ? u.S0 + (size_t)b0 * u.H * cp::D * cp::D : nullptr;
        // 1. segments 0..nseg-2 from their first-pass states (S0 for segment 0, else 0, seeded into the
        //    buffer step 2 fills later): segment 0's final state and the others' local states
        hipLaunchKernelGGL(cp::kda_cp_seed_kernel, dim3(1024), dim3(256), 0, stream, S0, Sst, Bg, nseg, u.H);
        if ((e = hipGetLastError()) != hipSuccess) break;
        Params p = cp::seg_params(u, b0, Bg, nseg, Ls);
        p.o = nullptr; p.S0 = Sst; p.S_T = Shat;
        p.B = Bg * (nseg - 1); p.seg_lo = 0; p.seg_cnt = nseg - 1; p.seg_n = nseg;
        if ((e = launch_fwd_bf16(p, stream)) != hipSuccess) break;
        //    the transitions of segments 1..nseg-2 (v = 0 from I, in place in M)
        if (nseg > 2) {
            hipLaunchKernelGGL(cp::kda_cp_identity_kernel, dim3(1024), dim3(256), 0, stream, M,
                               (size_t)Bg * nseg * u.H);
            if ((e = hipGetLastError()) != hipSuccess) break;
            p.v = nullptr; p.S0 = M; p.S_T = M;
            p.B = Bg * (nseg - 2); p.seg_lo = 1; p.seg_cnt = nseg - 2;
            if ((e = launch_fwd_bf16(p, stream)) != hipSuccess) break;
        }
        // 2. initial state of every segment
        hipLaunchKernelGGL(cp::kda_cp_scan_kernel, dim3((unsigned)(Bg * u.H * (cp::D / cp::SCOLS))), dim3(cp::NTHR), 0,
                           stream, Shat, M, S0, Sst, nseg, u.H);
        if ((e = hipGetLastError()) != hipSuccess) break;
        // 3. outputs, and each segment's final state (into Shat, no longer needed)
        p = cp::seg_params(u, b0, Bg, nseg, Ls);
        p.S0 = Sst; p.S_T = Shat;
        if ((e = launch_fwd_bf16(p, stream)) != hipSuccess) break;
        // the sequence's final state: the last segment's, or carried through the tail
        for (int b = 0; b < Bg && e == hipSuccess; ++b) {
            const float* last = Shat + ((size_t)(b * nseg + nseg - 1) * u.H) * cp::D * cp::D;
            float* ST = u.S_T ? u.S_T + (size_t)(b0 + b) * u.H * cp::D * cp::D : nullptr;
            Params t = u;
            t.B = 1; t.S0 = last; t.S_T = ST;
            t.S_ckpt = nullptr; t.ckpt_chunks = 1; t.n_ckpt = 0;
            if (Tm < u.T) {  // Bg == 1 here
                const size_t tok = ((size_t)(b0 + b) * u.T + Tm) * u.H;
                const size_t esz = u.in_f32 ? 4 : 2;
                t.q = (const char*)u.q + tok * cp::D * esz;
                t.k = (const char*)u.k + tok * cp::D * esz;
                t.v = (const char*)u.v + tok * cp::D * esz;
                t.g = u.g + tok * cp::D;
                t.beta = u.beta + tok;
                t.o = (char*)u.o + tok * cp::D * (u.o_f32 ? 4 : 2);
                t.T = u.T - Tm;
                t.tstride = t.T;
                e = launch_fwd_bf16(t, stream);
            } else if (ST) {
                t.T = 0;
                e = launch_state_copy(t, stream);
            }
        }
    }
    return e;
}

// Scratch of kda_fwd_cp_noalloc: the segment states (S_hat, M, S_start) in a fixed device array, so
// that the call allocates nothing.  Each device holds its own copy of the array from the moment the
// library's code object is loaded on it until the process ends.  Every call on a device shares that
// device's copy; nothing in it needs to start at zero (each pass writes what the next one reads).
namespace {

constexpr size_t kNoallocScratchBytes = KDA_CP_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, looked up once

// Device address of the current device's copy of `scratch`.  In host code the array's name stands
// for a host-side shadow, not device memory, so kernels are given this address instead.
hipError_t scratch_on_current_device(float** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = static_cast<float*>(ptr);
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_fwd_cp_noalloc(const Params& u, int nseg_req, hipStream_t stream) {
    if (cp_workspace_bytes(u.B, u.T, u.H, nseg_req) > kNoallocScratchBytes) return hipErrorInvalidValue;
    float* ws = nullptr;
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return e;
    return launch_fwd_cp(u, nseg_req, ws, stream);
}

}  // namespace kda
