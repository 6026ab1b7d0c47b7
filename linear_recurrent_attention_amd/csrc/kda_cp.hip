// In-device context parallelism for long sequences, on gfx950.
//
// The explainer page "Kimi K3：开放前沿智能", section 13.3.1, splits one long sequence into segments
// evaluated side by side on one device, then merges them to recover each segment's initial state;
// section 13.3.2 states the decomposition that makes the merge possible: the state after segment i
// is M_i S_start(i) + S_hat_i, with M_i the segment's accumulated transition and S_hat_i its local
// state estimate (the segment run from a zero state).  Here each sequence is cut into nseg segments,
// the first nseg - 1 of Ls tokens (whole chunks) and the last one the rest, and:
//   1. one launch of the chunkwise kernel's state-only instantiation runs
//        S_hat_i: segments 0..nseg-2 from S = 0, except segment 0, which runs from the call's S0 and
//                 so gives S_start(1) itself, and
//        M_i:     segments 1..nseg-2 with v = 0 from S = I: the gated delta rule is linear in (S, v),
//                 so with v = 0 it maps the initial state through the segment, and from I it yields
//                 the transition matrix itself
//      (the last segment needs neither, and segment 0 no transition);
//   2. the scan S_start(0) = S0, S_start(1) = the first pass's segment 0,
//      S_start(i+1) = M_i S_start(i) + S_hat_i, in float32;
//   3. the chunkwise kernel over every segment at once from S_start(i), writing o and the segment's
//      final state; the last segment's is S_T.
// This is about three passes of work in exchange for nseg times more workgroups: worth it when
// 2*B*H workgroups leave most of the 256 compute units idle.  The automatic segment count minimises
// a small model of the three passes' time (rounds of 256 workgroups times tokens per segment, plus
// the scan's steps).
#include <cmath>
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

// Initial states of the first pass, in one launch: Sst gets S0 (or 0) for segment 0 of each of the B
// sequences and 0 for segments 1..nseg-2; M gets I for segments 1..nseg-2 (the transitions' start).
// Sst, M: [B][nseg][H][D][D]; S0: [B][H][D][D] or NULL.
__global__ void kda_cp_init_kernel(const float* __restrict__ S0, float* __restrict__ Sst, float* __restrict__ M,
                                   int B, int nseg, int H) {
    const size_t mat = (size_t)D * D, per_b = (size_t)(nseg - 1) * H * mat;  // segments 0..nseg-2
    const size_t n = (size_t)B * per_b;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < 2 * n; e += (size_t)gridDim.x * blockDim.x) {
        const bool ism = e >= n;
        const size_t f = ism ? e - n : e;
        const int b = (int)(f / per_b);
        const size_t r = f - (size_t)b * per_b;           // within sequence b: (s * H + h) * mat + w
        const int s = (int)(r / ((size_t)H * mat)), h = (int)((r / mat) % H);
        const size_t w = r % mat;
        const size_t at = (size_t)b * nseg * H * mat + r;  // [b][s][h][w]
        if (!ism)
            Sst[at] = (s == 0 && S0) ? S0[((size_t)b * H + h) * mat + w] : 0.f;
        else if (s > 0)
            M[at] = (w / D == w % D) ? 1.f : 0.f;
    }
}

// S_T[b] = the last segment's final state of sequence b (Shat: [B][nseg][H][D][D]; S_T: [B][H][D][D]).
__global__ void kda_cp_last_state_kernel(const float* __restrict__ Shat, float* __restrict__ ST, int B, int nseg,
                                         int H) {
    const size_t mat = (size_t)D * D, per_b = (size_t)H * mat;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < (size_t)B * per_b;
         e += (size_t)gridDim.x * blockDim.x) {
        const size_t b = e / per_b;
        ST[e] = Shat[(b * nseg + nseg - 1) * per_b + (e - b * per_b)];
    }
}

// Params of the chunkwise kernel over the nseg segments of all B sequences: row r is segment r % nseg
// of sequence r / nseg (Ls tokens, the last one the rest of the sequence).
Params seg_params(const Params& u, int nseg, int Ls) {
    Params p = u;
    p.B = u.B * nseg;
    p.T = Ls;
    p.tstride = Ls;
    p.seg_T = u.T;
    p.seg_n = nseg;
    p.S_ckpt = nullptr; p.ckpt_chunks = 1; p.n_ckpt = 0;
    return p;
}

// Modelled time of a plan, in units of one chunk step of one round of workgroups: the first pass
// (state-only, about 0.8 of a full step) and the output pass over T / nseg tokens, each in rounds of
// 256 workgroups, plus four chunk steps per scan step; nseg = 1 is the plain kernel.
double plan_cost(int B, int T, int H, int nseg) {
    const double n0 = 2.0 * B * H, chunks = T / 32.0;
    auto rounds = [](double wg) { return std::ceil(wg / 256.0); };
    if (nseg == 1) return chunks * rounds(n0);
    const double w1 = n0 * (nseg - 1) + n0 * (nseg > 2 ? nseg - 2 : 0);
    return chunks / nseg * (0.8 * rounds(w1) + rounds(n0 * nseg)) + 4.0 * (nseg - 2);
}

}  // namespace cp

// Number of segments the orchestration below will use, and the tokens of each but the last (0: plain
// run).  A requested count is kept if every segment gets at least one chunk; 0 picks the count of
// least modelled time among those with segments of at least 1024 tokens.
void cp_plan(int B, int T, int H, int nseg_req, int& nseg, int& Ls) {
    nseg = nseg_req;
    if (nseg == 0) {
        nseg = 1;
        double best = cp::plan_cost(B, T, H, 1);
        for (int n = 2; n <= 64 && T / n >= 1024; ++n) {
            const double c = cp::plan_cost(B, T, H, n);
            if (c < best) { best = c; nseg = n; }
        }
    }
    Ls = nseg >= 2 ? (T / (nseg * 32)) * 32 : 0;
    if (Ls == 0) nseg = 1;
}

size_t cp_workspace_bytes(int B, int T, int H, int nseg_req) {
    int nseg, Ls;
    cp_plan(B, T, H, nseg_req, nseg, Ls);
    if (nseg == 1) return 0;
    return 3 * cp::seg_floats(B, nseg, H) * sizeof(float);
}

hipError_t launch_fwd_cp(const Params& u, int nseg_req, float* ws, hipStream_t stream) {
    int nseg, Ls;
    cp_plan(u.B, u.T, u.H, nseg_req, nseg, Ls);
    if (nseg == 1) return launch_fwd_bf16(u, stream);
    const size_t n = cp::seg_floats(u.B, nseg, u.H);
    float* Shat = ws;
    float* M = ws + n;
    float* Sst = ws + 2 * n;
    hipError_t e;
    // 1. first-pass initial states (S0 or 0 into Sst, I into M), then one state-only launch: segments
    //    0..nseg-2 with v from their initial states into Shat (segment 0's final state, the others'
    //    local states), and as the launch's second row set the transitions of segments 1..nseg-2
    //    (v = 0 from I, in place in M)
    hipLaunchKernelGGL(cp::kda_cp_init_kernel, dim3(1024), dim3(256), 0, stream, u.S0, Sst, M, u.B, nseg, u.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    Params p = cp::seg_params(u, nseg, Ls);
    p.o = nullptr; p.S0 = Sst; p.S_T = Shat;
    p.B = u.B * (nseg - 1); p.seg_lo = 0; p.seg_cnt = nseg - 1;
    if (nseg > 2) {
        p.alt_b0 = p.B;
        p.B += u.B * (nseg - 2);
        p.alt_seg_lo = 1; p.alt_seg_cnt = nseg - 2;
        p.alt_S0 = M; p.alt_ST = M;
    }
    if ((e = launch_fwd_bf16(p, stream)) != hipSuccess) return e;
    // 2. initial state of every segment
    hipLaunchKernelGGL(cp::kda_cp_scan_kernel, dim3((unsigned)(u.B * u.H * (cp::D / cp::SCOLS))), dim3(cp::NTHR), 0,
                       stream, Shat, M, u.S0, Sst, nseg, u.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 3. outputs, and each segment's final state (into Shat, no longer needed); S_T is the last one's
    p = cp::seg_params(u, nseg, Ls);
    p.S0 = Sst; p.S_T = Shat;
    if ((e = launch_fwd_bf16(p, stream)) != hipSuccess) return e;
    if (u.S_T) {
        hipLaunchKernelGGL(cp::kda_cp_last_state_kernel, dim3(1024), dim3(256), 0, stream, Shat, u.S_T, u.B, nseg, u.H);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
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
