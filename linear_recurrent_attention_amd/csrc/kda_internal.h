// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Validated problem, passed by value to the kernels.
struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* S0;   // may be null (zero state)
    void* o;
    float* S_T;        // may be null
    int B, T, H, Dk, Dv;
    int tstride;       // tokens between consecutive batch rows of every [B, *, H, D] tensor (>= T)
    float scale;
    int o_f32;         // bf16 inputs with a float32 output
    int in_f32;        // matrix-core path with float32 q, k, v (and float32 output); layer use
    int precise;       // matrix-core path: split-bf16 L and state update (always on with in_f32)
    float* S_ckpt;     // may be null: [B, H, n_ckpt, Dk, Dv] states at every ckpt_chunks-th chunk boundary
    int ckpt_chunks;   // chunks between checkpoints (>= 1 when S_ckpt is set)
    int n_ckpt;        // checkpoints per sequence: full multiples of ckpt_chunks chunks within T
    // bf16 path, optional (seg_cnt = 0: off): run batch rows (b / seg_cnt) * seg_n + seg_lo + b % seg_cnt
    // for b < B, i.e. seg_cnt of every seg_n rows, starting at row seg_lo (the context-parallel passes
    // that need only some segments of each sequence); every tensor is indexed by that row
    int seg_lo, seg_cnt, seg_n;
    // bf16 path, optional (seg_T = 0: off): rows are the seg_n segments of sequences of seg_T tokens;
    // row r is segment r % seg_n of sequence r / seg_n, starting at token (r % seg_n) * tstride of it,
    // tstride tokens long except the last segment, which runs to seg_T (T is then ignored)
    int seg_T;
    // bf16 path, optional (alt_b0 = 0: off): batch rows b >= alt_b0 of a launch are rows b - alt_b0 of a
    // second run with v = 0, initial and final states alt_S0 / alt_ST (may be the same array) and the
    // row subset alt_seg_lo, alt_seg_cnt (same seg_n): two state-only runs in one launch
    int alt_b0, alt_seg_lo, alt_seg_cnt;
    const float* alt_S0;
    float* alt_ST;
};

// Backward problem (all float32 gradients; NULL outputs are skipped).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* S0;   // may be null
    const void* dO;    // may be null (zero); dtype: bf16 or float32
    const float* dST;  // may be null (zero)
    float* dq;
    float* dk;
    float* dv;
    float* dg;
    float* dbeta;
    float* dS0;
    const float* Sck;  // workspace: states after each full interval [B*H][nck][D][D]
    float* dSb;        // workspace: state gradients after each interval [B*H][nint][D][D]
    int B, T, H, D;
    float scale;
    int nint, nck;     // intervals (ceil(T / interval)), checkpoints (T / interval)
    int zero_in_state; // the state pass zeroes dq, dk, dg (16-byte aligned) and dbeta
};

hipError_t launch_fwd_bf16(const Params& p, hipStream_t stream);  // Dk = Dv = 128, chunk 32 (in_f32 too)
hipError_t launch_fwd_f32(const Params& p, hipStream_t stream);   // Dk = Dv in {64, 128}, chunk 16
hipError_t launch_state_copy(const Params& p, hipStream_t stream); // T = 0: S_T = S0 (or 0)
// input checks of KDA_VALIDATE: clears *flags, then ORs in VALIDATE_* bits (device word, stream-ordered)
enum : uint32_t { VALIDATE_G_RANGE = 1u, VALIDATE_NONFINITE = 2u };
hipError_t launch_validate(const Params& p, bool in_bf16, uint32_t* flags, hipStream_t stream);
hipError_t launch_decode(const Params& p, bool in_bf16, hipStream_t stream);  // token by token, Dk = Dv in {64, 128}
// in-device context parallelism (bf16 I/O, Dk = Dv = 128): segment count nseg_req (0 = automatic)
size_t cp_workspace_bytes(int B, int T, int H, int nseg_req);
hipError_t launch_fwd_cp(const Params& p, int nseg_req, float* ws, hipStream_t stream);
// bf16 GEMM C = A Bt^T (A [M][K], Bt [N][K] row-major; K a multiple of 32, both row strides multiples
// of 8, A and Bt 16-byte aligned), float32 sums; the columns of C split into segments
// [start[s], start[s+1]), each written to ptr[s] (row stride ld[s], column start[s] at column 0,
// 16-byte aligned), as float32 or bf16.  Segment starts must be multiples of 4, start[0] = 0 and
// start[nseg] >= N.  epi = GEMM_GATE (one float32 segment) writes -5 sigmoid(exp(head_scale[n / 128])
// (C + bias[n])) instead of C: the decay gate of the fused layer.  epi = GEMM_QKCONV (float32 output,
// M a multiple of 256, qk_cols and qk_hd multiples of 128): columns [0, qk_cols) are the layer's q
// (the first qk_hd) and k projections, heads of 128 columns; each of their rows r of a 256-row tile
// gets the causal depthwise convolution over rows r-3..r (taps conv_q / conv_k, [column][4], tap 3
// on row r), SiLU and L2 over its head (x / sqrt(sum x^2 + eps)); rows 0-2 of each tile are not
// written (their window reaches into the tile above) and the tile's first and last three raw rows go
// to side[tile row][6][qk_cols] for the caller to finish them.
enum { GEMM_STORE = 0, GEMM_GATE = 1, GEMM_QKCONV = 2 };
struct GemmOut {
    static constexpr int kMaxSeg = 6;
    void* ptr[kMaxSeg];
    int start[kMaxSeg + 1];
    int ld[kMaxSeg];
    int nseg;
    int epi;
    const float* bias;
    const float* head_scale;
    const float* conv_q;  // GEMM_QKCONV
    const float* conv_k;
    float* side;
    int qk_cols, qk_hd;
    float eps;
    // bit s: segment s (float32 sums, width W = start[s+1] - start[s]) is written as bf16 hi + lo
    // halves into ptr[s] (bf16, row stride ld[s] >= 2W): hi = bf16(C) in columns [0, W), lo =
    // bf16(C - hi) in [W, 2W)
    int split_segs;
};
hipError_t launch_gemm_nt(const uint16_t* A, int lda, const uint16_t* Bt, int ldb, const GemmOut& out, bool out_f32,
                          int M, int N, int K, hipStream_t stream);
// Transposes in one launch: job i writes dst[n * ldd + k] = src[k * lds + n] for k < K, n < N (bf16).
// The caller fills src, dst, lds, ldd, K, N; the launch fills the rest.
struct TransposeJob {
    const uint16_t* src;
    uint16_t* dst;
    int lds, ldd, K, N;
    int tiles_n, first, vec;
};
struct TransposeBatch {
    static constexpr int kMax = 12;
    TransposeJob job[kMax];
    int njobs;
};
hipError_t launch_transpose_batch(TransposeBatch& b, hipStream_t stream);
// Fused layer decode step (four launches); see kda_layer_decode.hip.
struct LayerDecodeParams {
    const uint16_t* x;              // [B*T][dm] bf16
    const uint16_t* W[6];           // Wq, Wk, Wv, Wg, Wdown, Wbeta ([dm][wn[i]] bf16)
    int wn[6];
    int noff[7];                    // column offsets of the six in the partial-sum rows; noff[6] = total
    const uint16_t* Wup;            // [R][H*D]
    const uint16_t* Wo;             // [H*D][dm]
    const float *conv_q, *conv_k, *b_alpha, *A, *rms_w;
    float* S;                       // [B][H][D][D], read; written unless spec
    float* conv;                    // [B][3][2*H*D] or NULL (zeros in, nothing out)
    uint16_t* y;                    // [B*T][dm]
    float* cache;                   // planar cache entries or NULL
    float* part;                    // partial sums (layer_decode_part_floats)
    float* gated;                   // [B*T][H*D]
    int B, T, H, dm, R, spec;
    float scale;
};
size_t layer_decode_part_floats(int M, int dm, int HD, int ntot);
hipError_t launch_layer_decode(const LayerDecodeParams& p, hipStream_t stream);
hipError_t launch_window_commit(float* conv, const float* qpre, const float* kpre, int B, int T, int HD, int n,
                                hipStream_t stream);
// launch_fwd_cp with the library's static per-device scratch array (KDA_CP_NOALLOC_SCRATCH_BYTES);
// hipErrorInvalidValue if the plan needs more than that
hipError_t launch_fwd_cp_noalloc(const Params& p, int nseg_req, hipStream_t stream);
// backward: intervals of 32 tokens (bf16 inputs, D = 128) or 16 (float32 inputs, D in {64, 128})
size_t bwd_workspace_bytes(int B, int T, int H, int D, bool in_bf16);
hipError_t launch_bwd(const BwdParams& p, bool in_bf16, bool do_bf16, bool precise, float* ws, hipStream_t stream);

}  // namespace kda
