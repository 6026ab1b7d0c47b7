/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The operation is the gated delta rule of the explainer page
 * "Kimi K3：开放前沿智能" (kimi-k3-paper.pages.dev):
 *   section 2.2 (paper Eq. 1): S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   section 2.3: alpha_t in (0,1)^{d_k}, one forget rate per key channel, given here as g = log(alpha),
 *   section 2.4: o_t = S_t^T q_t, read after the update,
 *   section 2.5 (paper Eq. 4): computed chunk by chunk, an inter-chunk term Gamma*Q*S plus an
 *   intra-chunk lower-triangular term A*V_hat, with the d_k x d_v state handed from chunk to chunk,
 *   section 3.2 (paper Eq. 5): log(alpha) is bounded below by g_min = -5, which the kernels rely on.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent), owned by the caller.
 *     The library allocates no device memory in its calls; a call that needs scratch memory takes
 *     it from a caller workspace, sized by the query beside it (kda_fwd_cp_noalloc: from a fixed
 *     array that is part of the library's code object).
 *   - Calls are asynchronous and ordered on `stream` (NULL = the default stream).  The return code
 *     covers argument validation and launch errors only; a fault inside a kernel surfaces at the
 *     caller's next synchronisation.
 *   - Tensors are dense, row-major, without padding, in the layouts given per argument.
 *   - No entry point keeps global mutable state, except kda_fwd_cp_noalloc's fixed scratch array
 *     (one per device).  Calls from several host threads are safe, except overlapping calls of
 *     kda_fwd_cp_noalloc on one device, which share that array.
 *   - Outputs must not alias inputs, except S_T == S0 (in-place state carry), which is allowed:
 *     each workgroup reads its slice of S0 before it writes the same slice of S_T.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer, bad flag */
    KDA_ERR_UNSUPPORTED = -2,  /* valid request this build has no kernel for (e.g. a head size) */
    KDA_ERR_HIP = -3,          /* the HIP runtime reported an error at launch */
    KDA_ERR_WORKSPACE = -4,    /* workspace pointer missing or smaller than the size query said */
    KDA_ERR_SCRATCH_LIMIT = -5 /* an allocation-free entry point was given a problem whose scratch
                                  exceeds its fixed buffer */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Problem description for kda_fwd. */
typedef struct {
    int B, T, H;        /* batch, tokens, heads; B, H >= 1, T >= 0 */
    int Dk, Dv;         /* key / value head size.  bf16 I/O: Dk = Dv = 128.  f32 I/O: Dk = Dv in {64, 128} */
    int chunk;          /* tokens per chunk of the chunkwise form that the caller asks for: 0 (library
                           default) or a multiple of the kernel's chunk up to 64, i.e. 32 or 64 for bf16
                           I/O and 16, 32, 48 or 64 for f32 I/O.  The kernels always block by their own
                           chunk (bf16: 32 tokens as two 16-token sub-tiles, so a decay reference inside
                           the chunk keeps every factor within float32 range; f32: 16); the chunkwise
                           form (section 2.5) gives the same result for any chunk length in exact
                           arithmetic, so a request for 64 is served by that blocking.  Other values
                           are KDA_ERR_UNSUPPORTED. */
    kda_dtype io_dtype; /* dtype of q, k, v */
    kda_dtype o_dtype;  /* dtype of o: io_dtype, or KDA_F32 with bf16 inputs (diagnostic output) */
    float scale;        /* o_t = S_t^T (scale * q_t); 1.0 reads the state with q as given */
    int flags;          /* KDA_FWD_PRECISE and/or KDA_VALIDATE (kda_fwd only); other bits are reserved
                           and must be 0 */
} kda_fwd_desc;

/* kda_fwd_desc.flags: bf16 I/O only (the f32 path computes in float32 throughout and ignores it).
 * Forms the intra-chunk key Gram matrix L with split-bf16 key operands instead of single bf16 ones
 * (every other product of the bf16 path is split-bf16 already).  Worth it when keys within a chunk
 * are strongly correlated (e.g. after a Swish activation), which makes I + Diag(beta) L
 * ill-conditioned and amplifies the rounding of L in o and S_T; costs a few percent of throughput. */
#define KDA_FWD_PRECISE 1

/* kda_fwd_desc.flags, kda_fwd only: check the inputs before computing (a debug mode).  A device
 * pass scans g for values outside the section 3.2 bound [-5, 0] (NaN included; the kernels rely on
 * the bound to keep their decay factors finite) and q, k, v, beta and S0 for non-finite values;
 * any finding makes kda_fwd return KDA_ERR_INVALID_ARG without launching the forward.  The pass
 * writes one flag word into the workspace (kda_fwd_workspace_size gives its size) and
 * synchronises `stream` to read it, so this mode is not asynchronous and cannot be captured into a
 * graph. */
#define KDA_VALIDATE 2

/*
 * kda_fwd -- forward pass of the gated delta rule over B*H independent sequences.
 *
 *   q, k   : [B, T, H, Dk]  io_dtype   (q, k are usually L2-normalised per head; not required)
 *   v      : [B, T, H, Dv]  io_dtype
 *   g      : [B, T, H, Dk]  float32    log(alpha); precondition -5 <= g <= 0 (section 3.2 bound).
 *                                      Values outside the bound can overflow intermediate factors.
 *   beta   : [B, T, H]      float32    write strength, usually in (0, 1)
 *   S0     : [B, H, Dk, Dv] float32    initial state (rows = key channels), or NULL for zeros
 *   o      : [B, T, H, Dv]  o_dtype    output; on the bf16 path NULL computes the state alone (a
 *                                      leaner kernel that skips the readout: to fill a prefix cache,
 *                                      section 13.9); then S_T must be given
 *   S_T    : [B, H, Dk, Dv] float32    final state, or NULL to skip it; may equal S0
 *   ws     : device workspace of at least kda_fwd_workspace_size(desc) bytes, 256-byte aligned; NULL
 *            when that size is 0 (the plain forward needs none); contents are scratch
 *
 * Pointer alignment: q, k, v, o 4-byte aligned; g, beta, S0, S_T 8-byte aligned.
 * bf16 path numerics: matrix-core products on bf16 operands with float32 accumulation, split-bf16
 * (hi + lo, three products) wherever a value-path or state operand enters, and a float32 state.
 * The value path works on the state scaled by exact powers of two, so the result does not depend
 * on the magnitude of v and S0: it holds its accuracy while the state entries and |v| stay within
 * 2^-75 <= |x| < 2^60 (entries below 2^-75 count as 0 against the rest).  Within a chunk the
 * decay factors are taken relative to its middle token, so with g >= -5 they stay within
 * [e^-80, e^80] and q, k of ordinary magnitude (e.g. L2-normalised) keep every key-side operand
 * normal.
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE or KDA_ERR_HIP.
 */
size_t kda_fwd_workspace_size(const kda_fwd_desc* desc);  /* 256 with KDA_VALIDATE, else 0 (NULL desc: 0) */
kda_status kda_fwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* S0,
                   void* o, float* S_T, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kda_fwd_ckpt -- kda_fwd that also records the state at regular token boundaries: the KDA half of
 * the prefix cache of the explainer page, section 13.9, where a cached prefix can be resumed only
 * at a boundary that holds a state checkpoint (the page places them every 512 tokens, its hash-block
 * size).
 *   every  : tokens between checkpoints; a positive multiple of the chunk (32 for bf16 I/O, 16 for
 *            float32 I/O)
 *   S_ckpt : [B, H, n_ckpt, Dk, Dv] float32 with n_ckpt = T / every (rounded down).  Entry m of
 *            sequence (b, h) is the state after its tokens [0, (m+1)*every): the S0 that resumes the
 *            sequence at token (m+1)*every.  Resuming there with kda_fwd reproduces the remaining
 *            outputs and S_T of the uninterrupted call bit for bit.  May be NULL only when n_ckpt = 0;
 *            must not alias any other argument; 8-byte aligned.
 * o may be NULL on the bf16 path, as for kda_fwd (then S_T or a checkpoint must be written): the
 * states alone, the cheap way to fill a prefix cache.
 * Every other argument and the return codes are those of kda_fwd.
 */
kda_status kda_fwd_ckpt(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* S0,
                        void* o, float* S_T, float* S_ckpt, int every, hipStream_t stream);

/*
 * kda_decode -- the same operation as kda_fwd, evaluated token by token (no chunking): the decode
 * step of the explainer page, section 13.10 (state update and readout of each newly generated
 * token; the projections around it are the caller's).  For a few tokens per call; its cost is one
 * read and one write of the float32 state per call, plus O(T * Dk * Dv) arithmetic.
 *   desc   : as kda_fwd, with chunk = 0 (anything else is KDA_ERR_INVALID_ARG) and Dk = Dv in
 *            {64, 128} for both io_dtypes; flags as kda_fwd (KDA_FWD_PRECISE has no effect here).
 *   tensors: layouts, dtypes and alignment as kda_fwd; S_T may equal S0 (the usual in-place decode
 *            update: each thread reads its state entries before writing the same entries).
 * Arithmetic is float32 throughout (bf16 inputs are widened exactly, a bf16 o is rounded once).
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP.
 */
kda_status kda_decode(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* S0,
                      void* o, float* S_T, hipStream_t stream);

/*
 * kda_fwd_cp -- kda_fwd for few, long sequences: in-device context parallelism (explainer page,
 * section 13.3.1, with the decomposition of section 13.3.2: the state after a segment is its
 * accumulated transition M_i times its initial state plus its local state estimate S_hat_i).
 * Each sequence is cut into nseg segments that run side by side: one pass gives every S_hat_i (from
 * S = 0) and every M_i (v = 0 from S = I), a float32 scan over segments gives every initial state,
 * and a last pass from those states writes o and S_T.  About three times the work of kda_fwd spread
 * over nseg times more workgroups: it pays when 2*B*H is well below the 256 compute units (e.g.
 * B = 1, H = 16 at a million tokens, or B = 2, H = 16 at 8192 tokens).
 *   desc    : as kda_fwd, bf16 I/O only (Dk = Dv = 128; float32 I/O is KDA_ERR_UNSUPPORTED)
 *   nseg    : segments per sequence; 0 = automatic (the count of least modelled time among those
 *             with segments of at least 1024 tokens; 1 when none pays), 1 = kda_fwd.  T need not
 *             be a multiple of anything: the first nseg - 1 segments hold floor(T / (32 nseg))
 *             chunks of 32 tokens each and the last one the rest (nseg larger than T / 32 runs
 *             kda_fwd).
 *   ws      : device workspace of at least kda_fwd_cp_workspace_size(desc, nseg) bytes, 256-byte
 *             aligned (may be NULL when that size is 0); its contents are scratch.
 * Other arguments as kda_fwd (S_T may equal S0).  The result matches kda_fwd to within the bf16
 * path's rounding, not bit for bit (the segments start from scanned states).
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE or KDA_ERR_HIP.
 */
size_t kda_fwd_cp_workspace_size(const kda_fwd_desc* desc, int nseg);  /* 0 if none is needed or desc is invalid */
kda_status kda_fwd_cp(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* S0,
                      void* o, float* S_T, int nseg, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kda_fwd_cp_noalloc -- kda_fwd_cp for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace argument and
 * no allocation.  The segment states live in a fixed array of KDA_CP_NOALLOC_SCRATCH_BYTES per
 * device, part of the library's code object, held from the library's first use on a device until
 * the process ends; its device address is looked up once per device (hipGetSymbolAddress) on the
 * first call made with that device current.
 *   desc, tensors, nseg : as kda_fwd_cp.  The caller still owns and passes every input and output.
 * A problem whose plan needs more than kda_fwd_cp_workspace_size(desc, nseg) <=
 * KDA_CP_NOALLOC_SCRATCH_BYTES (about 170 segment-heads: e.g. B = 1, H = 16 with 8 segments needs
 * 24 MiB) returns KDA_ERR_SCRATCH_LIMIT before anything is launched.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (different streams, or different
 * host threads without ordering) race on it and give wrong results; calls ordered on one stream are
 * safe.  Nothing in the array needs to start at zero.  The result is bit for bit that of kda_fwd_cp
 * with the same arguments.
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_SCRATCH_LIMIT or KDA_ERR_HIP.
 */
#define KDA_CP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
kda_status kda_fwd_cp_noalloc(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* S0,
                              void* o, float* S_T, int nseg, hipStream_t stream);

/*
 * kda_bwd -- gradients of kda_fwd (training; the explainer page's P3 section 5.1 says FlashKDA covers
 * training, and the pages give no backward formulas: these are reverse-mode through the chunkwise
 * form of section 2.5).  Same desc and inputs as the forward call; given the gradients of a loss
 * with respect to o and S_T it returns those with respect to every input.
 *   dO     : [B, T, H, Dv] o_dtype   dL/do, or NULL for zero
 *   dS_T   : [B, H, Dk, Dv] float32  dL/dS_T, or NULL for zero
 *   dq, dk, dg : [B, T, H, Dk] float32;  dv : [B, T, H, Dv] float32;  dbeta : [B, T, H] float32;
 *   dS0    : [B, H, Dk, Dv] float32 (the gradient for S0, or for a zero initial state when S0 is NULL)
 *            Each output may be NULL (not computed); outputs must not alias inputs or each other.
 *   ws     : device workspace of at least kda_bwd_workspace_size(desc) bytes, 256-byte aligned:
 *            the forward state and the state gradient at every 32-token (bf16 inputs) or 16-token
 *            (float32 inputs) boundary, 2 * B * H * ceil(T / interval) * Dk * Dv floats.
 *   desc   : chunk must be 0; bf16 I/O needs Dk = Dv = 128, float32 I/O Dk = Dv in {64, 128};
 *            KDA_FWD_PRECISE is implied for the state recompute of bf16 inputs.
 * Arithmetic is float32 (bf16 inputs and dO are widened exactly; the recomputed states carry the
 * forward path's rounding).  Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED,
 * KDA_ERR_WORKSPACE or KDA_ERR_HIP.
 */
size_t kda_bwd_workspace_size(const kda_fwd_desc* desc);  /* 0 for an invalid descriptor */
kda_status kda_bwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* S0,
                   const void* dO, const float* dS_T,
                   float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------------------------
 * Fused layer forward.  The layer of the explainer page "Kimi K3：开放前沿智能":
 *   section 2.4 (paper Eq. 2): q, k = L2norm(Swish(ShortConv(x W))); v = x W_v;
 *   section 2.3 (paper Eq. 2): decay logit z = W_up W_down x + b_alpha (low rank);
 *   section 3.2 (paper Eq. 5): log(alpha) = -5 * sigmoid(exp(A_h) * z), A per head;
 *   beta = sigmoid(x W_beta) (not on the page: the plainest reading);
 *   the gated delta rule above (kda_fwd's matrix-core path on float32 q, k, v with KDA_FWD_PRECISE,
 *   float32 output);
 *   section 3.3 (paper Eq. 6): per-head RMSNorm of o, times the full-rank data-dependent gate
 *   sigmoid(x W_g); then the output projection W_o.
 * Short convolution: causal, depthwise, 4 taps, no bias; tap 3 multiplies the current token.
 * L2 norm: x / sqrt(sum x^2 + 1e-6); RMSNorm: x / sqrt(mean x^2 + 1e-6) * rms_w.
 * --------------------------------------------------------------------------------------------- */
typedef struct {
    int B, T;           /* batch, tokens (T >= 1) */
    int d_model;        /* width of x and y (multiple of 32; other widths are KDA_ERR_UNSUPPORTED) */
    int H, Dk, Dv;      /* heads; Dk = Dv = 128 */
    int rank;           /* rank of the decay projection W_down W_up (multiple of 16) */
    int conv;           /* short-convolution taps; 4 */
    float scale;        /* multiplies q in the readout; 1.0 for the plain readout */
    int flags;          /* reserved, must be 0 */
} kda_layer_desc;

/* Layer parameters, all DEVICE pointers owned by the caller.  Matrices are row-major [in, out],
 * so a projection is x @ W. */
typedef struct {
    const void* Wq;       /* [d_model, H*Dk] bf16 */
    const void* Wk;       /* [d_model, H*Dk] bf16 */
    const void* Wv;       /* [d_model, H*Dv] bf16 */
    const void* Wg;       /* [d_model, H*Dv] bf16  output gate */
    const void* Wo;       /* [H*Dv, d_model] bf16  output projection */
    const void* Wbeta;    /* [d_model, H]    bf16 */
    const void* Wdown;    /* [d_model, rank] bf16 */
    const void* Wup;      /* [rank, H*Dk]    bf16 */
    const float* conv_q;  /* [H*Dk, conv] float32 */
    const float* conv_k;  /* [H*Dk, conv] float32 */
    const float* b_alpha; /* [H*Dk] float32 */
    const float* A;       /* [H] float32 */
    const float* rms_w;   /* [Dv] float32 */
} kda_layer_weights;

/* Bytes of device workspace kda_layer_fwd needs for this problem (0 for an invalid descriptor). */
size_t kda_layer_workspace_size(const kda_layer_desc* desc);

/*
 * kda_layer_fwd -- y = layer(x).
 *   x              : [B, T, d_model] bf16, 16-byte aligned
 *   S0, S_T        : [B, H, Dk, Dv] float32 KDA state in / out (NULL: zeros / not written; may alias)
 *   conv_state_in  : [B, 3, 2*H*Dk] float32, the last 3 pre-convolution q rows then k rows of the
 *                    previous segment, oldest first (NULL: zeros)
 *   conv_state_out : same layout for this segment's end (NULL: not written); must not alias the input
 *   y              : [B, T, d_model] bf16, 16-byte aligned
 *   ws             : device workspace of at least kda_layer_workspace_size(desc) bytes, 256-byte aligned
 * The projections run on the library's bf16 matrix-core GEMM with float32 sums: one product over
 * the concatenated q, k, v, gate, decay-down and beta weights; the rank-R up-projection over the
 * hi and lo bf16 halves of the float32 down-projection (about 16 significant bits), with the decay
 * gate applied in its epilogue; the output projection.  The weights are transposed into the
 * workspace on each call.  Nothing is allocated and no state is kept between calls.
 * Returns KDA_OK, KDA_ERR_INVALID_ARG (also for a misaligned x or y), KDA_ERR_UNSUPPORTED,
 * KDA_ERR_WORKSPACE or KDA_ERR_HIP.
 */
kda_status kda_layer_fwd(const kda_layer_desc* desc, const void* x, const kda_layer_weights* weights,
                         const float* S0, const float* conv_state_in, void* y, float* S_T,
                         float* conv_state_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kda_layer_decode -- the layer (as kda_layer_fwd) over T new tokens of each of B sequences, from a
 * given state and convolution window: the decode step of the explainer page, section 13.10 (one fused
 * call for the projections, the state update and the readout, with a projection-input cache), with
 * the speculative-decoding rollback of section 13.4 (the state is updated in place, so rejected draft
 * tokens cannot be undone from it; each token's projection inputs are cached instead, far fewer
 * numbers than a state).  Four stream-ordered launches: the input projections (bf16 matrix-core
 * products of the weights as given, float32 sums), one workgroup per (sequence, head) for the gates,
 * convolution, recurrence and readout, the output projection (the float32 gated rows as bf16 hi + lo
 * halves), its sum.
 *   desc          : as kda_layer_fwd, with d_model a multiple of 4, rank <= 128, B*T <= 16 rows (else
 *                   KDA_ERR_UNSUPPORTED); flags = 0 or KDA_DECODE_SPECULATIVE
 *   x             : [B, T, d_model] bf16;  y: [B, T, d_model] bf16 (output); both 16-byte aligned
 *   S             : [B, H, Dk, Dv] float32 state (required).  Read, then overwritten with the state
 *                   after the T tokens -- unless KDA_DECODE_SPECULATIVE, which leaves it unchanged
 *   conv_state    : [B, 3, 2*H*Dk] float32 window as kda_layer_fwd (NULL: zeros, not written); updated
 *                   like S
 *   cache         : the tokens' cache entries (kda_layer_decode_cache_bytes(desc) bytes, float32, planar
 *                   with N = B*T token rows in [b][t] order: k [N][H*Dk] after conv/SiLU/L2, v [N][H*Dv],
 *                   g (log decay) [N][H*Dk], beta [N][H], pre-convolution q rows [N][H*Dk], pre-convolution
 *                   k rows [N][H*Dk]); required with KDA_DECODE_SPECULATIVE, else may be NULL
 *   ws            : device workspace of kda_layer_decode_workspace_size(desc) bytes, 256-byte aligned
 * With KDA_DECODE_SPECULATIVE the T tokens are drafts: token t's output is computed as if drafts
 * 0..t-1 were accepted.  Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE or
 * KDA_ERR_HIP.
 */
#define KDA_DECODE_SPECULATIVE 1
size_t kda_layer_decode_workspace_size(const kda_layer_desc* desc);  /* 0 for an invalid descriptor */
size_t kda_layer_decode_cache_bytes(const kda_layer_desc* desc);      /* 0 for an invalid descriptor */
kda_status kda_layer_decode(const kda_layer_desc* desc, const void* x, const kda_layer_weights* weights,
                            float* S, float* conv_state, void* y, float* cache, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * kda_layer_decode_commit -- accept the first n_accept (0 <= n_accept <= desc->T) tokens of each
 * sequence of a speculative kda_layer_decode call: advances S (in place) and conv_state (if not NULL)
 * over their cache entries with the token-by-token step, without the projections (section 13.4's
 * rollback: the rejected drafts never touched S).  desc is the speculative call's (its flags are
 * ignored).  Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP.
 */
kda_status kda_layer_decode_commit(const kda_layer_desc* desc, const float* cache, int n_accept, float* S,
                                   float* conv_state, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_error_string(kda_status status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
