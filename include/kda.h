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
 *     The library allocates no device memory in kda_fwd.
 *   - Calls are asynchronous and ordered on `stream` (NULL = the default stream).  The return code
 *     covers argument validation and launch errors only; a fault inside a kernel surfaces at the
 *     caller's next synchronisation.
 *   - Tensors are dense, row-major, without padding, in the layouts given per argument.
 *   - No global mutable state: calls from several host threads are safe.
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
    KDA_ERR_WORKSPACE = -4     /* workspace pointer missing or smaller than the size query said */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Problem description for kda_fwd. */
typedef struct {
    int B, T, H;        /* batch, tokens, heads; B, H >= 1, T >= 0 */
    int Dk, Dv;         /* key / value head size.  bf16 I/O: Dk = Dv = 128.  f32 I/O: Dk = Dv in {64, 128} */
    int chunk;          /* tokens per chunk of the chunkwise form; 0 = library default.
                           Supported: 32 for bf16 I/O (two 16-token sub-tiles), 16 for f32 I/O. */
    kda_dtype io_dtype; /* dtype of q, k, v */
    kda_dtype o_dtype;  /* dtype of o: io_dtype, or KDA_F32 with bf16 inputs (diagnostic output) */
    float scale;        /* o_t = S_t^T (scale * q_t); 1.0 reads the state with q as given */
    int flags;          /* reserved, must be 0 */
} kda_fwd_desc;

/*
 * kda_fwd -- forward pass of the gated delta rule over B*H independent sequences.
 *
 *   q, k   : [B, T, H, Dk]  io_dtype   (q, k are usually L2-normalised per head; not required)
 *   v      : [B, T, H, Dv]  io_dtype
 *   g      : [B, T, H, Dk]  float32    log(alpha); precondition -5 <= g <= 0 (section 3.2 bound).
 *                                      Values outside the bound can overflow intermediate factors.
 *   beta   : [B, T, H]      float32    write strength, usually in (0, 1)
 *   S0     : [B, H, Dk, Dv] float32    initial state (rows = key channels), or NULL for zeros
 *   o      : [B, T, H, Dv]  o_dtype    output
 *   S_T    : [B, H, Dk, Dv] float32    final state, or NULL to skip it; may equal S0
 *
 * Pointer alignment: q, k, v, o 4-byte aligned; g, beta, S0, S_T 8-byte aligned.
 * bf16 path numerics: intermediate products use bf16/f16 matrix-core operands with float32
 * accumulation (split-bf16 where a single rounding is too coarse); the state is float32.
 * The value path uses f16 operands, so |v| and the state entries must stay below 6.5e4;
 * beyond that o and S_T become non-finite.
 * Returns KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED or KDA_ERR_HIP.
 */
kda_status kda_fwd(const kda_fwd_desc* desc, const void* q, const void* k, const void* v,
                   const float* g, const float* beta, const float* S0,
                   void* o, float* S_T, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* kda_error_string(kda_status status);

/* Library version as major*10000 + minor*100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
