/*
 * CPU oracle for the Kimi Delta Attention (KDA) forward pass -- TEST
 * INFRASTRUCTURE ONLY.  Nothing in the product path links or calls this file;
 * only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * What it computes: the token-by-token gated delta rule in float64, one
 * (batch, head) pair at a time, as the recurrence is described on the explainer
 * page "Kimi K3：开放前沿智能" (kimi-k3-paper.pages.dev), section 2.2 (paper
 * Eq. 1, whose formula the page text lost; its two terms are described there)
 * and section 2.4 (readout):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T (scale * q_t)          (read after the update, section 2.4)
 *
 * with alpha_t = exp(g_t) per key channel (section 2.3: one forget rate per
 * channel, in (0,1)).  Section 2.2 orders the first term as decay first, then
 * erase: the state is first scaled per key channel by alpha_t, then the part
 * of it that overlaps k_t is removed and beta_t k_t v_t^T is written.  Written
 * out for one token:
 *
 *     S  <- Diag(alpha_t) S
 *     w  <- S^T k_t                       (what the state holds along k_t)
 *     S  <- S + beta_t k_t (v_t - w)^T    (= (I - beta k k^T) S + beta k v^T)
 *     o_t <- S^T (scale q_t)
 *
 * Layouts (row-major, contiguous):
 *   q, k, g : [B, T, H, Dk]      v : [B, T, H, Dv]      beta : [B, T, H]
 *   S0, S_T : [B, H, Dk, Dv]     o : [B, T, H, Dv]
 * Inputs are float32 (in_f64 == 0) or float64 (in_f64 != 0); the arithmetic
 * and the outputs are float64.  S0 == NULL means a zero initial state;
 * o == NULL or S_T == NULL skips that output.  Returns 0, or -1 on bad sizes.
 *
 * Parity status: pinned (closed forms, invariants, the chunkwise form and a
 * hand-worked example in the test suite).
 */
#include <stdlib.h>
#include <string.h>
#include <math.h>

static inline double ld(const void* p, size_t i, int f64) {
    return f64 ? ((const double*)p)[i] : (double)((const float*)p)[i];
}

int kda_oracle_recurrence(int B, int T, int H, int Dk, int Dv, int in_f64,
                          const void* q, const void* k, const void* v,
                          const void* g, const void* beta, const double* S0,
                          double scale, double* o, double* S_T, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (nthreads < 1) nthreads = 1;
    const long nbh = (long)B * H;
    int bad = 0;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const long b = bh / H, h = bh % H;
        double* S = (double*)malloc(sizeof(double) * (size_t)Dk * Dv);
        double* kt = (double*)malloc(sizeof(double) * (size_t)(3 * Dk + 2 * Dv));
        if (!S || !kt) { free(S); free(kt);
#pragma omp atomic write
            bad = 1;
            continue; }
        double* qt = kt + Dk;
        double* at = qt + Dk;
        double* vt = at + Dk;
        double* w = vt + Dv;

        if (S0) memcpy(S, S0 + bh * (size_t)Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);

        for (long t = 0; t < T; ++t) {
            const size_t row = (size_t)((b * T + t) * H + h);
            for (int i = 0; i < Dk; ++i) {
                kt[i] = ld(k, row * Dk + i, in_f64);
                qt[i] = scale * ld(q, row * Dk + i, in_f64);
                at[i] = exp(ld(g, row * Dk + i, in_f64));
            }
            for (int j = 0; j < Dv; ++j) vt[j] = ld(v, row * Dv + j, in_f64);
            const double bt = ld(beta, row, in_f64);

            /* decay each key channel (row i of S) by alpha_t[i] */
            for (int i = 0; i < Dk; ++i) {
                double* Si = S + (size_t)i * Dv;
                for (int j = 0; j < Dv; ++j) Si[j] *= at[i];
            }
            /* w = S^T k_t */
            for (int j = 0; j < Dv; ++j) w[j] = 0.0;
            for (int i = 0; i < Dk; ++i) {
                const double* Si = S + (size_t)i * Dv;
                for (int j = 0; j < Dv; ++j) w[j] += Si[j] * kt[i];
            }
            /* S += beta k (v - w)^T */
            for (int j = 0; j < Dv; ++j) w[j] = vt[j] - w[j];
            for (int i = 0; i < Dk; ++i) {
                double* Si = S + (size_t)i * Dv;
                const double c = bt * kt[i];
                for (int j = 0; j < Dv; ++j) Si[j] += c * w[j];
            }
            /* o_t = S^T (scale q_t) */
            if (o) {
                double* ot = o + row * Dv;
                for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
                for (int i = 0; i < Dk; ++i) {
                    const double* Si = S + (size_t)i * Dv;
                    for (int j = 0; j < Dv; ++j) ot[j] += Si[j] * qt[i];
                }
            }
        }
        if (S_T) memcpy(S_T + bh * (size_t)Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        free(S);
        free(kt);
    }
    return bad ? -1 : 0;
}

/*
 * Backward pass of the same recurrence (float64), by reverse-mode differentiation of the token
 * steps above.  Given the output gradients dO = dL/do [B,T,H,Dv] and dS_T = dL/dS_T [B,H,Dk,Dv]
 * (either may be NULL = zero), it returns dL/dq, dL/dk, dL/dg [B,T,H,Dk], dL/dv [B,T,H,Dv],
 * dL/dbeta [B,T,H] and dL/dS0 [B,H,Dk,Dv] (NULL outputs are skipped), in float64.
 *
 * With the per-token quantities of the forward step
 *     St = Diag(alpha) S_prev,  w = St^T k,  u = beta (v - w),  S = St + k u^T,  o = S^T (scale q),
 * and dS = dL/dS (after this token, including what later tokens send back), one token backwards is
 *     dS  += scale q dO^T                      (readout)
 *     dq   = scale S dO
 *     du   = dS^T k;   dv = beta du;   dbeta = du . (v - w);   dw = -beta du
 *     dk   = dS u + St dw
 *     dSt  = dS + k dw^T
 *     dg_i = sum_j dSt_ij St_ij                (alpha = exp(g): d alpha_i / d g_i = alpha_i)
 *     dS_prev = Diag(alpha) dSt
 * The states S_prev are rebuilt block by block (64 tokens) from states kept at block starts.
 * Returns 0, or -1 on bad sizes or allocation failure.
 */
#define KDA_ORACLE_BLOCK 64

int kda_oracle_backward(int B, int T, int H, int Dk, int Dv, int in_f64,
                        const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const double* S0, double scale,
                        const double* dO, const double* dST,
                        double* dq, double* dk, double* dv, double* dg, double* dbeta, double* dS0,
                        int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return -1;
    if (nthreads < 1) nthreads = 1;
    const long nbh = (long)B * H;
    const size_t SS = (size_t)Dk * Dv;
    const long nblk = (T + KDA_ORACLE_BLOCK - 1) / KDA_ORACLE_BLOCK;
    int bad = 0;

#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1)
    for (long bh = 0; bh < nbh; ++bh) {
        const long b = bh / H, h = bh % H;
        double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nblk > 0 ? nblk : 1));  /* S before each block */
        double* blk = (double*)malloc(sizeof(double) * SS * KDA_ORACLE_BLOCK);                  /* S before each token */
        double* S = (double*)malloc(sizeof(double) * SS);
        double* St = (double*)malloc(sizeof(double) * SS);
        double* dS = (double*)malloc(sizeof(double) * SS);
        double* vec = (double*)malloc(sizeof(double) * (size_t)(4 * Dk + 5 * Dv));
        if (!ck || !blk || !S || !St || !dS || !vec) {
            free(ck); free(blk); free(S); free(St); free(dS); free(vec);
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double *kt = vec, *qt = kt + Dk, *at = qt + Dk, *tmpk = at + Dk;
        double *vt = tmpk + Dk, *w = vt + Dv, *u = w + Dv, *du = u + Dv, *dot = du + Dv;

        /* forward sweep: the state entering every block */
        if (S0) memcpy(S, S0 + bh * SS, sizeof(double) * SS);
        else memset(S, 0, sizeof(double) * SS);
        for (long t = 0; t < T; ++t) {
            if (t % KDA_ORACLE_BLOCK == 0) memcpy(ck + (t / KDA_ORACLE_BLOCK) * SS, S, sizeof(double) * SS);
            const size_t row = (size_t)((b * T + t) * H + h);
            for (int i = 0; i < Dk; ++i) { kt[i] = ld(k, row * Dk + i, in_f64); at[i] = exp(ld(g, row * Dk + i, in_f64)); }
            for (int j = 0; j < Dv; ++j) vt[j] = ld(v, row * Dv + j, in_f64);
            const double bt = ld(beta, row, in_f64);
            for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= at[i];
            for (int j = 0; j < Dv; ++j) w[j] = 0.0;
            for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) w[j] += S[(size_t)i * Dv + j] * kt[i];
            for (int j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - w[j]);
            for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += kt[i] * u[j];
        }

        /* reverse sweep */
        if (dST) memcpy(dS, dST + bh * SS, sizeof(double) * SS);
        else memset(dS, 0, sizeof(double) * SS);
        for (long bi = nblk - 1; bi >= 0; --bi) {
            const long t0 = bi * KDA_ORACLE_BLOCK;
            const long t1 = (t0 + KDA_ORACLE_BLOCK < T) ? t0 + KDA_ORACLE_BLOCK : T;
            /* rebuild the states before each token of the block */
            memcpy(S, ck + bi * SS, sizeof(double) * SS);
            for (long t = t0; t < t1; ++t) {
                memcpy(blk + (t - t0) * SS, S, sizeof(double) * SS);
                const size_t row = (size_t)((b * T + t) * H + h);
                for (int i = 0; i < Dk; ++i) { kt[i] = ld(k, row * Dk + i, in_f64); at[i] = exp(ld(g, row * Dk + i, in_f64)); }
                for (int j = 0; j < Dv; ++j) vt[j] = ld(v, row * Dv + j, in_f64);
                const double bt = ld(beta, row, in_f64);
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= at[i];
                for (int j = 0; j < Dv; ++j) w[j] = 0.0;
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) w[j] += S[(size_t)i * Dv + j] * kt[i];
                for (int j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - w[j]);
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += kt[i] * u[j];
            }
            for (long t = t1 - 1; t >= t0; --t) {
                const size_t row = (size_t)((b * T + t) * H + h);
                const double* Sp = blk + (t - t0) * SS;
                for (int i = 0; i < Dk; ++i) {
                    kt[i] = ld(k, row * Dk + i, in_f64);
                    qt[i] = scale * ld(q, row * Dk + i, in_f64);
                    at[i] = exp(ld(g, row * Dk + i, in_f64));
                }
                for (int j = 0; j < Dv; ++j) { vt[j] = ld(v, row * Dv + j, in_f64); dot[j] = dO ? dO[row * Dv + j] : 0.0; }
                const double bt = ld(beta, row, in_f64);
                /* this token's forward quantities */
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) St[(size_t)i * Dv + j] = at[i] * Sp[(size_t)i * Dv + j];
                for (int j = 0; j < Dv; ++j) w[j] = 0.0;
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) w[j] += St[(size_t)i * Dv + j] * kt[i];
                for (int j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - w[j]);
                /* readout: dS += scale q dO^T; dq = scale S dO with S = St + k u^T */
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) dS[(size_t)i * Dv + j] += qt[i] * dot[j];
                if (dq) {
                    double* dqt = dq + row * Dk;
                    for (int i = 0; i < Dk; ++i) {
                        double a = 0.0;
                        for (int j = 0; j < Dv; ++j) a += (St[(size_t)i * Dv + j] + kt[i] * u[j]) * dot[j];
                        dqt[i] = scale * a;
                    }
                }
                /* du = dS^T k */
                for (int j = 0; j < Dv; ++j) du[j] = 0.0;
                for (int i = 0; i < Dk; ++i) for (int j = 0; j < Dv; ++j) du[j] += dS[(size_t)i * Dv + j] * kt[i];
                if (dv) for (int j = 0; j < Dv; ++j) dv[row * Dv + j] = bt * du[j];
                if (dbeta) {
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) a += du[j] * (vt[j] - w[j]);
                    dbeta[row] = a;
                }
                /* dw = -beta du (kept in du from here) */
                for (int j = 0; j < Dv; ++j) du[j] *= -bt;
                /* dk = dS u + St dw */
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) a += dS[(size_t)i * Dv + j] * u[j] + St[(size_t)i * Dv + j] * du[j];
                    tmpk[i] = a;
                }
                if (dk) for (int i = 0; i < Dk; ++i) dk[row * Dk + i] = tmpk[i];
                /* dSt = dS + k dw^T;  dg = rowsum(dSt * St);  dS_prev = Diag(alpha) dSt */
                for (int i = 0; i < Dk; ++i) {
                    double a = 0.0;
                    for (int j = 0; j < Dv; ++j) {
                        const double d = dS[(size_t)i * Dv + j] + kt[i] * du[j];
                        a += d * St[(size_t)i * Dv + j];
                        dS[(size_t)i * Dv + j] = at[i] * d;
                    }
                    if (dg) dg[row * Dk + i] = a;
                }
            }
        }
        if (dS0) memcpy(dS0 + bh * SS, dS, sizeof(double) * SS);
        free(ck); free(blk); free(S); free(St); free(dS); free(vec);
    }
    return bad ? -1 : 0;
}
