/*
 * KDA prefill oracle: the gated delta rule, token by token, in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the package's smoke() entry and the
 * bench's cpu_baseline leg may load this library.  It shares no code with the
 * HIP path and never runs on the GPU.
 *
 * What it computes (the reading taken of the pages): Kimi Delta Attention, the
 * gated delta-rule recurrence that the TensorRT-LLM KDA prefill kernel
 * (PR #19826) and the cudnn-frontend Hopper KDA prefill (PR #1056) implement.
 * The pages name the method but never print its equations; this oracle reads it
 * as, for every sequence n and head h independently, over the sequence's tokens
 * t in order,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with S a d_k x d_v matrix (row = key channel), S_{-1} the initial state
 * (zeros when none is given), and the final state S after the last token.
 * Decay is applied first, the delta correction is taken against the decayed
 * state, and the output reads the updated state.  The cudnn-frontend PR checks
 * its kernel against a float64 oracle run at the production gate bound with a
 * non-zero initial state (Correctness section); this file is such an oracle.
 *
 * The update is written as the equivalent rank-one form
 *     S <- D S;  r = k^T S;  S <- S + beta k (v - r)^T
 * which is (I - beta k k^T) D S + beta k v^T expanded.
 *
 * Layout: packed tokens, q/k/g [T, H, DK], v/o [T, H, DV], beta [T, H],
 * states [N, H, DK, DV], all contiguous float64.  cu[n]..cu[n+1] are the tokens
 * of sequence n.  Cost: about 7*DK*DV flops per token-head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void run_chain(int64_t t_begin, int64_t t_end, int64_t h, int64_t H, int64_t DK, int64_t DV,
                      const double *q, const double *k, const double *v, const double *g,
                      const double *beta, const double *s0, double *o, double *sT, double *S,
                      double *r)
{
    if (s0)
        memcpy(S, s0, sizeof(double) * DK * DV);
    else
        memset(S, 0, sizeof(double) * DK * DV);

    for (int64_t t = t_begin; t < t_end; ++t) {
        const double *qt = q + (t * H + h) * DK;
        const double *kt = k + (t * H + h) * DK;
        const double *gt = g + (t * H + h) * DK;
        const double *vt = v + (t * H + h) * DV;
        const double bt = beta[t * H + h];

        /* S <- Diag(exp g_t) S : row i of S is key channel i */
        for (int64_t i = 0; i < DK; ++i) {
            const double e = exp(gt[i]);
            for (int64_t j = 0; j < DV; ++j)
                S[i * DV + j] *= e;
        }
        /* r = k_t^T (D S) */
        for (int64_t j = 0; j < DV; ++j)
            r[j] = 0.0;
        for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j)
                r[j] += kt[i] * S[i * DV + j];
        /* S <- S + beta k (v - r)^T */
        for (int64_t i = 0; i < DK; ++i) {
            const double bk = bt * kt[i];
            for (int64_t j = 0; j < DV; ++j)
                S[i * DV + j] += bk * (vt[j] - r[j]);
        }
        /* o_t = S_t^T q_t */
        double *ot = o + (t * H + h) * DV;
        for (int64_t j = 0; j < DV; ++j)
            ot[j] = 0.0;
        for (int64_t i = 0; i < DK; ++i)
            for (int64_t j = 0; j < DV; ++j)
                ot[j] += qt[i] * S[i * DV + j];
    }
    if (sT)
        memcpy(sT, S, sizeof(double) * DK * DV);
}

/* Returns 0 on success, 1 on a bad argument, 2 on allocation failure.
 * n_threads <= 0 keeps the OpenMP default.  Returns the thread count used
 * through *threads_used when that pointer is not NULL. */
int kda_oracle_f64(int64_t n_seq, int64_t H, int64_t DK, int64_t DV, const int64_t *cu,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const double *s0, double *o, double *sT, int n_threads,
                   int *threads_used)
{
    if (n_seq < 0 || H <= 0 || DK <= 0 || DV <= 0 || !cu)
        return 1;
    for (int64_t n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n])
            return 1;
    int failed = 0;
    int used = 1;
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#endif
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *S = (double *)malloc(sizeof(double) * DK * DV);
        double *r = (double *)malloc(sizeof(double) * DV);
        if (!S || !r) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t c = 0; c < n_seq * H; ++c) {
            if (!S || !r)
                continue;
            const int64_t n = c / H, h = c % H;
            run_chain(cu[n], cu[n + 1], h, H, DK, DV, q, k, v, g, beta,
                      s0 ? s0 + (n * H + h) * DK * DV : NULL, o,
                      sT ? sT + (n * H + h) * DK * DV : NULL, S, r);
        }
        free(S);
        free(r);
    }
    if (threads_used)
        *threads_used = used;
    return failed ? 2 : 0;
}
