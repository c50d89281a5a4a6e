/* Plain C fp64 reference of the KDA recurrence -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package smoke check and the benchmark's CPU-baseline
 * leg load this library.  It shares no code with the GPU library.
 *
 * Recurrence ("Understanding Kimi Delta Attention", section "The KDA
 * Recurrence"; "kimi delta attn from first principles", sections "KDA" and
 * "three gates"), for one chain with state S (dk rows = key channels,
 * dv columns), per token:
 *   alpha = exp(g_t); S <- Diag(alpha) S; u = beta_t (v_t - S^T k_t);
 *   S <- S + k_t u^T; o_t = scale * S^T q_t.
 * Chains are independent; OpenMP runs them in parallel.  Inside a chain the
 * loops are the plain definition, in fp64, with no blocking or reordering.
 *
 * Inputs are row-major float arrays (bf16 inputs are widened exactly by the
 * caller).  Chain i reads rows start[i] .. start[i]+len[i]-1 of q/k/g
 * ([rows, dk]), v ([rows, dv]) and beta ([rows]); it writes the same rows of
 * o ([rows, dv], may be NULL) and s_final[i] ([dk, dv]).  h0 (fp64) is
 * [n_chains, dk, dv] or NULL for zeros.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int kda_ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void run_chain(int64_t start, int64_t len, int dk, int dv, double scale,
                      const float* q, const float* k, const float* v, const float* g,
                      const float* beta, const double* h0, double* o, double* S, double* u) {
    if (h0) {
        for (int64_t i = 0; i < (int64_t)dk * dv; ++i) S[i] = h0[i];
    } else {
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    }
    for (int64_t t = start; t < start + len; ++t) {
        const float* qt = q + t * dk;
        const float* kt = k + t * dk;
        const float* vt = v + t * dv;
        const float* gt = g + t * dk;
        double bt = (double)beta[t];
        /* step 1-2: decay every row c by its own gate */
        for (int c = 0; c < dk; ++c) {
            double a = exp((double)gt[c]);
            for (int j = 0; j < dv; ++j) S[c * dv + j] *= a;
        }
        /* step 3: u = beta (v - S^T k) on the decayed state */
        for (int j = 0; j < dv; ++j) u[j] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) u[j] += S[c * dv + j] * (double)kt[c];
        for (int j = 0; j < dv; ++j) u[j] = bt * ((double)vt[j] - u[j]);
        /* step 4: S <- S + k u^T */
        for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) S[c * dv + j] += (double)kt[c] * u[j];
        /* step 5: o = scale * S^T q */
        if (o) {
            double* ot = o + t * dv;
            for (int j = 0; j < dv; ++j) ot[j] = 0.0;
            for (int c = 0; c < dk; ++c)
                for (int j = 0; j < dv; ++j) ot[j] += S[c * dv + j] * (double)qt[c];
            for (int j = 0; j < dv; ++j) ot[j] *= scale;
        }
    }
}

/* Returns 0 on success, -1 on a bad argument or allocation failure.
 * The state of chain i evolves in place in s_final[i]. */
int kda_ref_chains(int n_chains, const int64_t* start, const int64_t* len, int dk, int dv,
                   double scale, const float* q, const float* k, const float* v, const float* g,
                   const float* beta, const double* h0, double* o, double* s_final, int n_threads) {
    if (n_chains < 0 || dk <= 0 || dv <= 0 || !start || !len || !s_final) return -1;
    int err = 0;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel
#endif
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!u) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int i = 0; i < n_chains; ++i) {
            if (!u) continue;
            run_chain(start[i], len[i], dk, dv, scale, q, k, v, g, beta,
                      h0 ? h0 + (size_t)i * dk * dv : NULL, o, s_final + (size_t)i * dk * dv, u);
        }
        free(u);
    }
    return err;
}
