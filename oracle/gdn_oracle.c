/*
 * gdn_oracle.c -- fp64 CPU oracle of the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * shares no code, header, table or helper with it, and never calls it.
 *
 * What it computes: the plain token-by-token recurrence, which is the
 * definition the chunkwise method reaches up to rounding order.
 *
 *   "RNN的复兴03:现代RNN的并行计算", section 1, equation (2): delta rule with
 *   separate erase strength beta_t and write strength eta_t,
 *       S_t = S_{t-1} (E - beta_t k_t k_t^T) + eta_t v_t k_t^T .
 *   "从零开始的 GDN 推导", recurrent form (first display under the notation
 *   section): the gate alpha_t multiplies the erased state, not the write,
 *       S_{t+1} = alpha_t (I - beta_t k_t^T k_t) S_t + beta_t k_t^T v_t
 *   (row-vector orientation; transposed here so that S is d_v x d_k).
 *   Output: "从零开始的 GDN 推导", section on O: o_t uses the state that has
 *   already absorbed token t (o_t = q_t S_{t+1}); equivalently o_t = S_t q_t
 *   with the 1-based index of the first page and the linear-RNN recurrence of
 *   the circuit-complexity page ("类 RNN 模型训练").
 *
 * Combined, with S of shape [d_v, d_k]:
 *     u   = S k_t                                   (d_v)
 *     S   = alpha_t (S - beta_t u k_t^T) + eta_t v_t k_t^T
 *     o_t = S q_t                                   (inclusive of token t)
 * eta defaults to beta (the gated delta rule); eta is only exposed so that the
 * special cases of the pages (linear attention, gated linear attention) can be
 * reached: erase strength 0 with write strength 1.
 *
 * Layouts (row-major, contiguous):
 *   q, k   [B, H, T, d_k]      v, O   [B, H, T, d_v]
 *   alpha, beta, eta  [B, H, T]
 *   S0, S_final       [B, H, d_v, d_k]
 * alpha == NULL means alpha = 1; eta == NULL means eta = beta;
 * S0 == NULL means a zero initial state.  O and S_final are written.
 * Each (b, h) sequence is independent; they are spread over OpenMP threads.
 *
 * Returns 0 on success, -1 on a bad argument (NULL required pointer or a
 * non-positive size); nothing is written in that case.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void run_one_sequence(int64_t T, int64_t dk, int64_t dv,
                             const double* q, const double* k, const double* v,
                             const double* alpha, const double* beta,
                             const double* eta, const double* S0,
                             double* O, double* S, double* u)
{
    /* S <- S0 (or zero) */
    if (S0) memmove(S, S0, (size_t)(dv * dk) * sizeof(double));
    else memset(S, 0, (size_t)(dv * dk) * sizeof(double));

    for (int64_t t = 0; t < T; ++t) {
        const double* kt = k + t * dk;
        const double* qt = q + t * dk;
        const double* vt = v + t * dv;
        double a = alpha ? alpha[t] : 1.0;
        double b = beta[t];
        double e = eta ? eta[t] : beta[t];
        /* u = S k_t */
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * kt[j];
            u[i] = acc;
        }
        /* S = a (S - b u k^T) + e v k^T */
        for (int64_t i = 0; i < dv; ++i) {
            for (int64_t j = 0; j < dk; ++j) {
                double s = S[i * dk + j];
                S[i * dk + j] = a * (s - b * u[i] * kt[j]) + e * vt[i] * kt[j];
            }
        }
        /* o_t = S q_t (state after token t) */
        double* ot = O + t * dv;
        for (int64_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int64_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qt[j];
            ot[i] = acc;
        }
    }
}

int gdn_oracle_recurrent_f64(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv,
                             const double* q, const double* k, const double* v,
                             const double* alpha, const double* beta, const double* eta,
                             const double* S0, double* O, double* S_final,
                             int nthreads)
{
    if (B <= 0 || H <= 0 || T <= 0 || dk <= 0 || dv <= 0) return -1;
    if (!q || !k || !v || !beta || !O || !S_final) return -1;
    const int64_t nseq = B * H;
    int ok = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double* u = (double*)malloc((size_t)dv * sizeof(double));
        if (!u) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            ok = -1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t s = 0; s < nseq; ++s) {
            if (!u) continue;
            run_one_sequence(T, dk, dv,
                             q + s * T * dk, k + s * T * dk, v + s * T * dv,
                             alpha ? alpha + s * T : NULL, beta + s * T,
                             eta ? eta + s * T : NULL,
                             S0 ? S0 + s * dv * dk : NULL,
                             O + s * T * dv, S_final + s * dv * dk, u);
        }
        free(u);
    }
    (void)nthreads;
    return ok;
}

/* Number of threads an unqualified call would use (for reporting). */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
