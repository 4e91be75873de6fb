/*
 * fp64 CPU oracle, rank-1 form, for Gated DeltaNet span replay.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
 * baseline of the benchmark.  It shares no code with the GPU library.
 *
 * Source: "Tail-Replay: Escaping the Curse of Linear Attention in Prefix
 * Caching for Hybrid LLMs", §2.3 eq. (1).  The state S is d_v x d_k (row-major,
 * d_k contiguous) and the key operator acts from the right:
 *     S <- alpha S (I - beta k k^T) + beta v k^T
 *        = alpha S + beta (v - alpha S k) k^T,
 * followed by the output o = S q on the post-update state.  Keys (and
 * optionally queries) are first divided by their exact L2 norm; a zero vector
 * stays zero.  Plain loops, no blocking, no reordering.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC gdn_oracle.c -o libgdn_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void unit_or_copy(const double *x, double *out, int32_t n, int normalize)
{
    if (!normalize) {
        memcpy(out, x, (size_t)n * sizeof(double));
        return;
    }
    double ss = 0.0;
    for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double nrm = sqrt(ss);
    for (int32_t i = 0; i < n; ++i) out[i] = nrm > 0.0 ? x[i] / nrm : 0.0;
}

/* One (request, head) pair: T tokens, state S (in: start, out: end). */
static void scan_one(int64_t T, int32_t dk, int32_t dv,
                     const double *q, const double *k, const double *v,
                     const double *alpha, const double *beta,
                     int normalize_k, int normalize_q,
                     double *S, double *o,
                     int64_t n_emit, const int64_t *emit_after, double *emit_states)
{
    double *kh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *qh = (double *)malloc(sizeof(double) * (size_t)dk);
    double *w = (double *)malloc(sizeof(double) * (size_t)dv);
    int64_t next_emit = 0;
    for (int64_t t = 0; t < T; ++t) {
        const double a = alpha[t];
        const double b = beta[t];
        unit_or_copy(k + t * dk, kh, dk, normalize_k);
        /* w = beta (v - alpha S k) */
        for (int32_t i = 0; i < dv; ++i) {
            double u = 0.0;
            for (int32_t j = 0; j < dk; ++j) u += S[(size_t)i * dk + j] * kh[j];
            w[i] = b * (v[t * dv + i] - a * u);
        }
        /* S <- alpha S + w k^T */
        for (int32_t i = 0; i < dv; ++i)
            for (int32_t j = 0; j < dk; ++j)
                S[(size_t)i * dk + j] = a * S[(size_t)i * dk + j] + w[i] * kh[j];
        /* o = S q */
        if (o) {
            unit_or_copy(q + t * dk, qh, dk, normalize_q);
            for (int32_t i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qh[j];
                o[t * dv + i] = acc;
            }
        }
        /* emission after t+1 tokens (list is in increasing order) */
        while (next_emit < n_emit && emit_after[next_emit] == t + 1) {
            memcpy(emit_states + (size_t)next_emit * dv * dk, S,
                   sizeof(double) * (size_t)dv * dk);
            ++next_emit;
        }
    }
    free(kh);
    free(qh);
    free(w);
}

int32_t gdn_oracle_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * P pairs, pair p owns token rows tok_off[p] .. tok_off[p+1]-1 of the
 * pair-major arrays q,k [rows][dk], v [rows][dv], alpha, beta [rows].
 * S: [P][dv][dk] in/out.  o: [rows][dv] or NULL (q may then be NULL).
 * Emissions: pair p records after token counts emit_after[emit_off[p] ..
 * emit_off[p+1]-1] (strictly increasing, each in 1..len) into emit_states.
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or 1 on bad arguments.
 */
int32_t gdn_oracle_scan_batch(int32_t P, const int64_t *tok_off, int32_t dk, int32_t dv,
                              const double *q, const double *k, const double *v,
                              const double *alpha, const double *beta,
                              int32_t normalize_k, int32_t normalize_q,
                              double *S, double *o,
                              const int64_t *emit_off, const int64_t *emit_after,
                              double *emit_states, int32_t nthreads)
{
    if (P < 0 || dk <= 0 || dv <= 0 || !tok_off || !k || !v || !alpha || !beta || !S)
        return 1;
    if (o && !q) return 1;
    for (int32_t p = 0; p < P; ++p) {
        if (tok_off[p + 1] < tok_off[p]) return 1;
        int64_t len = tok_off[p + 1] - tok_off[p];
        if (emit_off) {
            for (int64_t e = emit_off[p]; e < emit_off[p + 1]; ++e) {
                if (emit_after[e] < 1 || emit_after[e] > len) return 1;
                if (e > emit_off[p] && emit_after[e] <= emit_after[e - 1]) return 1;
            }
        }
    }
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int32_t p = 0; p < P; ++p) {
        const int64_t r0 = tok_off[p];
        const int64_t T = tok_off[p + 1] - r0;
        const int64_t e0 = emit_off ? emit_off[p] : 0;
        const int64_t ne = emit_off ? emit_off[p + 1] - e0 : 0;
        scan_one(T, dk, dv, q ? q + r0 * dk : NULL, k + r0 * dk, v + r0 * dv,
                 alpha + r0, beta + r0, normalize_k, normalize_q,
                 S + (size_t)p * dv * dk, o ? o + r0 * dv : NULL,
                 ne, emit_after + e0, emit_states + (size_t)e0 * dv * dk);
    }
    return 0;
}
