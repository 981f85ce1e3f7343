/*
 * Test infrastructure: the CPU oracle's sequential selective scan, in fp64.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * this file; the HIP library neither links nor includes it.
 *
 * What it computes (the Mamba selective state-space recurrence that the Jamba
 * paper's Mamba layers use -- Jamba: A Hybrid Transformer-Mamba Language Model,
 * §2 "Model architecture", citation [17]; the pages print no formula, so the
 * plain Euler-for-B / exponential-for-A discretisation is taken):
 *
 *   for every channel d and state index n, with h[-1] = h0[d, n]:
 *     h_t[d, n] = exp(dt_t[d] * A[d, n]) * h_{t-1}[d, n] + dt_t[d] * B_t[n] * x_t[d]
 *     y_t[d]    = sum_n C_t[n] * h_t[d, n] + D[d] * x_t[d]
 *
 * One plain loop per channel, time ascending; nothing is blocked or reordered.
 * Layouts (row-major, fp64): x, dt, y (T, d_inner); A, h0, h_last (d_inner, N);
 * B, C (T, N); D (d_inner). h0 may be NULL (zero state).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

void jm_oracle_scan(int64_t T, int64_t d_inner, int64_t N,
                    const double *x, const double *dt, const double *A,
                    const double *B, const double *C, const double *D,
                    const double *h0, double *y, double *h_last)
{
    #pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < d_inner; ++d) {
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? h0[d * N + n] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double dt_td = dt[t * d_inner + d];
            const double x_td = x[t * d_inner + d];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double decay = exp(dt_td * A[d * N + n]);
                h[n] = decay * h[n] + dt_td * B[t * N + n] * x_td;
                acc += C[t * N + n] * h[n];
            }
            y[t * d_inner + d] = acc + D[d] * x_td;
        }
        for (int64_t n = 0; n < N; ++n)
            h_last[d * N + n] = h[n];
        free(h);
    }
}
