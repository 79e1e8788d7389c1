/*
 * sscan_oracle.c -- plain, sequential fp64 CPU reference of the selective scan (S6).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load or call this library.  The product
 * (the HIP library and its Python binding) never links, imports or calls it,
 * and it shares no code, header, table or helper with the HIP path.
 *
 * What it computes, for every batch row b, channel d and state index n, in
 * the order the pages state it (no blocking, no reassociation):
 *
 *   1. Zero-order-hold discretisation of the diagonal continuous system
 *      h'(t) = A h(t) + B x(t)   ("The loop that beats attention", section
 *      "Where A, B and C come from", eq. (2); also "Mamba and State Space
 *      Models", "Mechanism: a continuous-time linear system"):
 *          Abar = exp(delta * A[d,n])
 *          Bbar = (delta*A)^-1 (exp(delta*A) - 1) * delta * B[t,n]
 *               = expm1(delta*A[d,n]) / A[d,n] * B[t,n]      (A diagonal)
 *      When A[d,n] == 0 the expression is read as its limit delta * B[t,n].
 *      expm1 is exp(z)-1 evaluated without cancellation; it is the same
 *      quantity, not a different formula.
 *   2. The linear recurrence ("The loop that beats attention", eq. (1);
 *      "Mamba and State Space Models", the selective pseudocode):
 *          h[n] = Abar * h[n] + Bbar * x[b,t,d]
 *      starting from h = 0, or from a caller-given initial state.
 *   3. The readout, with the skip term of the continuous form y = C h + D x
 *      ("State space models and Mamba", the continuous linear SSM):
 *          y[b,t,d] = sum over n (ascending) of C[b,t,n] * h[n] + Dskip[d] * x[b,t,d]
 *   4. The state after the last token is the final state ("Mamba and State
 *      Space Models", failure mode 2: a prefix is resumed from a snapshot of
 *      the state).
 *
 * Selection ("Mamba and State Space Models", "Mamba: making the state
 * selective"; "Mamba matches the Transformer...", "Selection makes the
 * recurrence read the token"): delta is given per (b, t, d); B and C per
 * (b, t, n), shared by all channels; A per (d, n).
 *
 * Layouts (row-major, contiguous):
 *   x, delta, y        (batch, L, dim)
 *   B, C               (batch, L, N)
 *   A                  (dim, N)
 *   Dskip              (dim)            NULL means 0
 *   h0, final_state    (batch, dim, N)  NULL means zero start / not written
 * The decode step uses (batch, dim) for x_t, delta_t, y_t and (batch, N) for
 * B_t, C_t, and updates state (batch, dim, N) in place.
 *
 * Pins (tests, not this file): LTI case == explicit and FFT convolution,
 * ZOH step == the ODE solved analytically and by RK4, the 1-D GRU gate,
 * forgetting at large delta, identity at delta = 0, brute-force unrolling,
 * hand-worked exact examples in tests/golden, split-sequence and per-step
 * consistency, linearity and causality.  Every function here is pinned.
 *
 * Threads: channels (b, d) are independent, so `nthreads` workers take
 * disjoint sets of channels; each channel's token loop stays sequential.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1

/* One token of one channel: discretise, update the N states, read out. */
static double token(double *h, double x, double delta, const double *A_row, const double *B_t,
                    const double *C_t, double dskip, int64_t N) {
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double a = A_row[n];
        const double z = delta * a;
        const double abar = exp(z);
        const double bbar = (a != 0.0) ? expm1(z) / a * B_t[n] : delta * B_t[n];
        h[n] = abar * h[n] + bbar * x;
    }
    for (int64_t n = 0; n < N; ++n) y += C_t[n] * h[n];
    return y + dskip * x;
}

typedef struct {
    const double *x, *delta, *A, *B, *C, *Dskip, *h0;
    double *y, *final_state;
    int64_t batch, L, dim, N;
    int64_t first, last; /* channel range [first, last) over batch*dim */
    double *scratch;     /* N doubles */
} fwd_job;

static void *fwd_worker(void *arg) {
    fwd_job *j = (fwd_job *)arg;
    double *h = j->scratch;
    for (int64_t c = j->first; c < j->last; ++c) {
        const int64_t b = c / j->dim, d = c % j->dim;
        for (int64_t n = 0; n < j->N; ++n) h[n] = j->h0 ? j->h0[c * j->N + n] : 0.0;
        const double dskip = j->Dskip ? j->Dskip[d] : 0.0;
        for (int64_t t = 0; t < j->L; ++t) {
            const int64_t e = (b * j->L + t) * j->dim + d;
            const int64_t r = (b * j->L + t) * j->N;
            j->y[e] = token(h, j->x[e], j->delta[e], j->A + d * j->N, j->B + r, j->C + r, dskip, j->N);
        }
        if (j->final_state)
            for (int64_t n = 0; n < j->N; ++n) j->final_state[c * j->N + n] = h[n];
    }
    return NULL;
}

/* Whole-sequence forward pass.  Returns 0, or ORACLE_ERR_ARG on bad arguments. */
int oracle_forward(const double *x, const double *delta, const double *A, const double *B,
                   const double *C, const double *Dskip, const double *h0, double *y,
                   double *final_state, int64_t batch, int64_t L, int64_t dim, int64_t N,
                   int nthreads) {
    if (!x || !delta || !A || !B || !C || !y) return ORACLE_ERR_ARG;
    if (batch < 0 || L < 0 || dim < 0 || N < 1) return ORACLE_ERR_ARG;
    const int64_t chans = batch * dim;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > chans) nthreads = chans > 0 ? (int)chans : 1;

    fwd_job *jobs = (fwd_job *)calloc((size_t)nthreads, sizeof(fwd_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    double *scratch = (double *)calloc((size_t)(nthreads * N), sizeof(double));
    if (!jobs || !tid || !scratch) {
        free(jobs); free(tid); free(scratch);
        return ORACLE_ERR_ARG;
    }
    for (int i = 0; i < nthreads; ++i) {
        fwd_job j = {x, delta, A, B, C, Dskip, h0, y, final_state, batch, L, dim, N,
                     chans * i / nthreads, chans * (i + 1) / nthreads, scratch + (int64_t)i * N};
        jobs[i] = j;
    }
    if (nthreads == 1) {
        fwd_worker(&jobs[0]);
    } else {
        /* a worker that cannot be started runs on the calling thread instead */
        char *started = (char *)calloc((size_t)nthreads, 1);
        for (int i = 0; i < nthreads; ++i) {
            if (started && pthread_create(&tid[i], NULL, fwd_worker, &jobs[i]) == 0)
                started[i] = 1;
            else
                fwd_worker(&jobs[i]);
        }
        for (int i = 0; i < nthreads; ++i)
            if (started && started[i]) pthread_join(tid[i], NULL);
        free(started);
    }
    free(jobs); free(tid); free(scratch);
    return ORACLE_OK;
}

/* One decode step for every (b, d): state (batch, dim, N) is read and written in place. */
int oracle_step(double *state, const double *x_t, const double *delta_t, const double *A,
                const double *B_t, const double *C_t, const double *Dskip, double *y_t,
                int64_t batch, int64_t dim, int64_t N) {
    if (!state || !x_t || !delta_t || !A || !B_t || !C_t || !y_t) return ORACLE_ERR_ARG;
    if (batch < 0 || dim < 0 || N < 1) return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t d = 0; d < dim; ++d) {
            const int64_t e = b * dim + d;
            y_t[e] = token(state + e * N, x_t[e], delta_t[e], A + d * N, B_t + b * N, C_t + b * N,
                           Dskip ? Dskip[d] : 0.0, N);
        }
    return ORACLE_OK;
}

int oracle_version(void) { return 1; }
