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
 * The backward pass (oracle_backward, below) is the chain rule through the same
 * definition.
 *
 * The front end of the fused entry points (oracle_frontend, below) is the
 * softplus of the step size and the short causal convolution in front of the
 * scan.
 *
 * Pins (tests, not this file): LTI case == explicit and FFT convolution,
 * ZOH step == the ODE solved analytically and by RK4, the 1-D GRU gate,
 * forgetting at large delta, identity at delta = 0, brute-force unrolling,
 * hand-worked exact examples in tests/golden, split-sequence and per-step
 * consistency, linearity and causality; the backward pass by central finite
 * differences of oracle_forward and the transpose identity of the x -> y map;
 * the front end by numpy's correlate and logaddexp, impulse responses, the
 * SiLU reflection identity and streaming in pieces; the scalar-A-per-head
 * variant by the per-channel forward with A[d,n] = A_h and by its dense
 * lower-triangular (semiseparable) matrix form built in numpy.
 * Every function here is pinned.
 *
 * Threads: channels (b, d) are independent, so `nthreads` workers take
 * disjoint sets of channels; each channel's token loop stays sequential.  The
 * scalar-A-per-head variant splits its independent (b, h, p) rows the same way.
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

/*
 * Backward pass: gradients of a scalar loss through the forward pass above.
 * Given dy = dLoss/dy (batch, L, dim) and dhT = dLoss/d(final state) (NULL = 0),
 * returns dx, ddelta (batch, L, dim), dA (dim, N), dB, dC (batch, L, N),
 * dDskip (dim) and dh0 = dLoss/d(initial state) (batch, dim, N; NULL = not wanted).
 *
 * Plain chain rule on the definition, token by token backwards in time with the
 * adjoint lam_t = dLoss/dh_t:
 *     lam_t   = C_t * dy_t + Abar_{t+1} * lam_{t+1}      (lam_{L-1} gets dhT instead)
 *     dx_t    = Dskip * dy_t + sum_n lam_t * Bbar_t
 *     ddelta  = sum_n lam_t * (dAbar/ddelta * h_{t-1} + dgain/ddelta * B_t x_t)
 *     dA      = sum_t lam_t * (dAbar/dA * h_{t-1} + dgain/dA * B_t x_t)
 *     dB_t    = sum_d lam_t * gain_t * x_t,   dC_t = sum_d dy_t * h_t,   dDskip = sum dy * x
 *     dh0     = Abar_0 * lam_0
 * with Abar = exp(delta*A), gain = (exp(delta*A) - 1)/A (delta when A = 0) and
 *     dAbar/ddelta = A*Abar,  dgain/ddelta = Abar,  dAbar/dA = delta*Abar,
 *     dgain/dA = (delta*Abar - gain)/A  (delta^2/2 when A = 0).
 * The forward states h_t of a channel are kept (L+1 rows of N doubles).
 * Pinned in tests by central finite differences of oracle_forward.
 */
typedef struct {
    const double *x, *delta, *A, *B, *C, *Dskip, *h0, *dy, *dhT;
    double *dx, *ddelta, *dA, *dB, *dC, *dD, *dh0;
    int64_t batch, L, dim, N;
    int64_t d_first, d_last; /* channel range [d_first, d_last) of this worker, all batch rows */
    double *hist;            /* (L+1)*N doubles */
    double *lam;             /* N doubles */
} bwd_job;

static void *bwd_worker(void *arg) {
    bwd_job *j = (bwd_job *)arg;
    const int64_t L = j->L, dim = j->dim, N = j->N;
    for (int64_t d = j->d_first; d < j->d_last; ++d) {
        const double *Ar = j->A + d * N;
        const double dsk = j->Dskip ? j->Dskip[d] : 0.0;
        for (int64_t b = 0; b < j->batch; ++b) {
            const int64_t c = b * dim + d;
            double *h = j->hist; /* row 0 = h_{-1}, row t+1 = h_t */
            for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[c * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t e = (b * L + t) * dim + d;
                const int64_t r = (b * L + t) * N;
                double *hp = h + t * N, *hn = h + (t + 1) * N;
                for (int64_t n = 0; n < N; ++n) {
                    const double z = j->delta[e] * Ar[n];
                    const double abar = exp(z);
                    const double gain = (Ar[n] != 0.0) ? expm1(z) / Ar[n] : j->delta[e];
                    hn[n] = abar * hp[n] + gain * j->B[r + n] * j->x[e];
                }
            }
            for (int64_t n = 0; n < N; ++n) j->lam[n] = j->dhT ? j->dhT[c * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t e = (b * L + t) * dim + d;
                const int64_t r = (b * L + t) * N;
                const double xv = j->x[e], dt = j->delta[e], g = j->dy[e];
                const double *hp = h + t * N, *hn = h + (t + 1) * N;
                double dxv = dsk * g, ddv = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double a = Ar[n];
                    const double z = dt * a;
                    const double abar = exp(z);
                    const double gain = (a != 0.0) ? expm1(z) / a : dt;
                    const double dgain_dA = (a != 0.0) ? (dt * abar - gain) / a : 0.5 * dt * dt;
                    const double lam = j->lam[n] + j->C[r + n] * g; /* lam_t */
                    const double bx = j->B[r + n] * xv;
                    dxv += lam * gain * j->B[r + n];
                    ddv += lam * (a * abar * hp[n] + abar * bx);
                    j->dA[d * N + n] += lam * (dt * abar * hp[n] + dgain_dA * bx);
                    j->dB[r + n] += lam * gain * xv;
                    j->dC[r + n] += g * hn[n];
                    j->lam[n] = abar * lam; /* carried to t-1 */
                }
                j->dx[e] = dxv;
                j->ddelta[e] = ddv;
                j->dD[d] += g * xv;
            }
            if (j->dh0)
                for (int64_t n = 0; n < N; ++n) j->dh0[c * N + n] = j->lam[n];
        }
    }
    return NULL;
}

int oracle_backward(const double *x, const double *delta, const double *A, const double *B,
                    const double *C, const double *Dskip, const double *h0, const double *dy,
                    const double *dhT, double *dx, double *ddelta, double *dA, double *dB, double *dC,
                    double *dD, double *dh0, int64_t batch, int64_t L, int64_t dim, int64_t N,
                    int nthreads) {
    if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC || !dD)
        return ORACLE_ERR_ARG;
    if (batch < 0 || L < 0 || dim < 0 || N < 1) return ORACLE_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > dim) nthreads = dim > 0 ? (int)dim : 1;
    const int64_t nbc = batch * L * N;
    /* dB and dC are sums over channels: each worker accumulates its own copy, and the
     * copies are added in worker order afterwards (deterministic). */
    double *acc = (double *)calloc((size_t)(nthreads * 2 * nbc + 1), sizeof(double));
    double *hist = (double *)calloc((size_t)(nthreads * ((L + 1) * N + N)), sizeof(double));
    bwd_job *jobs = (bwd_job *)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    char *started = (char *)calloc((size_t)nthreads, 1);
    if (!acc || !hist || !jobs || !tid || !started) {
        free(acc); free(hist); free(jobs); free(tid); free(started);
        return ORACLE_ERR_ARG;
    }
    for (int64_t i = 0; i < dim * N; ++i) dA[i] = 0.0;
    for (int64_t i = 0; i < dim; ++i) dD[i] = 0.0;
    for (int i = 0; i < nthreads; ++i) {
        double *hi = hist + (int64_t)i * ((L + 1) * N + N);
        bwd_job j = {x, delta, A, B, C, Dskip, h0, dy, dhT, dx, ddelta, dA,
                     acc + (int64_t)i * 2 * nbc, acc + (int64_t)i * 2 * nbc + nbc, dD, dh0,
                     batch, L, dim, N, dim * i / nthreads, dim * (i + 1) / nthreads,
                     hi, hi + (L + 1) * N};
        jobs[i] = j;
    }
    if (nthreads == 1) {
        bwd_worker(&jobs[0]);
    } else {
        for (int i = 0; i < nthreads; ++i) {
            if (pthread_create(&tid[i], NULL, bwd_worker, &jobs[i]) == 0)
                started[i] = 1;
            else
                bwd_worker(&jobs[i]);
        }
        for (int i = 0; i < nthreads; ++i)
            if (started[i]) pthread_join(tid[i], NULL);
    }
    for (int64_t k = 0; k < nbc; ++k) {
        double sb = 0.0, sc = 0.0;
        for (int i = 0; i < nthreads; ++i) {
            sb += acc[(int64_t)i * 2 * nbc + k];
            sc += acc[(int64_t)i * 2 * nbc + nbc + k];
        }
        dB[k] = sb;
        dC[k] = sc;
    }
    free(acc); free(hist); free(jobs); free(tid); free(started);
    return ORACLE_OK;
}

/*
 * Front end that feeds the scan, for the fused entry points.
 *
 * Step size ("Mamba and State Space Models", the selective pseudocode;
 * knowledge-base entry on Mamba, section 3.2, algorithm 2): the projection of
 * the token plus a bias, made positive by softplus(v) = log(1 + e^v):
 *     delta[b,t,d] = softplus(delta_raw[b,t,d] + delta_bias[d])
 * evaluated as max(v,0) + log1p(exp(-|v|)), which is the same function
 * without overflow.  NULL delta_bias means 0.
 *
 * Short convolution in front of the SSM ("Mamba and State Space Models",
 * "How this shows up in practice", d_conv): causal, per channel, of width K:
 *     c[b,t,d] = conv_bias[d] + sum_{k=0}^{K-1} w[d,k] * xin[b, t-K+1+k, d]
 * where inputs before token 0 are the K-1 rows of conv_state (row j is token
 * j-(K-1)), or zero when conv_state is NULL; NULL conv_bias means 0.  The
 * pages name no nonlinearity after it: act = 0 leaves c as the scan input,
 * act = 1 applies SiLU, u = c / (1 + exp(-c)).
 * conv_state_out (may be NULL) receives the last K-1 inputs (the state a
 * following call continues from), rows in token order.
 *
 * Layouts: xin, delta_raw, u, delta (batch, L, dim); w (dim, K); conv_bias,
 * delta_bias (dim); conv_state, conv_state_out (batch, K-1, dim).
 */
static double softplus(double v) {
    return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

int oracle_frontend(const double *xin, const double *w, const double *conv_bias, int K, int act,
                    const double *conv_state, const double *delta_raw, const double *delta_bias,
                    double *u, double *delta, double *conv_state_out, int64_t batch, int64_t L,
                    int64_t dim) {
    if (!xin || !w || !delta_raw || !u || !delta || K < 1 || batch < 0 || L < 0 || dim < 0 ||
        (act != 0 && act != 1))
        return ORACLE_ERR_ARG;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            for (int64_t t = 0; t < L; ++t) {
                double c = conv_bias ? conv_bias[d] : 0.0;
                for (int k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k; /* input token of tap k */
                    double v;
                    if (s >= 0)
                        v = xin[(b * L + s) * dim + d];
                    else /* row s + K - 1 of the carried inputs */
                        v = conv_state ? conv_state[(b * (K - 1) + (s + K - 1)) * dim + d] : 0.0;
                    c += w[d * K + k] * v;
                }
                const int64_t e = (b * L + t) * dim + d;
                u[e] = act == 1 ? c / (1.0 + exp(-c)) : c;
                delta[e] = softplus(delta_raw[e] + (delta_bias ? delta_bias[d] : 0.0));
            }
            if (conv_state_out) {
                for (int j = 0; j < K - 1; ++j) {
                    const int64_t s = L - (K - 1) + j; /* token of row j */
                    double v;
                    if (s >= 0)
                        v = xin[(b * L + s) * dim + d];
                    else
                        v = conv_state ? conv_state[(b * (K - 1) + (s + K - 1)) * dim + d] : 0.0;
                    conv_state_out[(b * (K - 1) + j) * dim + d] = v;
                }
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Scalar-A-per-head variant (Mamba-2's state space model: "Mamba and State
 * Space Models" and "Mamba matches the Transformer...", the section on the
 * state space duality).  The same zero-order-hold recurrence as above with
 * A[d,n] = A_h for every state n and every channel p of head h, delta
 * per (b, t, h), and B, C per (b, t, group), shared by the heads of a group
 * (head h reads group h / (H/G)):
 *     abar = exp(delta[b,t,h] * A_h)
 *     gain = expm1(delta * A_h) / A_h          (delta when A_h == 0)
 *     h[p][n] = abar * h[p][n] + gain * B[b,t,g,n] * x[b,t,h,p]
 *     y[b,t,h,p] = sum over n (ascending) of C[b,t,g,n] * h[p][n] + D[h] * x[b,t,h,p]
 * Layouts (row-major): x, y (batch, L, H, P); delta (batch, L, H); A, D (H);
 * B, C (batch, L, G, N); h0, hT (batch, H, P, N).  NULL D means 0, NULL h0
 * zero, NULL hT not written.  Written as its own loop (not through token()),
 * so that the two can be checked against each other.
 */
typedef struct {
    const double *x, *delta, *A, *B, *C, *D, *h0;
    double *y, *hT;
    int64_t batch, L, H, P, G, N;
    int64_t first, last; /* state-row range [first, last) over batch*H*P */
    double *st;          /* N doubles */
} ssd_job;

/* The rows (b, h, p) of [first, last), each with its own sequential token loop. */
static void *ssd_worker(void *arg) {
    const ssd_job *j = (const ssd_job *)arg;
    const int64_t L = j->L, H = j->H, P = j->P, G = j->G, N = j->N;
    const int64_t hpg = H / G;
    double *st = j->st;
    for (int64_t row = j->first; row < j->last; ++row) {
        const int64_t p = row % P, h = (row / P) % H, b = row / (P * H);
        const int64_t g = h / hpg;
        const double a = j->A[h];
        const double dsk = j->D ? j->D[h] : 0.0;
        const int64_t so = row * N; /* state row of (b, h, p) */
        for (int64_t n = 0; n < N; ++n) st[n] = j->h0 ? j->h0[so + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double dt = j->delta[(b * L + t) * H + h];
            const double abar = exp(dt * a);
            const double gain = (a != 0.0) ? expm1(dt * a) / a : dt;
            const double xv = j->x[((b * L + t) * H + h) * P + p];
            const double *Bt = j->B + ((b * L + t) * G + g) * N;
            const double *Ct = j->C + ((b * L + t) * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                st[n] = abar * st[n] + gain * Bt[n] * xv;
                acc += Ct[n] * st[n];
            }
            j->y[((b * L + t) * H + h) * P + p] = acc + dsk * xv;
        }
        if (j->hT)
            for (int64_t n = 0; n < N; ++n) j->hT[so + n] = st[n];
    }
    return NULL;
}

/* Rows (b, h, p) are independent: `nthreads` workers take disjoint row ranges, and
 * every row's token loop stays sequential, so the result does not depend on the
 * thread count. */
int oracle_ssd_forward(const double *x, const double *delta, const double *A, const double *B,
                       const double *C, const double *D, const double *h0, double *y, double *hT,
                       int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                       int nthreads) {
    if (!x || !delta || !A || !B || !C || !y || batch < 0 || L < 0 || H < 1 || P < 1 || G < 1 ||
        N < 1 || H % G != 0)
        return ORACLE_ERR_ARG;
    const int64_t rows = batch * H * P;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    ssd_job *jobs = (ssd_job *)calloc((size_t)nthreads, sizeof(ssd_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    double *st = (double *)calloc((size_t)(nthreads * N), sizeof(double));
    char *started = (char *)calloc((size_t)nthreads, 1);
    if (!jobs || !tid || !st || !started) {
        free(jobs); free(tid); free(st); free(started);
        return ORACLE_ERR_ARG;
    }
    for (int i = 0; i < nthreads; ++i) {
        ssd_job j = {x, delta, A, B, C, D, h0, y, hT, batch, L, H, P, G, N,
                     rows * i / nthreads, rows * (i + 1) / nthreads, st + (int64_t)i * N};
        jobs[i] = j;
    }
    /* a worker that cannot be started runs on the calling thread instead */
    for (int i = 0; i < nthreads; ++i) {
        if (nthreads > 1 && pthread_create(&tid[i], NULL, ssd_worker, &jobs[i]) == 0)
            started[i] = 1;
        else
            ssd_worker(&jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i)
        if (started[i]) pthread_join(tid[i], NULL);
    free(jobs); free(tid); free(st); free(started);
    return ORACLE_OK;
}

int oracle_version(void) { return 5; }
