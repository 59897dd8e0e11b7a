/*
 * m3_oracle.c -- plain fp64 CPU oracle for the Mamba-3 SSM sequence mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (one independent instance per (batch b, head h)):
 *
 *   The exponential-trapezoidal recurrence of the Mamba-3 review
 *   (junhanzang.github.io, "Mamba-3: expressive SSM with MIMO"), section 3.1.1,
 *   Proposition 3.1.1, eqs. (5)-(6) and the coefficient table:
 *       alpha_t = exp(dt_t * A),  beta_t = (1 - lam_t) dt_t alpha_t,
 *       gamma_t = lam_t dt_t,
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t.
 *   The same coefficients are restated in the koala.ai.kr Mamba-3 post,
 *   section 1 (discretisation comparison).
 *
 *   with the complex-valued state of section 3.2 (Propositions 3.2.1 and
 *   3.2.3): a complex SSM of N/2 states is a real SSM of N states whose
 *   transition is block-diagonal 2x2 rotations.  Row pair (2k, 2k+1) of the
 *   real state is the complex number z_k = h[2k] + i h[2k+1]; the rotation
 *   for token t multiplies z_k by exp(i theta_{t,k}).  Applying the
 *   trapezoid rule of Prop. 3.1.1 to that complex system gives, in the
 *   state's own ("true") frame,
 *       z_t = exp(dt_t A + i theta_t) * ( z_{t-1} + delta_t b_{t-1} x_{t-1} )
 *             + gamma_t b_t x_t,                 delta_t = (1 - lam_t) dt_t,
 *   which is Prop. 3.2.3 multiplied through by the cumulative rotation
 *   prod_{i<=t} R_i (so that the rotated B_{t-1}, B_t and C_t of the
 *   proposition become the raw inputs).  The per-step angle is theta_t
 *   itself (reading: the caller passes any dt-scaling pre-multiplied).
 *
 *   and the MIMO generalisation of section 3.3: B_t, C_t are N x R, x_t is
 *   R x P, the rank-1 update B x^T becomes the rank-R product
 *   sum_r B[:,r] x[r,:], and the output has R rows,
 *       y_t[i, p] = sum_n C_t[n, i] h_t[n, p] = Re sum_k conj(c_k,i) z_k,p.
 *
 *   On a fresh sequence there is no previous token (row 0 of the 2-band
 *   matrix of eq. (7) holds only gamma_0), so the beta term of t = 0 is
 *   zero.  A carried state supplies the previous token's B and x.
 *
 * Memory layouts (row-major, contiguous, fp64):
 *   x, y        [batch][T][H][R][P]
 *   B, C        [batch][T][H][R][N]     (rank-major: B[..][r][n] = B_t[n, r])
 *   dt, lam     [batch][T][H]
 *   theta       [batch][T][H][N/2]      (angle of row pair k)
 *   A           [H]
 *   h0, hT      [batch][H][N][P]        (true frame)
 *   prevB0      [batch][H][R][N]        (true-frame B of the previous token)
 *   prevx0      [batch][H][R][P]
 *
 * The arithmetic is a plain sequential loop over t per instance; instances
 * run on a pthread pool, which changes nothing in the result.
 */
#include <complex.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int64_t batch, T;
    int32_t H, P, N, R;
    const double *x, *dt, *A, *lam, *theta, *B, *C;
    const double *h0, *prevB0, *prevx0;
    double *y, *hT;
    int64_t next;           /* next instance to take */
    pthread_mutex_t lock;
    int failed;
} job_t;

/* One (b, h) instance: the recurrence written out term by term. */
static int run_instance(const job_t *j, int64_t b, int32_t h)
{
    const int32_t H = j->H, P = j->P, N = j->N, R = j->R, K = N / 2;
    const int64_t T = j->T;
    const double A = j->A[h];

    double complex *z = calloc((size_t)K * P, sizeof(double complex));
    double complex *bprev = calloc((size_t)K * R, sizeof(double complex));
    double complex *bcur = calloc((size_t)K * R, sizeof(double complex));
    double complex *ccur = calloc((size_t)K * R, sizeof(double complex));
    double *xprev = calloc((size_t)R * P, sizeof(double));
    if (!z || !bprev || !bcur || !ccur || !xprev) {
        free(z); free(bprev); free(bcur); free(ccur); free(xprev);
        return -1;
    }

    /* Carried state: z_{-1}, and the previous token's b and x (zero on a
       fresh sequence). */
    if (j->h0) {
        const double *h0 = j->h0 + ((b * H + h) * (int64_t)N) * P;
        for (int32_t k = 0; k < K; ++k)
            for (int32_t p = 0; p < P; ++p)
                z[k * P + p] = h0[(2 * k) * P + p] + I * h0[(2 * k + 1) * P + p];
    }
    if (j->prevB0) {
        const double *pb = j->prevB0 + ((b * H + h) * (int64_t)R) * N;
        for (int32_t r = 0; r < R; ++r)
            for (int32_t k = 0; k < K; ++k)
                bprev[k * R + r] = pb[r * N + 2 * k] + I * pb[r * N + 2 * k + 1];
    }
    if (j->prevx0) {
        const double *px = j->prevx0 + ((b * H + h) * (int64_t)R) * P;
        memcpy(xprev, px, sizeof(double) * (size_t)R * P);
    }

    for (int64_t t = 0; t < T; ++t) {
        const int64_t th = (b * T + t) * H + h;          /* token-head index */
        const double dt = j->dt[th];
        const double lam = j->lam[th];
        const double gamma = lam * dt;
        const double delta = (1.0 - lam) * dt;
        const double *xt = j->x + th * (int64_t)R * P;
        const double *Bt = j->B + th * (int64_t)R * N;
        const double *Ct = j->C + th * (int64_t)R * N;
        const double *tht = j->theta + th * (int64_t)K;

        for (int32_t r = 0; r < R; ++r)
            for (int32_t k = 0; k < K; ++k) {
                bcur[k * R + r] = Bt[r * N + 2 * k] + I * Bt[r * N + 2 * k + 1];
                ccur[k * R + r] = Ct[r * N + 2 * k] + I * Ct[r * N + 2 * k + 1];
            }

        for (int32_t k = 0; k < K; ++k) {
            /* exp(dt A + i theta): decay times rotation of pair k. */
            const double complex e = cexp(dt * A + I * tht[k]);
            for (int32_t p = 0; p < P; ++p) {
                double complex vprev = 0.0, vcur = 0.0;
                for (int32_t r = 0; r < R; ++r) {
                    vprev += bprev[k * R + r] * xprev[r * P + p];
                    vcur += bcur[k * R + r] * xt[r * P + p];
                }
                z[k * P + p] = e * (z[k * P + p] + delta * vprev) + gamma * vcur;
            }
        }

        double *yt = j->y + th * (int64_t)R * P;
        for (int32_t i = 0; i < R; ++i)
            for (int32_t p = 0; p < P; ++p) {
                double complex acc = 0.0;
                for (int32_t k = 0; k < K; ++k)
                    acc += conj(ccur[k * R + i]) * z[k * P + p];
                yt[i * P + p] = creal(acc);
            }

        /* This token becomes the previous token of t + 1. */
        memcpy(bprev, bcur, sizeof(double complex) * (size_t)K * R);
        memcpy(xprev, xt, sizeof(double) * (size_t)R * P);
    }

    if (j->hT) {
        double *hT = j->hT + ((b * H + h) * (int64_t)N) * P;
        for (int32_t k = 0; k < K; ++k)
            for (int32_t p = 0; p < P; ++p) {
                hT[(2 * k) * P + p] = creal(z[k * P + p]);
                hT[(2 * k + 1) * P + p] = cimag(z[k * P + p]);
            }
    }
    free(z); free(bprev); free(bcur); free(ccur); free(xprev);
    return 0;
}

static void *worker(void *arg)
{
    job_t *j = (job_t *)arg;
    const int64_t n = j->batch * j->H;
    for (;;) {
        pthread_mutex_lock(&j->lock);
        const int64_t i = j->next++;
        pthread_mutex_unlock(&j->lock);
        if (i >= n) break;
        if (run_instance(j, i / j->H, (int32_t)(i % j->H)) != 0) {
            pthread_mutex_lock(&j->lock);
            j->failed = 1;
            pthread_mutex_unlock(&j->lock);
        }
    }
    return NULL;
}

/* Number of threads a call with nthreads <= 0 uses. */
int m3o_default_threads(void)
{
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Run the recurrence over every (b, h).  Returns the number of threads used
 * (> 0), or a negative value on bad arguments (-1) or allocation failure (-2).
 * h0, prevB0, prevx0 may be NULL (zero); hT may be NULL (not written).
 */
int m3o_run(int64_t batch, int64_t T, int32_t H, int32_t P, int32_t N, int32_t R,
            const double *x, const double *dt, const double *A, const double *lam,
            const double *theta, const double *B, const double *C,
            const double *h0, const double *prevB0, const double *prevx0,
            double *y, double *hT, int nthreads)
{
    if (batch < 0 || T < 0 || H < 1 || P < 1 || N < 2 || (N % 2) != 0 || R < 1)
        return -1;
    if (!A || (T > 0 && (!x || !dt || !lam || !theta || !B || !C || !y)))
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.batch = batch; j.T = T; j.H = H; j.P = P; j.N = N; j.R = R;
    j.x = x; j.dt = dt; j.A = A; j.lam = lam; j.theta = theta; j.B = B; j.C = C;
    j.h0 = h0; j.prevB0 = prevB0; j.prevx0 = prevx0; j.y = y; j.hT = hT;
    pthread_mutex_init(&j.lock, NULL);

    if (nthreads <= 0) nthreads = m3o_default_threads();
    const int64_t n = batch * H;
    if (nthreads > n) nthreads = n > 0 ? (int)n : 1;
    pthread_t *tid = malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!tid) { pthread_mutex_destroy(&j.lock); return -2; }
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &j) != 0) break;
        ++started;
    }
    if (started == 0) worker(&j);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&j.lock);
    if (j.failed) return -2;
    return started > 0 ? started : 1;
}
