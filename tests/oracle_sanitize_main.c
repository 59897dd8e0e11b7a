/*
 * oracle_sanitize_main.c -- drives the C oracle (oracle/m3_oracle.c) over a
 * set of shapes for a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer (tests/test_oracle_sanitized.py).  Every buffer is allocated at
 * its exact size, so a read or write past any of them is reported.  Exit
 * status 0: every call returned the expected status, every output is finite,
 * and results do not depend on the thread count (bit for bit).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int m3o_run(int64_t batch, int64_t T, int32_t H, int32_t P, int32_t N, int32_t R,
            const double *x, const double *dt, const double *A, const double *lam,
            const double *theta, const double *B, const double *C,
            const double *h0, const double *prevB0, const double *prevx0,
            double *y, double *hT, int nthreads);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double uni(void) /* xorshift64*, uniform in [0, 1) */
{
    g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
    return (double)((g_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}

static double *fill(size_t n, double lo, double hi)
{
    double *p = malloc(n * sizeof(double));
    if (!p) exit(3);
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * uni();
    return p;
}

static int finite_all(const double *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

static int run_case(int64_t b, int64_t T, int32_t H, int32_t P, int32_t N, int32_t R, int with_init,
                    int with_final)
{
    const size_t K = (size_t)N / 2, BT = (size_t)(b * T * H), BH = (size_t)(b * H);
    double *x = fill(BT * R * P, -1, 1), *B = fill(BT * R * N, -1, 1), *C = fill(BT * R * N, -1, 1);
    double *dt = fill(BT, 0.01, 1.5), *lam = fill(BT, 0, 1), *theta = fill(BT * K, 0, 3.14159);
    double *A = fill((size_t)H, -4, 0);
    double *h0 = with_init ? fill(BH * N * P, -1, 1) : NULL;
    double *pB = with_init ? fill(BH * R * N, -1, 1) : NULL;
    double *px = with_init ? fill(BH * R * P, -1, 1) : NULL;
    double *y1 = malloc((BT * R * P + 1) * sizeof(double)), *y2 = malloc((BT * R * P + 1) * sizeof(double));
    double *hT1 = with_final ? malloc(BH * N * P * sizeof(double)) : NULL;
    double *hT2 = with_final ? malloc(BH * N * P * sizeof(double)) : NULL;
    int ok = 1;
    const int r1 = m3o_run(b, T, H, P, N, R, x, dt, A, lam, theta, B, C, h0, pB, px, y1, hT1, 1);
    const int r2 = m3o_run(b, T, H, P, N, R, x, dt, A, lam, theta, B, C, h0, pB, px, y2, hT2, 3);
    if (r1 <= 0 || r2 <= 0) ok = 0;
    if (ok && !finite_all(y1, BT * R * P)) ok = 0;
    if (ok && memcmp(y1, y2, BT * R * P * sizeof(double)) != 0) ok = 0;
    if (ok && with_final && (!finite_all(hT1, BH * N * P) || memcmp(hT1, hT2, BH * N * P * sizeof(double)) != 0))
        ok = 0;
    if (!ok) fprintf(stderr, "case b%lld T%lld H%d P%d N%d R%d init %d final %d failed (%d, %d)\n",
                     (long long)b, (long long)T, H, P, N, R, with_init, with_final, r1, r2);
    free(x); free(B); free(C); free(dt); free(lam); free(theta); free(A);
    free(h0); free(pB); free(px); free(y1); free(y2); free(hT1); free(hT2);
    return ok;
}

int main(void)
{
    int ok = 1;
    ok &= run_case(1, 1, 1, 4, 2, 1, 0, 1);
    ok &= run_case(1, 37, 2, 8, 6, 3, 1, 1);
    ok &= run_case(2, 19, 3, 5, 8, 2, 1, 0);
    ok &= run_case(3, 64, 2, 16, 16, 4, 0, 1);
    ok &= run_case(1, 130, 1, 3, 4, 1, 1, 1);
    /* bad arguments are rejected before any access */
    double a = -1.0;
    if (m3o_run(1, 4, 1, 4, 3, 1, NULL, NULL, &a, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1)
        ok = 0;
    if (m3o_run(1, 4, 1, 4, 4, 1, NULL, NULL, &a, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1)
        ok = 0;
    /* T = 0: nothing to read or write */
    if (m3o_run(2, 0, 1, 4, 4, 1, NULL, NULL, &a, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 2) <= 0)
        ok = 0;
    puts(ok ? "oracle sanitize driver: ok" : "oracle sanitize driver: FAILED");
    return ok ? 0 : 1;
}
