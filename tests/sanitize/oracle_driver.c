/* Drives the C oracle (oracle/m3ref.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: scans of several shapes (empty, single token,
 * ragged, MIMO, with and without angles and carry), the split-and-resume
 * identity, and every validation error path.  Exits 0 and prints "oracle ok"
 * when nothing fails; a sanitizer report aborts the process. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int m3ref_validate(int, int, int, int, int, int, const double*, const double*, const double*, const double*,
                   const double*, const double*, const double*, const double*, const double*, const double*);
int m3ref_scan(int, int, int, int, int, int, const double*, const double*, const double*, const double*,
               const double*, const double*, const double*, const double*, const double*, const double*,
               double*, double*, int);

static unsigned long long rng = 0x9e3779b97f4a7c15ull;
static double urand(void) {   /* xorshift64*, uniform in [0, 1) */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 9007199254740992.0;
}
static double* fill(size_t n, double lo, double hi) {
    double* p = (double*)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}
static int fails = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s\n", msg); ++fails; } } while (0)

static void run_case(int b, int L, int H, int P, int N, int R, int with_theta, int with_carry) {
    size_t tok = (size_t)b * L * H, bh = (size_t)b * H;
    double *x = fill(tok * R * P, -1, 1), *B = fill(tok * R * N, -0.3, 0.3), *C = fill(tok * R * N, -0.3, 0.3);
    double *dt = fill(tok, 0.01, 0.5), *A = fill(H, -2, -0.1), *lam = fill(tok, 0, 1);
    double* th = with_theta ? fill(tok * (N / 2), -1, 1) : NULL;
    double* h0 = with_carry ? fill(bh * N * P, -1, 1) : NULL;
    double* Bp = with_carry ? fill(bh * R * N, -0.3, 0.3) : NULL;
    double* xp = with_carry ? fill(bh * R * P, -1, 1) : NULL;
    double* y = (double*)calloc(tok * R * P + 1, sizeof(double));
    double* h = (double*)calloc(bh * N * P + 1, sizeof(double));
    CHECK(m3ref_scan(b, L, H, P, N, R, x, B, C, dt, A, lam, th, h0, Bp, xp, y, h, 1) == 0, "scan rc");
    for (size_t i = 0; i < tok * R * P; ++i) CHECK(isfinite(y[i]), "y finite");
    for (size_t i = 0; i < bh * N * P; ++i) CHECK(isfinite(h[i]), "h finite");
    if (b == 1 && L >= 2) {   /* split at L1 and resume: the same y and final state */
        int L1 = L / 2, L2 = L - L1;
        double* y1 = (double*)calloc((size_t)L1 * H * R * P + 1, sizeof(double));
        double* y2 = (double*)calloc((size_t)L2 * H * R * P + 1, sizeof(double));
        double* h1 = (double*)calloc(bh * N * P + 1, sizeof(double));
        double* h2 = (double*)calloc(bh * N * P + 1, sizeof(double));
        double* Bl = (double*)malloc((size_t)H * R * N * sizeof(double));
        double* xl = (double*)malloc((size_t)H * R * P * sizeof(double));
        CHECK(m3ref_scan(1, L1, H, P, N, R, x, B, C, dt, A, lam, th, h0, Bp, xp, y1, h1, 1) == 0, "first half");
        memcpy(Bl, B + (size_t)(L1 - 1) * H * R * N, (size_t)H * R * N * sizeof(double));
        memcpy(xl, x + (size_t)(L1 - 1) * H * R * P, (size_t)H * R * P * sizeof(double));
        CHECK(m3ref_scan(1, L2, H, P, N, R, x + (size_t)L1 * H * R * P, B + (size_t)L1 * H * R * N,
                         C + (size_t)L1 * H * R * N, dt + (size_t)L1 * H, A, lam + (size_t)L1 * H,
                         th ? th + (size_t)L1 * H * (N / 2) : NULL, h1, Bl, xl, y2, h2, 1) == 0, "second half");
        double err = 0, ref = 0;
        for (size_t i = 0; i < (size_t)L1 * H * R * P; ++i) { err = fmax(err, fabs(y1[i] - y[i])); ref = fmax(ref, fabs(y[i])); }
        for (size_t i = 0; i < (size_t)L2 * H * R * P; ++i) err = fmax(err, fabs(y2[i] - y[(size_t)L1 * H * R * P + i]));
        for (size_t i = 0; i < bh * N * P; ++i) err = fmax(err, fabs(h2[i] - h[i]));
        CHECK(err <= 1e-12 * (1 + ref), "split and resume");
        free(y1); free(y2); free(h1); free(h2); free(Bl); free(xl);
    }
    free(x); free(B); free(C); free(dt); free(A); free(lam); free(th); free(h0); free(Bp); free(xp); free(y); free(h);
}

static void validation_errors(void) {
    const int b = 1, L = 3, H = 2, P = 4, N = 4, R = 1;
    size_t tok = (size_t)b * L * H;
    double *x = fill(tok * R * P, -1, 1), *B = fill(tok * R * N, -1, 1), *C = fill(tok * R * N, -1, 1);
    double *dt = fill(tok, 0.1, 0.2), *A = fill(H, -1, -0.5), *lam = fill(tok, 0.2, 0.8), *th = fill(tok * N / 2, -1, 1);
    double* Bp = fill((size_t)b * H * R * N, -1, 1);
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 0, "valid");
    CHECK(m3ref_validate(b, L, H, 0, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 1, "bad dims");
    CHECK(m3ref_validate(b, L, H, P, 3, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 6, "odd N with theta");
    CHECK(m3ref_validate(b, L, H, P, N, R, NULL, B, C, dt, A, lam, th, NULL, NULL, NULL) == 7, "null x");
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, NULL, lam, th, NULL, NULL, NULL) == 7, "null A");
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, Bp, NULL) == 7, "B_prev without x_prev");
    dt[1] = -0.1;
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 3, "negative dt");
    dt[1] = 0.1; lam[2] = 1.5;
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 5, "lam range");
    lam[2] = 0.5; A[1] = 0.5;
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 4, "positive A");
    A[1] = -0.5; x[3] = NAN;
    CHECK(m3ref_validate(b, L, H, P, N, R, x, B, C, dt, A, lam, th, NULL, NULL, NULL) == 2, "non-finite x");
    free(x); free(B); free(C); free(dt); free(A); free(lam); free(th); free(Bp);
}

int main(void) {
    run_case(1, 64, 1, 16, 16, 1, 1, 0);
    run_case(2, 37, 3, 8, 32, 2, 1, 1);
    run_case(1, 9, 2, 4, 8, 4, 0, 1);
    run_case(1, 1, 2, 4, 8, 8, 1, 1);
    run_case(1, 0, 1, 4, 4, 1, 1, 1);
    run_case(0, 5, 2, 4, 4, 1, 1, 0);
    run_case(1, 17, 1, 2, 1, 1, 0, 1);   /* N = 1 without angles */
    validation_errors();
    if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
    printf("oracle ok\n");
    return 0;
}
