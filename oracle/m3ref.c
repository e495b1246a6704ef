/*
 * m3ref.c -- CPU oracle for the Mamba-3 SSM recurrence (float64, plain loops).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * What it computes (Mamba-3, "Mamba-3: Improved Sequence Modeling using State
 * Space Principles" explainer page, panels 1, 3 and 4; paper page Table 1
 * caption for the generalized recurrence):
 *
 *   For every (batch b, head h) independently, with the state H (N x P) and the
 *   previous token's write V_prev = B_prev X_prev^T (N x P):
 *     alpha_t = exp(dt_t * A_h)                  (exponential decay, Eq. 6)
 *     beta_t  = (1 - lam_t) * dt_t * alpha_t     (delayed-endpoint weight, Eq. 6)
 *     gamma_t = lam_t * dt_t                     (current-endpoint weight, Eq. 6)
 *     V_t     = B_t X_t^T                        (MIMO write, Sec. 3.3 Eq. 12-14)
 *     H_t     = alpha_t R(phi_t) H_{t-1} + beta_t R(phi_t) V_{t-1} + gamma_t V_t
 *               (physical frame: both the retained state and the previous write
 *                are rotated by the current step's angle before the new write is
 *                added; rotating-frame panel 3, Prop. 2 / Prop. 4)
 *     Y_t     = H_t^T C_t                        (readout after the update, Eq. 14)
 *   R(phi) acts on the adjacent row pairs (2k, 2k+1) of the state as
 *   [[cos, -sin], [sin, cos]] with the pair's own angle phi_t[k] (the real form of
 *   a complex state of N/2 entries, Prop. 2).
 *
 * Preconditions are validated like the explainer's coefficient helper (panel 1):
 * every value finite, dt >= 0, A <= 0, lam in [0, 1]; dstate even when angles
 * are given.  Violations return a nonzero code and write nothing.
 *
 * Layouts (row-major, contiguous):
 *   x [b,L,H,R,P]  B,C [b,L,H,R,N]  dt,lam [b,L,H]  A [H]  theta [b,L,H,N/2]
 *   h0, h_out [b,H,N,P]  B_prev [b,H,R,N]  x_prev [b,H,R,P]  y [b,L,H,R,P]
 * theta, h0, B_prev/x_prev may be NULL (no rotation / zero state / zero write).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum {
    M3REF_OK = 0,
    M3REF_BAD_DIMS = 1,
    M3REF_NONFINITE = 2,
    M3REF_NEG_DT = 3,
    M3REF_POS_A = 4,
    M3REF_LAM_RANGE = 5,
    M3REF_ODD_N = 6,
    M3REF_NULL = 7,
    M3REF_NOMEM = 8
};

static int all_finite(const double* v, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

int m3ref_validate(int batch, int seqlen, int nheads, int headdim, int dstate, int rank,
                   const double* x, const double* B, const double* C,
                   const double* dt, const double* A, const double* lam,
                   const double* theta, const double* h0,
                   const double* B_prev, const double* x_prev) {
    if (batch < 0 || seqlen < 0 || nheads < 0 || headdim < 1 || dstate < 1 || rank < 1)
        return M3REF_BAD_DIMS;
    if (theta && (dstate % 2)) return M3REF_ODD_N;
    size_t tok = (size_t)batch * seqlen * nheads;
    if (tok && (!x || !B || !C || !dt || !lam)) return M3REF_NULL;
    if (nheads && !A) return M3REF_NULL;
    if ((B_prev == NULL) != (x_prev == NULL)) return M3REF_NULL;
    if (tok) {
        if (!all_finite(x, tok * rank * headdim) || !all_finite(B, tok * rank * dstate) ||
            !all_finite(C, tok * rank * dstate) || !all_finite(dt, tok) || !all_finite(lam, tok))
            return M3REF_NONFINITE;
        if (theta && !all_finite(theta, tok * (dstate / 2))) return M3REF_NONFINITE;
    }
    if (nheads && !all_finite(A, (size_t)nheads)) return M3REF_NONFINITE;
    size_t bh = (size_t)batch * nheads;
    if (h0 && !all_finite(h0, bh * dstate * headdim)) return M3REF_NONFINITE;
    if (B_prev && (!all_finite(B_prev, bh * rank * dstate) || !all_finite(x_prev, bh * rank * headdim)))
        return M3REF_NONFINITE;
    for (size_t i = 0; i < tok; ++i) {
        if (dt[i] < 0) return M3REF_NEG_DT;
        if (lam[i] < 0 || lam[i] > 1) return M3REF_LAM_RANGE;
    }
    for (int h = 0; h < nheads; ++h)
        if (A[h] > 0) return M3REF_POS_A;
    return M3REF_OK;
}

/* Rotates every row pair (2k, 2k+1) of an N x P matrix by angle ang[k]. */
static void rotate_pairs(double* M, int N, int P, const double* ang) {
    for (int k = 0; k < N / 2; ++k) {
        double c = cos(ang[k]), s = sin(ang[k]);
        double* r0 = M + (size_t)(2 * k) * P;
        double* r1 = M + (size_t)(2 * k + 1) * P;
        for (int p = 0; p < P; ++p) {
            double u = r0[p], v = r1[p];
            r0[p] = c * u - s * v;
            r1[p] = s * u + c * v;
        }
    }
}

/* W = sum_r Bm[r, :]^T Xm[r, :]  (N x P), with Bm [R,N], Xm [R,P]. */
static void mimo_write(double* W, const double* Bm, const double* Xm, int N, int P, int R) {
    for (int n = 0; n < N; ++n)
        for (int p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int r = 0; r < R; ++r) acc += Bm[(size_t)r * N + n] * Xm[(size_t)r * P + p];
            W[(size_t)n * P + p] = acc;
        }
}

int m3ref_scan(int batch, int seqlen, int nheads, int headdim, int dstate, int rank,
               const double* x, const double* B, const double* C,
               const double* dt, const double* A, const double* lam,
               const double* theta, const double* h0,
               const double* B_prev, const double* x_prev,
               double* y, double* h_out, int nthreads) {
    int rc = m3ref_validate(batch, seqlen, nheads, headdim, dstate, rank, x, B, C, dt, A, lam,
                            theta, h0, B_prev, x_prev);
    if (rc) return rc;
    const int L = seqlen, H = nheads, P = headdim, N = dstate, R = rank;
    const size_t NP = (size_t)N * P;
    const long nbh = (long)batch * H;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel reduction(| : fail)
    {
        double* Hs = (double*)malloc(NP * sizeof(double));
        double* Vp = (double*)malloc(NP * sizeof(double));
        double* Vc = (double*)malloc(NP * sizeof(double));
        if (!Hs || !Vp || !Vc) {
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < nbh; ++bh) {
                const long b = bh / H;
                const int h = (int)(bh % H);
                /* initial state and previous write */
                if (h0) memcpy(Hs, h0 + (size_t)bh * NP, NP * sizeof(double));
                else memset(Hs, 0, NP * sizeof(double));
                if (B_prev)
                    mimo_write(Vp, B_prev + (size_t)bh * R * N, x_prev + (size_t)bh * R * P, N, P, R);
                else
                    memset(Vp, 0, NP * sizeof(double));
                for (int t = 0; t < L; ++t) {
                    const size_t tok = ((size_t)b * L + t) * H + h;
                    const double d = dt[tok], lm = lam[tok];
                    const double alpha = exp(d * A[h]);
                    const double beta = (1.0 - lm) * d * alpha;
                    const double gamma = lm * d;
                    mimo_write(Vc, B + tok * R * N, x + tok * R * P, N, P, R);
                    /* retained state and previous write, both rotated by phi_t */
                    for (size_t i = 0; i < NP; ++i) Hs[i] = alpha * Hs[i] + beta * Vp[i];
                    if (theta) rotate_pairs(Hs, N, P, theta + tok * (N / 2));
                    for (size_t i = 0; i < NP; ++i) Hs[i] += gamma * Vc[i];
                    /* readout Y_t = H_t^T C_t, stored [r][p] */
                    const double* Ct = C + tok * R * N;
                    double* yt = y + tok * R * P;
                    for (int r = 0; r < R; ++r)
                        for (int p = 0; p < P; ++p) {
                            double acc = 0.0;
                            for (int n = 0; n < N; ++n) acc += Hs[(size_t)n * P + p] * Ct[(size_t)r * N + n];
                            yt[(size_t)r * P + p] = acc;
                        }
                    double* sw = Vp; Vp = Vc; Vc = sw;
                }
                if (h_out) memcpy(h_out + (size_t)bh * NP, Hs, NP * sizeof(double));
            }
        }
        free(Hs); free(Vp); free(Vc);
    }
    return fail ? M3REF_NOMEM : M3REF_OK;
}

int m3ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
