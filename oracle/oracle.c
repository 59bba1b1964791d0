/*
 * oracle.c -- fp64 sequential reference for the linear-recurrence scans.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Loaded by tests, the smoke check and
 * the CPU-baseline leg of the benchmark; never by the product path.
 *
 * Every function is the plain definition of its op, taken from the minGRU
 * documentation page "Triton kernels", section "Kernel entry points".  There is
 * no blocking, no chunking and no reassociation: one channel (or one head) is
 * walked through time, one step after another, exactly as the recurrence reads.
 * Independent channels/heads are spread over OpenMP threads; that only changes
 * which core computes a channel, never the arithmetic inside it.
 *
 * The two backward functions are gradients.  The page fixes only their contract
 * (inputs, outputs, and that the outputs are the gradients with respect to the
 * forward inputs); the formulas used here
 * are the chain rule applied to the forward definitions, derived step by step in
 * the comments and pinned by finite differences and brute-force Jacobians in
 * tests/test_oracle.py.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int lrs_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the independent channels or heads of later calls (timing of the
 * oracle at one thread and at all host threads; the arithmetic per channel is
 * the same either way). */
void lrs_oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

/* Flat index of element (b, t, d) of a contiguous (B, T, D) array. */
static int64_t idx3(int64_t b, int64_t t, int64_t d, int64_t T, int64_t D) {
    return (b * T + t) * D + d;
}

/* ------------------------------------------------------------------------- */
/* linear_scan_fwd  ("Triton kernels" page, Kernel entry points:             */
/* linear_scan_fwd).  For each channel (b, d):                               */
/*     A_0 = 1, h_0 = 0;  A_t = a_t * A_{t-1};  h_t = a_t * h_{t-1} + b_t;    */
/*     outputs A_t and Bc_t = h_t for t = 1..T.                              */
/* ------------------------------------------------------------------------- */
void lrs_oracle_linear_fwd(int64_t B, int64_t T, int64_t D,
                           const double *a, const double *b,
                           double *A, double *Bc) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double A_prev = 1.0; /* A_0 */
        double h_prev = 0.0; /* h_0 = 0: Bc is the zero-initial-state solution */
        for (int64_t t = 0; t < T; ++t) {
            int64_t i = idx3(bb, t, dd, T, D);
            double A_t = a[i] * A_prev;
            double h_t = a[i] * h_prev + b[i];
            A[i] = A_t;
            Bc[i] = h_t;
            A_prev = A_t;
            h_prev = h_t;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* linear_scan_bwd  ("Triton kernels" page, Kernel entry points:             */
/* linear_scan_bwd).  Loss L = sum_t gA_t*A_t + gBc_t*Bc_t.                  */
/*                                                                           */
/* Write lam_t = dL/dh_t and mu_t = dL/dA_t (total derivatives through all   */
/* later steps).  h_{t+1} = a_{t+1} h_t + b_{t+1} and A_{t+1} = a_{t+1} A_t,  */
/* so                                                                        */
/*     lam_t = gBc_t + a_{t+1} * lam_{t+1},   mu_t = gA_t + a_{t+1} * mu_{t+1}*/
/* with nothing after T (a_{T+1} := 0).  Step t uses a_t as                  */
/*     dh_t/da_t = h_{t-1},  dA_t/da_t = A_{t-1},  dh_t/db_t = 1,            */
/* hence db_t = lam_t and da_t = lam_t * Bc_{t-1} + mu_t * A_{t-1}, with     */
/* Bc_0 = h_0 = 0 and A_0 = 1.  A and Bc are read from the arguments.        */
/* ------------------------------------------------------------------------- */
void lrs_oracle_linear_bwd(int64_t B, int64_t T, int64_t D,
                           const double *a, const double *A, const double *Bc,
                           const double *gA, const double *gBc,
                           double *da, double *db) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double lam = 0.0, mu = 0.0; /* lam_{T+1} = mu_{T+1} = 0 */
        double a_next = 0.0;        /* a_{T+1} := 0 */
        for (int64_t t = T - 1; t >= 0; --t) {
            int64_t i = idx3(bb, t, dd, T, D);
            lam = gBc[i] + a_next * lam;
            mu = gA[i] + a_next * mu;
            double A_prev = (t > 0) ? A[idx3(bb, t - 1, dd, T, D)] : 1.0;
            double Bc_prev = (t > 0) ? Bc[idx3(bb, t - 1, dd, T, D)] : 0.0;
            db[i] = lam;
            da[i] = lam * Bc_prev + mu * A_prev;
            a_next = a[i];
        }
    }
}

/* ------------------------------------------------------------------------- */
/* parallel_scan_log_fwd  ("Triton kernels" page, Kernel entry points:       */
/* parallel_scan_log_fwd).  log_values slot 0 holds log h_0, slots 1..T hold */
/* log b_t; log_coeffs row t-1 holds log a_t.  The states are those of the   */
/* same first-order recurrence, h_t = a_t h_{t-1} + b_t, returned for t=1..T.*/
/* Plain definition, in linear space.                                         */
/* ------------------------------------------------------------------------- */
void lrs_oracle_scan_log_fwd(int64_t B, int64_t T, int64_t D,
                             const double *log_coeffs, const double *log_values,
                             double *h) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double h_prev = exp(log_values[idx3(bb, 0, dd, T + 1, D)]); /* h_0 */
        for (int64_t t = 1; t <= T; ++t) {
            double a_t = exp(log_coeffs[idx3(bb, t - 1, dd, T, D)]);
            double b_t = exp(log_values[idx3(bb, t, dd, T + 1, D)]);
            double h_t = a_t * h_prev + b_t;
            h[idx3(bb, t - 1, dd, T, D)] = h_t;
            h_prev = h_t;
        }
    }
}

/* logaddexp(x, y) = log(exp(x) + exp(y)), evaluated as max + log1p(exp(-|x-y|)).
 * log(0 + 0) = -inf is returned for two -inf arguments; NaN propagates. */
static double logaddexp(double x, double y) {
    if (isnan(x) || isnan(y)) return x + y;
    double m = (x > y) ? x : y;
    if (isinf(m)) return m; /* -inf,-inf -> -inf; any +inf -> +inf */
    double lo = (x > y) ? y : x;
    return m + log1p(exp(lo - m));
}

void lrs_oracle_scan_log_fwd_logspace(int64_t B, int64_t T, int64_t D,
                                      const double *log_coeffs,
                                      const double *log_values, double *h) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double lh = log_values[idx3(bb, 0, dd, T + 1, D)]; /* log h_0 */
        for (int64_t t = 1; t <= T; ++t) {
            double lc = log_coeffs[idx3(bb, t - 1, dd, T, D)];
            double lv = log_values[idx3(bb, t, dd, T + 1, D)];
            lh = logaddexp(lc + lh, lv); /* log(a_t h_{t-1} + b_t) */
            h[idx3(bb, t - 1, dd, T, D)] = exp(lh);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Gradient of parallel_scan_log_fwd.  The page ships the log-space scan as  */
/* a forward op only ("Triton kernels" page, Kernel entry points:            */
/* parallel_scan_log_fwd); this is the adjoint of that forward definition.   */
/* With a_t = exp(log a_t), b_t = exp(log b_t), h_0 = exp(log h_0) and g_t = */
/* dL/dh_t the upstream gradient of output t, the total derivative          */
/*     lam_t = dL/dh_t (through every later state)                           */
/*           = g_t + a_{t+1} lam_{t+1},   a_{T+1} = 0,                        */
/* and since h_t = a_t h_{t-1} + b_t:                                         */
/*     d log a_t = lam_t * dh_t/dlog a_t = lam_t a_t h_{t-1}   (t = 1..T),   */
/*     d log b_t = lam_t * dh_t/dlog b_t = lam_t b_t           (t = 1..T),   */
/*     d log h_0 = (dL/dh_0) h_0 = a_1 lam_1 h_0.                             */
/* h_1..h_T are taken from the given forward output h (not recomputed);     */
/* h_0 comes from log_values slot 0.  dlog_values has slot 0 and slots 1..T */
/* like log_values.                                                           */
/* ------------------------------------------------------------------------- */
void lrs_oracle_scan_log_bwd(int64_t B, int64_t T, int64_t D,
                             const double *log_coeffs, const double *log_values,
                             const double *h, const double *g,
                             double *dlog_coeffs, double *dlog_values) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double h0 = exp(log_values[idx3(bb, 0, dd, T + 1, D)]);
        double lam = 0.0, a_next = 0.0; /* lam_{T+1} = 0, a_{T+1} = 0 */
        for (int64_t t = T; t >= 1; --t) {
            int64_t i = idx3(bb, t - 1, dd, T, D);
            double a_t = exp(log_coeffs[i]);
            double b_t = exp(log_values[idx3(bb, t, dd, T + 1, D)]);
            double h_prev = (t > 1) ? h[idx3(bb, t - 2, dd, T, D)] : h0;
            lam = g[i] + a_next * lam;
            dlog_coeffs[i] = lam * a_t * h_prev;
            dlog_values[idx3(bb, t, dd, T + 1, D)] = lam * b_t;
            a_next = a_t;
        }
        /* lam now holds lam_1 and a_next holds a_1 (0 when T = 0) */
        dlog_values[idx3(bb, 0, dd, T + 1, D)] = a_next * lam * h0;
    }
}

/* ------------------------------------------------------------------------- */
/* k x k helpers on row-major dense matrices (plain triple loops).            */
/* ------------------------------------------------------------------------- */

/* C (r x c) = X (r x m) @ Y (m x c) */
static void matmul(const double *X, const double *Y, double *C,
                   int64_t r, int64_t m, int64_t c) {
    for (int64_t i = 0; i < r; ++i)
        for (int64_t j = 0; j < c; ++j) {
            double s = 0.0;
            for (int64_t p = 0; p < m; ++p) s += X[i * m + p] * Y[p * c + j];
            C[i * c + j] = s;
        }
}

/* C (r x c) = X^T @ Y, X is (m x r), Y is (m x c) */
static void matmul_tn(const double *X, const double *Y, double *C,
                      int64_t r, int64_t m, int64_t c) {
    for (int64_t i = 0; i < r; ++i)
        for (int64_t j = 0; j < c; ++j) {
            double s = 0.0;
            for (int64_t p = 0; p < m; ++p) s += X[p * r + i] * Y[p * c + j];
            C[i * c + j] = s;
        }
}

/* C (r x c) = X @ Y^T, X is (r x m), Y is (c x m) */
static void matmul_nt(const double *X, const double *Y, double *C,
                      int64_t r, int64_t m, int64_t c) {
    for (int64_t i = 0; i < r; ++i)
        for (int64_t j = 0; j < c; ++j) {
            double s = 0.0;
            for (int64_t p = 0; p < m; ++p) s += X[i * m + p] * Y[j * m + p];
            C[i * c + j] = s;
        }
}

/* Offset of matrix (b, t, head) in a (B, T, n, r, c) array. */
static int64_t mat_off(int64_t b, int64_t t, int64_t hd, int64_t T, int64_t n,
                       int64_t r, int64_t c) {
    return ((b * T + t) * n + hd) * r * c;
}

/* ------------------------------------------------------------------------- */
/* affine_scan_fwd  ("Triton kernels" page, Kernel entry points:             */
/* affine_scan_fwd).  For each head (b, head):                               */
/*     Abar_0 = I, H_0 = 0;                                                  */
/*     Abar_t = A_t @ Abar_{t-1}      (composition A_current @ A_earlier)    */
/*     H_t    = A_t @ H_{t-1} + Bm_t  (Bbar_t = H_t, the H_0 = 0 solution)   */
/* ------------------------------------------------------------------------- */
void lrs_oracle_affine_fwd(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                           const double *A, const double *Bm,
                           double *Abar, double *Bbar) {
    int64_t heads = B * n;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t hidx = 0; hidx < heads; ++hidx) {
        int64_t bb = hidx / n, hd = hidx % n;
        double *P = (double *)malloc(sizeof(double) * k * k);    /* Abar_{t-1} */
        double *H = (double *)malloc(sizeof(double) * k * v);    /* H_{t-1} */
        double *Pn = (double *)malloc(sizeof(double) * k * k);
        double *Hn = (double *)malloc(sizeof(double) * k * v);
        for (int64_t i = 0; i < k; ++i)
            for (int64_t j = 0; j < k; ++j) P[i * k + j] = (i == j) ? 1.0 : 0.0;
        for (int64_t i = 0; i < k * v; ++i) H[i] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double *At = A + mat_off(bb, t, hd, T, n, k, k);
            const double *Bt = Bm + mat_off(bb, t, hd, T, n, k, v);
            matmul(At, P, Pn, k, k, k); /* A_t @ Abar_{t-1} */
            matmul(At, H, Hn, k, k, v); /* A_t @ H_{t-1} */
            for (int64_t i = 0; i < k * v; ++i) Hn[i] += Bt[i];
            memcpy(P, Pn, sizeof(double) * k * k);
            memcpy(H, Hn, sizeof(double) * k * v);
            memcpy(Abar + mat_off(bb, t, hd, T, n, k, k), P, sizeof(double) * k * k);
            memcpy(Bbar + mat_off(bb, t, hd, T, n, k, v), H, sizeof(double) * k * v);
        }
        free(P); free(H); free(Pn); free(Hn);
    }
}

/* ------------------------------------------------------------------------- */
/* affine_scan_bwd  ("Triton kernels" page, Kernel entry points:             */
/* affine_scan_bwd).  Loss L = sum_t <gAbar_t, Abar_t> + <gBbar_t, Bbar_t>.   */
/*                                                                           */
/* Let M_t = dL/dAbar_t and Lam_t = dL/dH_t (total derivatives).  Since      */
/* Abar_{t+1} = A_{t+1} Abar_t and H_{t+1} = A_{t+1} H_t + Bm_{t+1},          */
/*     M_t   = gAbar_t + A_{t+1}^T M_{t+1},                                  */
/*     Lam_t = gBbar_t + A_{t+1}^T Lam_{t+1},   nothing after T.             */
/* Step t uses A_t and Bm_t as Abar_t = A_t Abar_{t-1}, H_t = A_t H_{t-1}+Bm_t*/
/* hence dB_t = Lam_t and dA_t = M_t Abar_{t-1}^T + Lam_t Bbar_{t-1}^T, with */
/* Abar_0 = I and Bbar_0 = 0.  Abar and Bbar are read from the arguments.    */
/* ------------------------------------------------------------------------- */
void lrs_oracle_affine_bwd(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                           const double *A, const double *Abar, const double *Bbar,
                           const double *gAbar, const double *gBbar,
                           double *dA, double *dB) {
    int64_t heads = B * n;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t hidx = 0; hidx < heads; ++hidx) {
        int64_t bb = hidx / n, hd = hidx % n;
        double *M = (double *)malloc(sizeof(double) * k * k);   /* M_{t+1} */
        double *L = (double *)malloc(sizeof(double) * k * v);   /* Lam_{t+1} */
        double *Mn = (double *)malloc(sizeof(double) * k * k);
        double *Ln = (double *)malloc(sizeof(double) * k * v);
        double *Pprev = (double *)malloc(sizeof(double) * k * k); /* Abar_{t-1} */
        double *Hprev = (double *)malloc(sizeof(double) * k * v); /* Bbar_{t-1} */
        double *T1 = (double *)malloc(sizeof(double) * k * k);
        double *T2 = (double *)malloc(sizeof(double) * k * k);
        for (int64_t i = 0; i < k * k; ++i) M[i] = 0.0;
        for (int64_t i = 0; i < k * v; ++i) L[i] = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const double *gAt = gAbar + mat_off(bb, t, hd, T, n, k, k);
            const double *gBt = gBbar + mat_off(bb, t, hd, T, n, k, v);
            if (t == T - 1) {
                /* A_{T+1} := 0: nothing flows back from beyond the last step. */
                memcpy(Mn, gAt, sizeof(double) * k * k);
                memcpy(Ln, gBt, sizeof(double) * k * v);
            } else {
                const double *Anext = A + mat_off(bb, t + 1, hd, T, n, k, k);
                matmul_tn(Anext, M, Mn, k, k, k); /* A_{t+1}^T M_{t+1} */
                matmul_tn(Anext, L, Ln, k, k, v); /* A_{t+1}^T Lam_{t+1} */
                for (int64_t i = 0; i < k * k; ++i) Mn[i] += gAt[i];
                for (int64_t i = 0; i < k * v; ++i) Ln[i] += gBt[i];
            }
            memcpy(M, Mn, sizeof(double) * k * k);
            memcpy(L, Ln, sizeof(double) * k * v);

            if (t > 0) {
                memcpy(Pprev, Abar + mat_off(bb, t - 1, hd, T, n, k, k), sizeof(double) * k * k);
                memcpy(Hprev, Bbar + mat_off(bb, t - 1, hd, T, n, k, v), sizeof(double) * k * v);
            } else {
                for (int64_t i = 0; i < k; ++i)
                    for (int64_t j = 0; j < k; ++j) Pprev[i * k + j] = (i == j) ? 1.0 : 0.0;
                for (int64_t i = 0; i < k * v; ++i) Hprev[i] = 0.0;
            }
            matmul_nt(M, Pprev, T1, k, k, k); /* M_t Abar_{t-1}^T */
            matmul_nt(L, Hprev, T2, k, v, k); /* Lam_t Bbar_{t-1}^T */
            double *dAt = dA + mat_off(bb, t, hd, T, n, k, k);
            for (int64_t i = 0; i < k * k; ++i) dAt[i] = T1[i] + T2[i];
            memcpy(dB + mat_off(bb, t, hd, T, n, k, v), L, sizeof(double) * k * v);
        }
        free(M); free(L); free(Mn); free(Ln); free(Pprev); free(Hprev); free(T1); free(T2);
    }
}

/* ------------------------------------------------------------------------- */
/* Given initial state.  The pages define Bc and Bbar as the solutions from  */
/* a zero state ("Triton kernels" page, Kernel entry points: linear_scan_fwd,*/
/* affine_scan_fwd); a caller with an initial state h_0 (or H_0) composes    */
/* h_t = A_t h_0 + Bc_t itself.  These four functions run the same           */
/* recurrences from a given h_0 / H_0 and return the states directly, with   */
/* the gradient of h_0 / H_0 in the backward.  A NULL h0 (H0) means zero.    */
/* ------------------------------------------------------------------------- */

/* h_t = a_t h_{t-1} + b_t from h_0 = h0[b, d]; A_t = a_t A_{t-1}, A_0 = 1.   */
void lrs_oracle_linear_fwd_h0(int64_t B, int64_t T, int64_t D,
                              const double *a, const double *b, const double *h0,
                              double *A, double *H) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double A_prev = 1.0;
        double h_prev = h0 ? h0[bb * D + dd] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            int64_t i = idx3(bb, t, dd, T, D);
            A_prev = a[i] * A_prev;
            h_prev = a[i] * h_prev + b[i];
            A[i] = A_prev;
            H[i] = h_prev;
        }
    }
}

/* Gradient of the above for L = sum_t gA_t A_t + gH_t H_t: the recurrences  */
/* of lrs_oracle_linear_bwd with H in place of Bc, H_0 = h_0 instead of 0 in */
/* da_1 = lam_1 h_0 + mu_1, and dh0 = dL/dh_0 = a_1 lam_1 (zero when T = 0). */
void lrs_oracle_linear_bwd_h0(int64_t B, int64_t T, int64_t D,
                              const double *a, const double *A, const double *H,
                              const double *h0, const double *gA, const double *gH,
                              double *da, double *db, double *dh0) {
    int64_t channels = B * D;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t c = 0; c < channels; ++c) {
        int64_t bb = c / D, dd = c % D;
        double lam = 0.0, mu = 0.0, a_next = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            int64_t i = idx3(bb, t, dd, T, D);
            lam = gH[i] + a_next * lam;
            mu = gA[i] + a_next * mu;
            double A_prev = (t > 0) ? A[idx3(bb, t - 1, dd, T, D)] : 1.0;
            double H_prev = (t > 0) ? H[idx3(bb, t - 1, dd, T, D)] : (h0 ? h0[bb * D + dd] : 0.0);
            db[i] = lam;
            da[i] = lam * H_prev + mu * A_prev;
            a_next = a[i];
        }
        dh0[bb * D + dd] = a_next * lam; /* a_1 lam_1; a_next stays 0 when T = 0 */
    }
}

/* X_t = A_t X_{t-1} + [0 | Bm_t] from X_0 = [I | H0[b, head]]: Abar_t as in */
/* lrs_oracle_affine_fwd, H_t = A_t H_{t-1} + Bm_t from H_0 = H0.             */
void lrs_oracle_affine_fwd_h0(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                              const double *A, const double *Bm, const double *H0,
                              double *Abar, double *H) {
    int64_t heads = B * n;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t hidx = 0; hidx < heads; ++hidx) {
        int64_t bb = hidx / n, hd = hidx % n;
        double *P = (double *)malloc(sizeof(double) * k * k);
        double *Hc = (double *)malloc(sizeof(double) * k * v);
        double *Pn = (double *)malloc(sizeof(double) * k * k);
        double *Hn = (double *)malloc(sizeof(double) * k * v);
        for (int64_t i = 0; i < k; ++i)
            for (int64_t j = 0; j < k; ++j) P[i * k + j] = (i == j) ? 1.0 : 0.0;
        for (int64_t i = 0; i < k * v; ++i) Hc[i] = H0 ? H0[hidx * k * v + i] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double *At = A + mat_off(bb, t, hd, T, n, k, k);
            const double *Bt = Bm + mat_off(bb, t, hd, T, n, k, v);
            matmul(At, P, Pn, k, k, k);
            matmul(At, Hc, Hn, k, k, v);
            for (int64_t i = 0; i < k * v; ++i) Hn[i] += Bt[i];
            memcpy(P, Pn, sizeof(double) * k * k);
            memcpy(Hc, Hn, sizeof(double) * k * v);
            memcpy(Abar + mat_off(bb, t, hd, T, n, k, k), P, sizeof(double) * k * k);
            memcpy(H + mat_off(bb, t, hd, T, n, k, v), Hc, sizeof(double) * k * v);
        }
        free(P); free(Hc); free(Pn); free(Hn);
    }
}

/* Gradient of the above: the recurrences of lrs_oracle_affine_bwd with H in  */
/* place of Bbar, H_0 = H0 instead of 0 in dA_1 = M_1 + Lam_1 H0^T, and        */
/* dH0 = dL/dH_0 = A_1^T Lam_1 (zero when T = 0).                             */
void lrs_oracle_affine_bwd_h0(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                              const double *A, const double *Abar, const double *H,
                              const double *H0, const double *gAbar, const double *gH,
                              double *dA, double *dB, double *dH0) {
    int64_t heads = B * n;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int64_t hidx = 0; hidx < heads; ++hidx) {
        int64_t bb = hidx / n, hd = hidx % n;
        double *M = (double *)malloc(sizeof(double) * k * k);
        double *L = (double *)malloc(sizeof(double) * k * v);
        double *Mn = (double *)malloc(sizeof(double) * k * k);
        double *Ln = (double *)malloc(sizeof(double) * k * v);
        double *Pprev = (double *)malloc(sizeof(double) * k * k);
        double *Hprev = (double *)malloc(sizeof(double) * k * v);
        double *T1 = (double *)malloc(sizeof(double) * k * k);
        double *T2 = (double *)malloc(sizeof(double) * k * k);
        for (int64_t i = 0; i < k * k; ++i) M[i] = 0.0;
        for (int64_t i = 0; i < k * v; ++i) L[i] = 0.0;
        for (int64_t t = T - 1; t >= 0; --t) {
            const double *gAt = gAbar + mat_off(bb, t, hd, T, n, k, k);
            const double *gHt = gH + mat_off(bb, t, hd, T, n, k, v);
            if (t == T - 1) {
                memcpy(Mn, gAt, sizeof(double) * k * k);
                memcpy(Ln, gHt, sizeof(double) * k * v);
            } else {
                const double *Anext = A + mat_off(bb, t + 1, hd, T, n, k, k);
                matmul_tn(Anext, M, Mn, k, k, k);
                matmul_tn(Anext, L, Ln, k, k, v);
                for (int64_t i = 0; i < k * k; ++i) Mn[i] += gAt[i];
                for (int64_t i = 0; i < k * v; ++i) Ln[i] += gHt[i];
            }
            memcpy(M, Mn, sizeof(double) * k * k);
            memcpy(L, Ln, sizeof(double) * k * v);
            if (t > 0) {
                memcpy(Pprev, Abar + mat_off(bb, t - 1, hd, T, n, k, k), sizeof(double) * k * k);
                memcpy(Hprev, H + mat_off(bb, t - 1, hd, T, n, k, v), sizeof(double) * k * v);
            } else {
                for (int64_t i = 0; i < k; ++i)
                    for (int64_t j = 0; j < k; ++j) Pprev[i * k + j] = (i == j) ? 1.0 : 0.0;
                for (int64_t i = 0; i < k * v; ++i) Hprev[i] = H0 ? H0[hidx * k * v + i] : 0.0;
            }
            matmul_nt(M, Pprev, T1, k, k, k);
            matmul_nt(L, Hprev, T2, k, v, k);
            double *dAt = dA + mat_off(bb, t, hd, T, n, k, k);
            for (int64_t i = 0; i < k * k; ++i) dAt[i] = T1[i] + T2[i];
            memcpy(dB + mat_off(bb, t, hd, T, n, k, v), L, sizeof(double) * k * v);
        }
        /* dH0 = A_1^T Lam_1: L holds Lam_1 after the loop */
        double *dH = dH0 + hidx * k * v;
        if (T > 0)
            matmul_tn(A + mat_off(bb, 0, hd, T, n, k, k), L, dH, k, k, v);
        else
            for (int64_t i = 0; i < k * v; ++i) dH[i] = 0.0;
        free(M); free(L); free(Mn); free(Ln); free(Pprev); free(Hprev); free(T1); free(T2);
    }
}
