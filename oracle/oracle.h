/*
 * oracle.h -- fp64 sequential reference for the linear-recurrence scans.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the correctness oracle.  It may be loaded by
 * the test suite, by the smoke check and by the CPU-baseline leg of the benchmark,
 * and by nothing else.  It shares no code, header, table or helper with the HIP
 * library; the HIP library never calls it.
 *
 * Source of the definitions: the minGRU documentation page "Triton kernels"
 * (API reference of mingru.triton_scans), section "Kernel entry points", entries
 * linear_scan_fwd, linear_scan_bwd, parallel_scan_log_fwd, affine_scan_fwd and
 * affine_scan_bwd.  Each function below names the entry it follows.
 *
 * Conventions shared by every function:
 *   - every array is a contiguous, row-major fp64 buffer owned by the caller;
 *   - time step t (counted from 1 to T) is row t-1 of the T axis;
 *   - work is sequential in time; independent channels (or heads) may run on
 *     separate OpenMP threads, which does not change any result;
 *   - no function allocates device memory, none fails: sizes are trusted.
 *
 * Parity status: every function here is pinned by CPU tests against closed forms,
 * library routines, brute force on tiny inputs, finite differences and exact
 * rational arithmetic (tests/test_oracle.py).  None is "parity unpinned".
 */
#ifndef LRS_ORACLE_H
#define LRS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of OpenMP threads the oracle will use (1 when built without OpenMP). */
int lrs_oracle_num_threads(void);
void lrs_oracle_set_threads(int n);

/* linear_scan_fwd: a, b are (B,T,D).  A_t is the running product of a, Bc_t is
 * the h_0 = 0 solution of h_t = a_t*h_{t-1} + b_t.  Outputs (B,T,D). */
void lrs_oracle_linear_fwd(int64_t B, int64_t T, int64_t D,
                           const double *a, const double *b,
                           double *A, double *Bc);

/* linear_scan_bwd: gradients (da, db) of L = <gA, A> + <gBc, Bc> with respect to
 * the forward inputs a and b, reading the given a, A, Bc (not recomputed). */
void lrs_oracle_linear_bwd(int64_t B, int64_t T, int64_t D,
                           const double *a, const double *A, const double *Bc,
                           const double *gA, const double *gBc,
                           double *da, double *db);

/* parallel_scan_log_fwd: log_coeffs (B,T,D), log_values (B,T+1,D) with slot 0 =
 * log h_0 and slots 1..T = log b_t.  Writes h_1..h_T as (B,T,D).
 * Plain definition: h_t = exp(lc_t)*h_{t-1} + exp(lv_t), h_0 = exp(lv_0). */
void lrs_oracle_scan_log_fwd(int64_t B, int64_t T, int64_t D,
                             const double *log_coeffs, const double *log_values,
                             double *h);

/* Same result computed a second, independent way: entirely in log space with
 * log h_t = logaddexp(lc_t + log h_{t-1}, lv_t), then h_t = exp(log h_t). */
void lrs_oracle_scan_log_fwd_logspace(int64_t B, int64_t T, int64_t D,
                                      const double *log_coeffs,
                                      const double *log_values, double *h);

/* Gradient of the log-space scan: dlog_coeffs (B,T,D) and dlog_values
 * (B,T+1,D, slot 0 = d log h_0) from log_coeffs, log_values, the forward
 * output h (B,T,D) and the upstream gradient g = dL/dh (B,T,D). */
void lrs_oracle_scan_log_bwd(int64_t B, int64_t T, int64_t D,
                             const double *log_coeffs, const double *log_values,
                             const double *h, const double *g,
                             double *dlog_coeffs, double *dlog_values);

/* affine_scan_fwd: A is (B,T,n,k,k), Bm is (B,T,n,k,v).  Abar_t = A_t @ Abar_{t-1}
 * (A_current @ A_earlier) with Abar_0 = I; Bbar_t = A_t @ Bbar_{t-1} + Bm_t with
 * Bbar_0 = 0.  Outputs have the input shapes. */
void lrs_oracle_affine_fwd(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                           const double *A, const double *Bm,
                           double *Abar, double *Bbar);

/* affine_scan_bwd: gradients (dA, dB) of L = <gAbar, Abar> + <gBbar, Bbar> with
 * respect to the forward inputs A and Bm, reading the given A, Abar, Bbar. */
void lrs_oracle_affine_bwd(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                           const double *A, const double *Abar, const double *Bbar,
                           const double *gAbar, const double *gBbar,
                           double *dA, double *dB);

/* Initial state (NULL = zero): states from h0 (B,D) / H0 (B,n,k,v) and the
 * gradients including dh0 / dH0.  H replaces Bc / Bbar. */
void lrs_oracle_linear_fwd_h0(int64_t B, int64_t T, int64_t D,
                              const double *a, const double *b, const double *h0,
                              double *A, double *H);
void lrs_oracle_linear_bwd_h0(int64_t B, int64_t T, int64_t D,
                              const double *a, const double *A, const double *H,
                              const double *h0, const double *gA, const double *gH,
                              double *da, double *db, double *dh0);
void lrs_oracle_affine_fwd_h0(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                              const double *A, const double *Bm, const double *H0,
                              double *Abar, double *H);
void lrs_oracle_affine_bwd_h0(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                              const double *A, const double *Abar, const double *H,
                              const double *H0, const double *gAbar, const double *gH,
                              double *dA, double *dB, double *dH0);

#ifdef __cplusplus
}
#endif

#endif /* LRS_ORACLE_H */
