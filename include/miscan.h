/*
 * miscan.h -- C ABI of libmiscan.so: parallel prefix scans of the first-order
 * affine recurrence h_t = a_t * h_{t-1} + b_t and its k x k matrix form, as
 * hand-written HIP kernels for gfx950 (MI355X, CDNA4), one GPU.
 *
 * The operations are those of the minGRU documentation page "Triton kernels"
 * (API reference of mingru.triton_scans), section "Kernel entry points":
 * linear_scan_fwd/bwd, parallel_scan_log_fwd and affine_scan_fwd/bwd.  Each
 * entry point below names the entry it implements.
 *
 * Common contract
 * ---------------
 *  - Tensors are device pointers to contiguous row-major storage.  Time is the
 *    second axis: (B, T, D) for the channel scans, (B, T, n, r, c) for the k x k
 *    scan.  Step t = 1..T of the recurrence is row t-1.
 *  - Outputs have the shape and dtype of the corresponding input.  With bf16
 *    or fp16 storage all arithmetic is fp32; results are rounded to the
 *    storage type (nearest-even) once, on store.  Every output element is
 *    written.
 *  - Ownership: the caller allocates every input, output and the workspace.  The
 *    library keeps no device memory and no state between calls, and never
 *    synchronises: a call enqueues its kernels on `stream` and returns.
 *  - Workspace: at least the bytes reported by the matching *_workspace query,
 *    256-byte aligned, contents need not be initialised (the call clears what
 *    it uses, on `stream`, before its scan kernel).  One workspace must not be
 *    used by two calls that may run concurrently (e.g. on two streams).  Word 1
 *    (bytes 4..7) counts cross-workgroup waits that hit their spin limit during
 *    the last call; it is 0 after every correct run.
 *  - Errors: every check runs before anything is enqueued; on any status other
 *    than MI_OK nothing was launched, except MI_ERR_LAUNCH, which reports that
 *    the HIP runtime refused a launch.  A problem with a zero-sized axis returns
 *    MI_OK without launching.  Inputs and outputs must not overlap.  There is no
 *    fallback to any other implementation.
 *  - Sizes are int64.  Element pointers must be aligned to their element size;
 *    wider alignment (16 bytes) and D (or k, v) divisible by the vector width
 *    select the vectorised kernels, other layouts run narrower ones.
 */
#ifndef MISCAN_H
#define MISCAN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MI_OK = 0,
    MI_ERR_INVALID_ARG = 1, /* null pointer, negative size, byte-size overflow,
                               misaligned element pointer, overlapping buffers */
    MI_ERR_UNSUPPORTED = 2, /* outside the envelope: k not in [1,16], v not in
                               [1,128], or a dtype not built for the op */
    MI_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than the query says */
    MI_ERR_LAUNCH = 4,      /* the HIP runtime reported an error at launch */
    MI_ERR_DEVICE = 5,      /* no usable gfx950 device */
    MI_ERR_CAPACITY = 6     /* the problem needs more than the fixed scratch of
                               mi_linear_scan_fwd_noalloc */
} mi_status;

typedef enum {
    MI_F32 = 0,  /* IEEE binary32 storage */
    MI_BF16 = 1, /* bfloat16 storage, fp32 arithmetic */
    MI_F16 = 2   /* IEEE binary16 storage, fp32 arithmetic */
} mi_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char *mi_status_string(mi_status s);

/* Analogue of the page's available() probe ("Triton kernels", Availability and
 * registry): MI_OK if `device` is a gfx950 GPU this library can launch on,
 * otherwise MI_ERR_DEVICE with a reason copied into `reason` (may be NULL). */
mi_status mi_device_check(int device, char *reason, size_t reason_len);

/* ------------------------------------------------------------------------ */
/* k = 1 channel scan ("Triton kernels", Kernel entry points:               */
/* linear_scan_fwd, linear_scan_bwd).  Dtypes: MI_F32, MI_BF16, MI_F16.     */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for mi_linear_scan_fwd / mi_linear_scan_bwd on (B, T, D). */
size_t mi_linear_scan_workspace(int64_t B, int64_t T, int64_t D, mi_dtype dt);

/* linear_scan_fwd: a, b (B,T,D) -> A (running product of a) and Bc (the h_0 = 0
 * solution of h_t = a_t h_{t-1} + b_t), both (B,T,D). */
mi_status mi_linear_scan_fwd(const void *a, const void *b, void *A, void *Bc,
                             int64_t B, int64_t T, int64_t D, mi_dtype dt,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* linear_scan_bwd: reads the forward input a, the forward outputs A, Bc and the
 * upstream grads gA, gBc (all (B,T,D)); writes da, db (B,T,D), the grads of
 * <gA, A> + <gBc, Bc> with respect to a and b.  A and Bc are used as given:
 * da_t = lam_t Bc_{t-1} + mu_t A_{t-1}, db_t = lam_t, with
 * lam_t = gBc_t + a_{t+1} lam_{t+1}, mu_t = gA_t + a_{t+1} mu_{t+1},
 * a_{T+1} = 0, A_0 = 1, Bc_0 = 0. */
mi_status mi_linear_scan_bwd(const void *a, const void *A, const void *Bc,
                             const void *gA, const void *gBc, void *da, void *db,
                             int64_t B, int64_t T, int64_t D, mi_dtype dt,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* The same forward as mi_linear_scan_fwd, through an entry point that
 * allocates nothing and takes no workspace.  For callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The look-back workspace is a file-scope device array
 * of MI_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call makes no hipMalloc/hipFree and no allocating library
 * call.  Its device address is looked up (hipGetSymbolAddress) on the first
 * call on each device, which must be the current device and the stream's.
 * The array keeps the last call's contents; each call clears what must start
 * at zero, on `stream`, before its scan kernel.  Every call on one GPU uses
 * the same array: calls that may overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Same dtypes, layouts,
 * results and argument checks as mi_linear_scan_fwd; a problem whose
 * workspace exceeds the array returns MI_ERR_CAPACITY before anything is
 * enqueued.  72 MiB covers the forward of 2^28 channel-steps in either dtype
 * (e.g. B=8, T=8192, D=4096), about 4.2 bytes of scratch per 16 channel-steps. */
#define MI_NOALLOC_SCRATCH_BYTES (72u << 20)
mi_status mi_linear_scan_fwd_noalloc(const void *a, const void *b, void *A, void *Bc,
                                     int64_t B, int64_t T, int64_t D, mi_dtype dt,
                                     hipStream_t stream);

/* Scans from a given initial state.  The page's linear_scan_fwd returns Bc,
 * the solution from h_0 = 0, and leaves the initial state to the caller
 * (h_t = A_t h_0 + Bc_t).  These two calls take h_0 directly; they are what a
 * caller that carries state across calls (a sequence processed in pieces, or
 * split in time across devices) needs.
 *
 * mi_linear_scan_fwd_h0: h0 (B, D), or NULL for a zero state.  Writes A (the
 * running product, as mi_linear_scan_fwd) and H (B, T, D) with
 * H_t = a_t H_{t-1} + b_t, H_0 = h0.  The final state (A_T, H_T) is the last
 * row of A and H.
 * mi_linear_scan_bwd_h0: the gradient for L = <gA, A> + <gH, H>: da, db as
 * mi_linear_scan_bwd with H in place of Bc and h0 as the state before the
 * first step, and dh0 (B, D) = dL/dh0 = a_1 lam_1 (zero when T = 0).
 * Same dtypes, layouts, workspace (mi_linear_scan_workspace) and errors as the
 * calls above; h0 and dh0 must be aligned like the other tensors and must not
 * overlap outputs. */
mi_status mi_linear_scan_fwd_h0(const void *a, const void *b, const void *h0, void *A, void *H,
                                int64_t B, int64_t T, int64_t D, mi_dtype dt,
                                void *ws, size_t ws_bytes, hipStream_t stream);
mi_status mi_linear_scan_bwd_h0(const void *a, const void *A, const void *H, const void *h0,
                                const void *gA, const void *gH, void *da, void *db, void *dh0,
                                int64_t B, int64_t T, int64_t D, mi_dtype dt,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Log-space scan ("Triton kernels", Kernel entry points:                   */
/* parallel_scan_log_fwd).  Dtypes: MI_F32, MI_BF16, MI_F16.                */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for mi_scan_log_fwd and mi_scan_log_bwd on (B, T, D). */
size_t mi_scan_log_workspace(int64_t B, int64_t T, int64_t D, mi_dtype dt);

/* parallel_scan_log_fwd: log_coeffs (B,T,D) holds log a_t; log_values (B,T+1,D)
 * holds log h_0 in slot 0 and log b_t in slots 1..T.  Writes h_1..h_T as one
 * (B,T,D) tensor `h`, where h_t = a_t h_{t-1} + b_t.  The scan state is kept in
 * log space (log-sum-exp combine); only the stored states are exponentiated. */
mi_status mi_scan_log_fwd(const void *log_coeffs, const void *log_values, void *h,
                          int64_t B, int64_t T, int64_t D, mi_dtype dt,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Gradient of parallel_scan_log_fwd.  The page defines the log-space scan as
 * a forward op; this is the adjoint of that forward definition, for training
 * through it.  Inputs: log_coeffs (B,T,D) and log_values (B,T+1,D) as in the
 * forward, h (B,T,D) the forward output, g (B,T,D) the upstream gradient
 * dL/dh.  Outputs: dlog_coeffs (B,T,D) and dlog_values (B,T+1,D), slot 0 being
 * the gradient of log h_0:
 *     lam_t = g_t + a_{t+1} lam_{t+1} (a_{T+1} = 0),
 *     dlog_coeffs_t = lam_t a_t h_{t-1},  dlog_values_t = lam_t b_t (t >= 1),
 *     dlog_values_0 = a_1 lam_1 h_0,
 * with a = exp(log_coeffs), b and h_0 = exp(log_values), and h_{t-1} taken
 * from the given h (not recomputed).  lam runs in linear space (g is
 * signed).  Outputs must not overlap inputs or each other; all arithmetic is
 * fp32, storage as dt.  With T = 0 (and B, D > 0) the only output is slot 0 of
 * dlog_values, which is set to zero; the other pointers are not used. */
mi_status mi_scan_log_bwd(const void *log_coeffs, const void *log_values, const void *h,
                          const void *g, void *dlog_coeffs, void *dlog_values,
                          int64_t B, int64_t T, int64_t D, mi_dtype dt,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* k x k matrix-affine scan ("Triton kernels", Kernel entry points:         */
/* affine_scan_fwd, affine_scan_bwd).  Dtypes: MI_F32, MI_BF16, MI_F16     */
/* (storage; arithmetic fp32).  1 <= k <= 16,                               */
/* 1 <= v <= 128.                                                           */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for mi_affine_scan_fwd / mi_affine_scan_bwd. */
size_t mi_affine_scan_workspace(int64_t B, int64_t T, int64_t n, int64_t k,
                                int64_t v, mi_dtype dt);

/* affine_scan_fwd: A (B,T,n,k,k), Bm (B,T,n,k,v) -> Abar (B,T,n,k,k), the
 * running product A_t @ ... @ A_1 (composition A_current @ A_earlier), and Bbar
 * (B,T,n,k,v), the H_0 = 0 solution of H_t = A_t @ H_{t-1} + Bm_t. */
mi_status mi_affine_scan_fwd(const void *A, const void *Bm, void *Abar, void *Bbar,
                             int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                             mi_dtype dt, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* affine_scan_bwd: reads the forward input A, the forward outputs Abar, Bbar and
 * the upstream grads gAbar (shape of Abar), gBbar (shape of Bbar); writes dA
 * (shape of A) and dB (shape of Bbar), the grads of <gAbar, Abar> +
 * <gBbar, Bbar> with respect to A and Bm.  With M_t = gAbar_t + A_{t+1}^T M_{t+1}
 * and Lam_t = gBbar_t + A_{t+1}^T Lam_{t+1} (nothing after T):
 * dB_t = Lam_t, dA_t = M_t Abar_{t-1}^T + Lam_t Bbar_{t-1}^T, Abar_0 = I,
 * Bbar_0 = 0.  Abar and Bbar are used as given. */
mi_status mi_affine_scan_bwd(const void *A, const void *Abar, const void *Bbar,
                             const void *gAbar, const void *gBbar, void *dA, void *dB,
                             int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                             mi_dtype dt, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* Scans from a given initial state (the k x k counterpart of
 * mi_linear_scan_fwd_h0 / _bwd_h0).  The page's affine_scan_fwd returns Bbar,
 * the solution from H_0 = 0.
 * mi_affine_scan_fwd_h0: H0 (B, n, k, v), or NULL for zero.  Writes Abar (as
 * mi_affine_scan_fwd) and H (B,T,n,k,v), H_t = A_t H_{t-1} + Bm_t, H_0 = H0;
 * equivalently X_t = A_t X_{t-1} + [0 | Bm_t] from X_0 = [I | H0].
 * mi_affine_scan_bwd_h0: gradient for L = <gAbar, Abar> + <gH, H>: dA, dB as
 * mi_affine_scan_bwd with H in place of Bbar and H0 as the state before the
 * first step (dA_1 = M_1 + Lam_1 H0^T), and dH0 (B,n,k,v) = A_1^T Lam_1 (zero
 * when T = 0).  Same dtype, envelope, workspace and errors as the calls
 * above; H0 and dH0 must not overlap outputs. */
mi_status mi_affine_scan_fwd_h0(const void *A, const void *Bm, const void *H0, void *Abar, void *H,
                                int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt,
                                void *ws, size_t ws_bytes, hipStream_t stream);
mi_status mi_affine_scan_bwd_h0(const void *A, const void *Abar, const void *H, const void *H0,
                                const void *gAbar, const void *gH, void *dA, void *dB, void *dH0,
                                int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt,
                                void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MISCAN_H */
