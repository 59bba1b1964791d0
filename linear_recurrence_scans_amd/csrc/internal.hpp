// internal.hpp -- host-side interface between the C ABI (api.hip) and the
// kernel launchers.  Arguments reaching these functions are already validated.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "miscan.h"

namespace miscan {

// k = 1 channel scan and its adjoint (B, T, D).
size_t linear_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt);
size_t linear_fwd_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec);
// h0_kernels selects the initial-state kernels (h0 in, dh0 out; h0 may be NULL).
mi_status launch_linear_fwd(const void *a, const void *b, void *A, void *Bc,
                            int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec,
                            void *ws, size_t ws_bytes, hipStream_t s, bool h0_kernels = false,
                            const void *h0 = nullptr);
mi_status launch_linear_bwd(const void *a, const void *A, const void *Bc,
                            const void *gA, const void *gBc, void *da, void *db,
                            int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec,
                            void *ws, size_t ws_bytes, hipStream_t s, bool h0_kernels = false,
                            const void *h0 = nullptr, void *dh0 = nullptr);
// Zero `bytes` bytes at p on stream s (a small fill kernel).
mi_status zero_async(void *p, size_t bytes, hipStream_t s);

// Log-space scan (B, T, D); log_values is (B, T+1, D).
size_t log_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt);
mi_status launch_log_fwd(const void *lc, const void *lv, void *h,
                         int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec,
                         void *ws, size_t ws_bytes, hipStream_t s);
mi_status launch_log_bwd(const void *lc, const void *lv, const void *h, const void *g, void *dlc, void *dlv,
                         int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                         hipStream_t s);

// k x k scan (B, T, n, k, v).
size_t affine_workspace_bytes(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v);
// h0_kernels selects the initial-state kernels (H0 in, dH0 out; H0 may be NULL).
mi_status launch_affine_fwd(const void *A, const void *Bm, void *Abar, void *Bbar,
                            int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt,
                            void *ws, size_t ws_bytes, hipStream_t s, bool h0_kernels = false,
                            const void *H0 = nullptr);
mi_status launch_affine_bwd(const void *A, const void *Abar, const void *Bbar,
                            const void *gAbar, const void *gBbar, void *dA, void *dB,
                            int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt,
                            void *ws, size_t ws_bytes, hipStream_t s, bool h0_kernels = false,
                            const void *H0 = nullptr, void *dH0 = nullptr);

}  // namespace miscan
