/*
 * miscan_bench.h -- C ABI of libmiscan_bench.so, the benchmark's own probe
 * kernels.  They are not scans and not part of libmiscan.so; bench.py uses
 * them to put the scans' measured rates in context.
 */
#ifndef MISCAN_BENCH_H
#define MISCAN_BENCH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "miscan.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The memory traffic of a channel scan without its carry: reads the n_in
 * (1..5) device tensors in[] and writes the n_out (1..2) device tensors out[],
 * all (B, T, D) contiguous of storage type dt (MI_F32 or MI_BF16), with the
 * k = 1 scans' work items, lane mapping and 16-byte accesses (D a multiple of
 * 16 bytes, pointers 16-byte aligned).  out[o] = sum of the in[] rows + o.
 * Enqueued on `stream`; the caller owns every buffer.  MI_ERR_INVALID_ARG or
 * MI_ERR_UNSUPPORTED before anything is enqueued if the arguments do not fit;
 * supported (n_in, n_out): (2, 2), (5, 2), (2, 1), (4, 2). */
mi_status mi_bench_stream(const void *const *in, int n_in, void *const *out, int n_out,
                          int64_t B, int64_t T, int64_t D, mi_dtype dt, hipStream_t stream);

/* Writes `bytes` bytes (rounded down to 16) at the 16-byte aligned device
 * buffer `buf`, with non-temporal 16-byte stores: used before a cold-cache
 * timing, with a buffer larger than the L2s and the Infinity Cache. */
mi_status mi_bench_flush(void *buf, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MISCAN_BENCH_H */
