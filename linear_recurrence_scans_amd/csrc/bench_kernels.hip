// bench_kernels.hip -- bench-only kernels of libmiscan_bench.so (declared in
// include/miscan_bench.h): not part of the scan library.
//
//  * mi_bench_stream: the memory traffic of a channel scan without its carry.
//    The work items, lane mapping and accesses are those of the k = 1 scans
//    (a tile of 64 * VEC channels x a chunk of NW * L rows per workgroup,
//    chunk-major; 16-byte buffer-resource loads with the non-temporal policy,
//    non-temporal global stores), reading NIN (B, T, D) tensors and writing
//    NOUT.  Each output row is a sum of the input rows, so no load is dead.
//    Its rate is the streaming ceiling that the scans' own rate is compared
//    with: what the same access shape reaches when nothing but memory traffic
//    is left.
//  * mi_bench_flush: writes a buffer (at least 1 GiB in the benchmark) with
//    16-byte stores, to evict the L2s and the Infinity Cache before a
//    cold-cache timing.
#include "common.hpp"
#include "miscan_bench.h"

namespace miscan {
namespace {

struct StreamArgs {
    const void *in[5];
    void *out[2];
    int64_t T, D;
    int n_dtiles, n_tiles;
};

template <typename T, int VEC, int NIN, int NOUT, int L, int NW>
__global__ __launch_bounds__(NW * 64) void stream_kernel(StreamArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int item = blockIdx.x;
    const int chunk = item / p.n_tiles;
    const int tile = item - chunk * p.n_tiles;
    const int bidx = tile / p.n_dtiles;
    const int dtile = tile - bidx * p.n_dtiles;
    const int64_t d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    const bool lane_ok = d < p.D;
    const int64_t row0 = (int64_t)chunk * (NW * L);
    const uint32_t wrow = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * L;
    const int64_t t0 = row0 + wrow;
    const uint32_t voff = lane_ok ? (uint32_t)(d * (int64_t)sizeof(T)) : 0u;
    const uint32_t rowb = (uint32_t)(p.D * (int64_t)sizeof(T));
    raw_t x[NIN][L];
#pragma unroll
    for (int i = 0; i < NIN; ++i) {
        const rsrc_t rs = batch_rows<T>(p.in[i], bidx, row0, p.T, p.D);
#pragma unroll
        for (int r = 0; r < L; ++r) x[i][r] = buf_load<T, VEC>(rs, voff, t0 + r < p.T ? (wrow + r) * rowb : 0u);
    }
    if (!lane_ok) return;
#pragma unroll
    for (int r = 0; r < L; ++r) {
        if (t0 + r >= p.T) break;
        float acc[VEC], f[VEC];
        PK::unpack(x[0][r], acc);
#pragma unroll
        for (int i = 1; i < NIN; ++i) {
            PK::unpack(x[i][r], f);
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] += f[v];
        }
#pragma unroll
        for (int o = 0; o < NOUT; ++o) {
            float y[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) y[v] = acc[v] + (float)o;
            row_store<T, VEC>(PK::pack(y), row_ptr<T>(p.out[o], bidx, row0, p.T, p.D) + (wrow + r) * rowb, voff);
        }
    }
}

template <typename T, int VEC, int NIN, int NOUT>
mi_status run_stream(const StreamArgs &a, hipStream_t s, int64_t n_items) {
    constexpr int L = 8, NW = 8;
    hipLaunchKernelGGL((stream_kernel<T, VEC, NIN, NOUT, L, NW>), dim3((unsigned)n_items), dim3(NW * 64), 0, s, a);
    return launch_status();
}

template <typename T, int VEC>
mi_status stream_dispatch(const StreamArgs &a, int nin, int nout, hipStream_t s, int64_t n_items) {
    if (nin == 2 && nout == 2) return run_stream<T, VEC, 2, 2>(a, s, n_items);
    if (nin == 5 && nout == 2) return run_stream<T, VEC, 5, 2>(a, s, n_items);
    if (nin == 2 && nout == 1) return run_stream<T, VEC, 2, 1>(a, s, n_items);
    if (nin == 4 && nout == 2) return run_stream<T, VEC, 4, 2>(a, s, n_items);
    return MI_ERR_UNSUPPORTED;
}

__global__ void flush_kernel(u32x4 *p, size_t n16, uint32_t v) {
    const u32x4 q = {v, v + 1, v + 2, v + 3};
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        __builtin_nontemporal_store(q, p + i);
}

}  // namespace
}  // namespace miscan

using namespace miscan;

extern "C" {

mi_status mi_bench_stream(const void *const *in, int n_in, void *const *out, int n_out, int64_t B, int64_t T,
                          int64_t D, mi_dtype dt, hipStream_t stream) {
    const bool shape_built = (n_in == 2 && n_out == 2) || (n_in == 5 && n_out == 2) || (n_in == 2 && n_out == 1) ||
                             (n_in == 4 && n_out == 2);
    if (!shape_built || (dt != MI_F32 && dt != MI_BF16)) return MI_ERR_UNSUPPORTED;
    if (B <= 0 || T <= 0 || D <= 0 || in == nullptr || out == nullptr) return MI_ERR_INVALID_ARG;
    const int vec = dt == MI_F32 ? 4 : 8;
    if (D % vec != 0 || (T * D * (dt == MI_F32 ? 4 : 2)) >= ((int64_t)1 << 32)) return MI_ERR_UNSUPPORTED;
    StreamArgs a;
    for (int i = 0; i < 5; ++i) a.in[i] = i < n_in ? in[i] : nullptr;
    for (int i = 0; i < 2; ++i) a.out[i] = i < n_out ? out[i] : nullptr;
    for (int i = 0; i < n_in; ++i)
        if (a.in[i] == nullptr || reinterpret_cast<uintptr_t>(a.in[i]) % 16) return MI_ERR_INVALID_ARG;
    for (int i = 0; i < n_out; ++i)
        if (a.out[i] == nullptr || reinterpret_cast<uintptr_t>(a.out[i]) % 16) return MI_ERR_INVALID_ARG;
    const int64_t tile = 64 * vec, chunk = 64;
    a.T = T;
    a.D = D;
    a.n_dtiles = (int)((D + tile - 1) / tile);
    a.n_tiles = (int)(B * a.n_dtiles);
    const int64_t n_items = (int64_t)a.n_tiles * ((T + chunk - 1) / chunk);
    if (n_items > INT32_MAX) return MI_ERR_UNSUPPORTED;
    return dt == MI_F32 ? stream_dispatch<float, 4>(a, n_in, n_out, stream, n_items)
                        : stream_dispatch<bf16_t, 8>(a, n_in, n_out, stream, n_items);
}

mi_status mi_bench_flush(void *buf, size_t bytes, hipStream_t stream) {
    if (buf == nullptr || reinterpret_cast<uintptr_t>(buf) % 16 || bytes < 16) return MI_ERR_INVALID_ARG;
    static uint32_t tag = 0;
    hipLaunchKernelGGL(flush_kernel, dim3(4096), dim3(256), 0, stream, static_cast<u32x4 *>(buf), bytes / 16, ++tag);
    return launch_status();
}

}  // extern "C"
