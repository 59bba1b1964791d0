// api.hip -- the C ABI declared in include/miscan.h: argument validation,
// vector-width selection and dispatch to the kernel launchers.
//
// Every check runs before anything is enqueued, so a rejected call leaves the
// stream untouched (the minGRU docs page "Triton kernels", angle_scan_impl
// entry, checks every shape invariant before it enqueues anything), and nothing
// ever falls back to another implementation (the page's ScanFallback entry
// rules that out).
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace miscan {

__global__ void clear_ws_kernel(uint32_t *hdr, uint32_t *flags, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < WS_HEADER / sizeof(uint32_t)) hdr[i] = 0u;
    for (size_t j = i; j < n; j += (size_t)gridDim.x * blockDim.x) flags[j] = 0u;
}

mi_status clear_workspace(const WsPtrs &w, size_t n_slots, hipStream_t stream) {
    const size_t blocks = std::min<size_t>(1024, (n_slots + 255) / 256 + 1);
    hipLaunchKernelGGL(clear_ws_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w.hdr,
                       w.flags, n_slots);
    return launch_status();
}

// Zero n bytes (a grid-stride byte loop; used only for tiny outputs).
__global__ void zero_bytes_kernel(uint8_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

mi_status zero_async(void *p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return MI_OK;
    const unsigned blocks = (unsigned)std::min<size_t>(256, (bytes + 255) / 256);
    hipLaunchKernelGGL(zero_bytes_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint8_t *>(p), bytes);
    return launch_status();
}

namespace {

size_t elem_size(mi_dtype dt) { return dt == MI_F32 ? 4 : 2; }
bool dtype_known(mi_dtype dt) { return dt == MI_F32 || dt == MI_BF16 || dt == MI_F16; }

// a*b*c*d into *out without int64 overflow; all factors non-negative.
bool mul_ok(int64_t a, int64_t b, int64_t c, int64_t d, int64_t *out) {
    int64_t r;
    if (__builtin_mul_overflow(a, b, &r)) return false;
    if (__builtin_mul_overflow(r, c, &r)) return false;
    if (__builtin_mul_overflow(r, d, &r)) return false;
    *out = r;
    return true;
}

struct Buf {
    const void *p;
    int64_t bytes;
};

bool overlaps(const Buf &x, const Buf &y) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), b0 = reinterpret_cast<uintptr_t>(y.p);
    return a0 < b0 + (uintptr_t)y.bytes && b0 < a0 + (uintptr_t)x.bytes;
}

// Null, misaligned or overlapping buffers.  `n_out` trailing entries of `bufs`
// are outputs: an output may overlap nothing else.
mi_status check_buffers(const Buf *bufs, int n, int n_out, size_t align) {
    for (int i = 0; i < n; ++i) {
        if (bufs[i].p == nullptr) return MI_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(bufs[i].p) % align != 0) return MI_ERR_INVALID_ARG;
    }
    for (int i = n - n_out; i < n; ++i)
        for (int j = 0; j < n; ++j)
            if (j != i && overlaps(bufs[i], bufs[j])) return MI_ERR_INVALID_ARG;
    return MI_OK;
}

mi_status check_ws(void *ws, size_t ws_bytes, size_t need, const Buf *bufs, int n) {
    if (ws == nullptr || ws_bytes < need) return MI_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return MI_ERR_INVALID_ARG;
    Buf w{ws, (int64_t)ws_bytes};
    for (int i = 0; i < n; ++i)
        if (overlaps(w, bufs[i])) return MI_ERR_INVALID_ARG;
    return MI_OK;
}

// Widest vector (elements per lane) such that D is a multiple of it and every
// pointer is aligned to the access width; 16-byte accesses at most.
int pick_vec(int64_t D, size_t esize, const Buf *bufs, int n) {
    const int maxv = (int)(16 / esize);
    for (int v = maxv; v > 1; v /= 2) {
        if (D % v != 0) continue;
        bool ok = true;
        for (int i = 0; i < n && ok; ++i)
            ok = reinterpret_cast<uintptr_t>(bufs[i].p) % (v * esize) == 0;
        if (ok) return v;
    }
    return 1;
}

// Shared validation of the (B, T, D) channel ops.  Returns MI_OK and sets
// *empty when there is nothing to do.
mi_status check_btd(int64_t B, int64_t T, int64_t D, mi_dtype dt, int64_t *bytes, bool *empty) {
    if (B < 0 || T < 0 || D < 0) return MI_ERR_INVALID_ARG;
    if (!dtype_known(dt)) return MI_ERR_UNSUPPORTED;
    *empty = (B == 0 || T == 0 || D == 0);
    // (T + 1) rows covers log_values; elements are addressed in int64.
    if (!mul_ok(B, T + 1, D, (int64_t)elem_size(dt), bytes)) return MI_ERR_INVALID_ARG;
    *bytes = B * T * D * (int64_t)elem_size(dt);
    return MI_OK;
}

}  // namespace
}  // namespace miscan

using namespace miscan;

extern "C" {

const char *mi_status_string(mi_status s) {
    switch (s) {
        case MI_OK: return "MI_OK: success";
        case MI_ERR_INVALID_ARG:
            return "MI_ERR_INVALID_ARG: null, misaligned or overlapping buffer, negative size or size overflow";
        case MI_ERR_UNSUPPORTED:
            return "MI_ERR_UNSUPPORTED: outside the kernel envelope (k in [1,16], v in [1,128], dtype, grid size)";
        case MI_ERR_WORKSPACE: return "MI_ERR_WORKSPACE: workspace missing or smaller than the size query";
        case MI_ERR_LAUNCH: return "MI_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
        case MI_ERR_DEVICE: return "MI_ERR_DEVICE: no usable gfx950 device";
        case MI_ERR_CAPACITY:
            return "MI_ERR_CAPACITY: the problem needs more than the fixed scratch of the no-allocation entry point";
    }
    return "unknown mi_status";
}

mi_status mi_device_check(int device, char *reason, size_t reason_len) {
    auto say = [&](const char *msg) {
        if (reason && reason_len) {
            strncpy(reason, msg, reason_len - 1);
            reason[reason_len - 1] = '\0';
        }
    };
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count == 0) {
        say("no HIP device available");
        return MI_ERR_DEVICE;
    }
    if (device < 0 || device >= count) {
        say("device index out of range");
        return MI_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        say("hipGetDeviceProperties failed");
        return MI_ERR_DEVICE;
    }
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        char buf[160];
        snprintf(buf, sizeof(buf), "device %d is %s; this library is built for gfx950 only", device,
                 prop.gcnArchName);
        say(buf);
        return MI_ERR_DEVICE;
    }
    say("ok");
    return MI_OK;
}

size_t mi_linear_scan_workspace(int64_t B, int64_t T, int64_t D, mi_dtype dt) {
    int64_t bytes;
    bool empty;
    if (check_btd(B, T, D, dt, &bytes, &empty) != MI_OK || empty) return 0;
    return linear_workspace_bytes(B, T, D, dt);
}

mi_status mi_linear_scan_fwd(const void *a, const void *b, void *A, void *Bc, int64_t B, int64_t T,
                             int64_t D, mi_dtype dt, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK || empty) return st;
    const Buf bufs[4] = {{a, bytes}, {b, bytes}, {A, bytes}, {Bc, bytes}};
    if ((st = check_buffers(bufs, 4, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, linear_workspace_bytes(B, T, D, dt), bufs, 4)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, 4);
    return launch_linear_fwd(a, b, A, Bc, B, T, D, dt, vec, ws, ws_bytes, stream);
}

mi_status mi_linear_scan_bwd(const void *a, const void *A, const void *Bc, const void *gA,
                             const void *gBc, void *da, void *db, int64_t B, int64_t T, int64_t D,
                             mi_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK || empty) return st;
    const Buf bufs[7] = {{a, bytes},  {A, bytes},  {Bc, bytes}, {gA, bytes},
                         {gBc, bytes}, {da, bytes}, {db, bytes}};
    if ((st = check_buffers(bufs, 7, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, linear_workspace_bytes(B, T, D, dt), bufs, 7)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, 7);
    return launch_linear_bwd(a, A, Bc, gA, gBc, da, db, B, T, D, dt, vec, ws, ws_bytes, stream);
}

mi_status mi_linear_scan_fwd_h0(const void *a, const void *b, const void *h0, void *A, void *H, int64_t B,
                                int64_t T, int64_t D, mi_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK || empty) return st;
    const int64_t sbytes = B * D * (int64_t)elem_size(dt);
    // h0 (optional) joins the inputs; A and H are the outputs
    const Buf with_h0[5] = {{a, bytes}, {b, bytes}, {h0, sbytes}, {A, bytes}, {H, bytes}};
    const Buf no_h0[4] = {{a, bytes}, {b, bytes}, {A, bytes}, {H, bytes}};
    const Buf *bufs = h0 ? with_h0 : no_h0;
    const int nb = h0 ? 5 : 4;
    if ((st = check_buffers(bufs, nb, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, linear_workspace_bytes(B, T, D, dt), bufs, nb)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, nb);
    return launch_linear_fwd(a, b, A, H, B, T, D, dt, vec, ws, ws_bytes, stream, true, h0);
}

mi_status mi_linear_scan_bwd_h0(const void *a, const void *A, const void *H, const void *h0, const void *gA,
                                const void *gH, void *da, void *db, void *dh0, int64_t B, int64_t T, int64_t D,
                                mi_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK) return st;
    const int64_t sbytes = B * D * (int64_t)elem_size(dt);
    if (empty && T == 0 && B > 0 && D > 0) {  // no step: dh0 = 0
        if (dh0 == nullptr || reinterpret_cast<uintptr_t>(dh0) % elem_size(dt) != 0) return MI_ERR_INVALID_ARG;
        return zero_async(dh0, (size_t)sbytes, stream);
    }
    if (empty) return st;
    const Buf with_h0[9] = {{a, bytes},  {A, bytes},  {H, bytes},  {h0, sbytes}, {gA, bytes},
                            {gH, bytes}, {da, bytes}, {db, bytes}, {dh0, sbytes}};
    const Buf no_h0[8] = {{a, bytes},  {A, bytes},  {H, bytes},  {gA, bytes},
                          {gH, bytes}, {da, bytes}, {db, bytes}, {dh0, sbytes}};
    const Buf *bufs = h0 ? with_h0 : no_h0;
    const int nb = h0 ? 9 : 8;
    if ((st = check_buffers(bufs, nb, 3, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, linear_workspace_bytes(B, T, D, dt), bufs, nb)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, nb);
    return launch_linear_bwd(a, A, H, gA, gH, da, db, B, T, D, dt, vec, ws, ws_bytes, stream, true, h0, dh0);
}

size_t mi_scan_log_workspace(int64_t B, int64_t T, int64_t D, mi_dtype dt) {
    int64_t bytes;
    bool empty;
    if (check_btd(B, T, D, dt, &bytes, &empty) != MI_OK || empty) return 0;
    return log_workspace_bytes(B, T, D, dt);
}

mi_status mi_scan_log_fwd(const void *log_coeffs, const void *log_values, void *h, int64_t B,
                          int64_t T, int64_t D, mi_dtype dt, void *ws, size_t ws_bytes,
                          hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK || empty) return st;
    const int64_t lv_bytes = B * (T + 1) * D * (int64_t)elem_size(dt);
    const Buf bufs[3] = {{log_coeffs, bytes}, {log_values, lv_bytes}, {h, bytes}};
    if ((st = check_buffers(bufs, 3, 1, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, log_workspace_bytes(B, T, D, dt), bufs, 3)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, 3);
    return launch_log_fwd(log_coeffs, log_values, h, B, T, D, dt, vec, ws, ws_bytes, stream);
}

mi_status mi_scan_log_bwd(const void *log_coeffs, const void *log_values, const void *h, const void *g,
                          void *dlog_coeffs, void *dlog_values, int64_t B, int64_t T, int64_t D, mi_dtype dt,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK) return st;
    if (empty && T == 0 && B > 0 && D > 0) {
        // dlog_values still has its slot 0, d log h_0 = 0 when there is no step
        const Buf out{dlog_values, B * D * (int64_t)elem_size(dt)};
        if (out.p == nullptr || reinterpret_cast<uintptr_t>(out.p) % elem_size(dt) != 0) return MI_ERR_INVALID_ARG;
        return zero_async(dlog_values, (size_t)out.bytes, stream);
    }
    if (empty) return st;
    const int64_t lv_bytes = B * (T + 1) * D * (int64_t)elem_size(dt);
    const Buf bufs[6] = {{log_coeffs, bytes}, {log_values, lv_bytes}, {h, bytes},
                         {g, bytes},          {dlog_coeffs, bytes},   {dlog_values, lv_bytes}};
    if ((st = check_buffers(bufs, 6, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, log_workspace_bytes(B, T, D, dt), bufs, 6)) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, 6);
    return launch_log_bwd(log_coeffs, log_values, h, g, dlog_coeffs, dlog_values, B, T, D, dt, vec, ws, ws_bytes,
                          stream);
}

}  // extern "C"

namespace miscan {
namespace {

// Shared validation of the (B, T, n, k, v) matrix ops.
mi_status check_affine(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt,
                       int64_t *a_bytes, int64_t *b_bytes, bool *empty) {
    if (B < 0 || T < 0 || n < 0 || k < 0 || v < 0) return MI_ERR_INVALID_ARG;
    if (!dtype_known(dt)) return MI_ERR_UNSUPPORTED;
    if (k < 1 || k > 16 || v < 1 || v > 128) return MI_ERR_UNSUPPORTED;
    *empty = (B == 0 || T == 0 || n == 0);
    int64_t s;
    const int64_t es = (int64_t)elem_size(dt);
    if (!mul_ok(B, T, n, 1, &s)) return MI_ERR_INVALID_ARG;
    if (!mul_ok(s, k, k, es, a_bytes)) return MI_ERR_INVALID_ARG;
    if (!mul_ok(s, k, v, es, b_bytes)) return MI_ERR_INVALID_ARG;
    return MI_OK;
}

}  // namespace
}  // namespace miscan

extern "C" {

size_t mi_affine_scan_workspace(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v,
                                mi_dtype dt) {
    int64_t ab, bb;
    bool empty;
    if (check_affine(B, T, n, k, v, dt, &ab, &bb, &empty) != MI_OK || empty) return 0;
    return affine_workspace_bytes(B, T, n, k, v);
}

mi_status mi_affine_scan_fwd(const void *A, const void *Bm, void *Abar, void *Bbar, int64_t B,
                             int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
    int64_t ab, bb;
    bool empty;
    mi_status st = check_affine(B, T, n, k, v, dt, &ab, &bb, &empty);
    if (st != MI_OK || empty) return st;
    const Buf bufs[4] = {{A, ab}, {Bm, bb}, {Abar, ab}, {Bbar, bb}};
    if ((st = check_buffers(bufs, 4, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, affine_workspace_bytes(B, T, n, k, v), bufs, 4)) != MI_OK) return st;
    return launch_affine_fwd(A, Bm, Abar, Bbar, B, T, n, k, v, dt, ws, ws_bytes, stream);
}

mi_status mi_affine_scan_bwd(const void *A, const void *Abar, const void *Bbar, const void *gAbar,
                             const void *gBbar, void *dA, void *dB, int64_t B, int64_t T, int64_t n,
                             int64_t k, int64_t v, mi_dtype dt, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
    int64_t ab, bb;
    bool empty;
    mi_status st = check_affine(B, T, n, k, v, dt, &ab, &bb, &empty);
    if (st != MI_OK || empty) return st;
    const Buf bufs[7] = {{A, ab},     {Abar, ab}, {Bbar, bb}, {gAbar, ab},
                         {gBbar, bb}, {dA, ab},   {dB, bb}};
    if ((st = check_buffers(bufs, 7, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, affine_workspace_bytes(B, T, n, k, v), bufs, 7)) != MI_OK) return st;
    return launch_affine_bwd(A, Abar, Bbar, gAbar, gBbar, dA, dB, B, T, n, k, v, dt, ws, ws_bytes, stream);
}

mi_status mi_affine_scan_fwd_h0(const void *A, const void *Bm, const void *H0, void *Abar, void *H, int64_t B,
                                int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    int64_t ab, bb;
    bool empty;
    mi_status st = check_affine(B, T, n, k, v, dt, &ab, &bb, &empty);
    if (st != MI_OK || empty) return st;
    const int64_t sb = B * n * k * v * (int64_t)elem_size(dt);
    const Buf with_h0[5] = {{A, ab}, {Bm, bb}, {H0, sb}, {Abar, ab}, {H, bb}};
    const Buf no_h0[4] = {{A, ab}, {Bm, bb}, {Abar, ab}, {H, bb}};
    const Buf *bufs = H0 ? with_h0 : no_h0;
    const int nb = H0 ? 5 : 4;
    if ((st = check_buffers(bufs, nb, 2, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, affine_workspace_bytes(B, T, n, k, v), bufs, nb)) != MI_OK) return st;
    return launch_affine_fwd(A, Bm, Abar, H, B, T, n, k, v, dt, ws, ws_bytes, stream, true, H0);
}

mi_status mi_affine_scan_bwd_h0(const void *A, const void *Abar, const void *H, const void *H0, const void *gAbar,
                                const void *gH, void *dA, void *dB, void *dH0, int64_t B, int64_t T, int64_t n,
                                int64_t k, int64_t v, mi_dtype dt, void *ws, size_t ws_bytes, hipStream_t stream) {
    int64_t ab, bb;
    bool empty;
    mi_status st = check_affine(B, T, n, k, v, dt, &ab, &bb, &empty);
    if (st != MI_OK) return st;
    const int64_t sb = B * n * k * v * (int64_t)elem_size(dt);
    if (empty && T == 0 && B > 0 && n > 0) {  // no step: dH0 = 0
        if (dH0 == nullptr || reinterpret_cast<uintptr_t>(dH0) % elem_size(dt) != 0) return MI_ERR_INVALID_ARG;
        return zero_async(dH0, (size_t)sb, stream);
    }
    if (empty) return st;
    const Buf with_h0[9] = {{A, ab},  {Abar, ab}, {H, bb},  {H0, sb}, {gAbar, ab},
                            {gH, bb}, {dA, ab},   {dB, bb}, {dH0, sb}};
    const Buf no_h0[8] = {{A, ab}, {Abar, ab}, {H, bb}, {gAbar, ab}, {gH, bb}, {dA, ab}, {dB, bb}, {dH0, sb}};
    const Buf *bufs = H0 ? with_h0 : no_h0;
    const int nb = H0 ? 9 : 8;
    if ((st = check_buffers(bufs, nb, 3, elem_size(dt))) != MI_OK) return st;
    if ((st = check_ws(ws, ws_bytes, affine_workspace_bytes(B, T, n, k, v), bufs, nb)) != MI_OK) return st;
    return launch_affine_bwd(A, Abar, H, gAbar, gH, dA, dB, B, T, n, k, v, dt, ws, ws_bytes, stream, true, H0, dH0);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The entry point that allocates nothing, for callers that cannot call
// hipMalloc (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  Its look-back workspace is `scratch`, a file-scope
// device array of MI_NOALLOC_SCRATCH_BYTES that every GPU the library runs on
// holds until the process ends.  Host code never passes the array's name to a
// kernel (on the host it only stands in for the symbol): the first call on a
// device, with that device current, looks up the array's device address with
// hipGetSymbolAddress and keeps it per device.  Every call on a GPU shares
// that GPU's array, which keeps the last call's contents; the scan clears
// what must start at zero (ticket, timeout counter, flags) on the stream
// before its kernel, as the other entry points do with their workspace.
// ---------------------------------------------------------------------------
namespace miscan {
namespace {

static __device__ __align__(256) uint8_t scratch[MI_NOALLOC_SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES];

// Device address of the current device's scratch array.
mi_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) return MI_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MI_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MI_OK;
}

}  // namespace
}  // namespace miscan

extern "C" mi_status mi_linear_scan_fwd_noalloc(const void *a, const void *b, void *A, void *Bc, int64_t B,
                                                int64_t T, int64_t D, mi_dtype dt, hipStream_t stream) {
    int64_t bytes;
    bool empty;
    mi_status st = check_btd(B, T, D, dt, &bytes, &empty);
    if (st != MI_OK || empty) return st;
    const Buf bufs[4] = {{a, bytes}, {b, bytes}, {A, bytes}, {Bc, bytes}};
    if ((st = check_buffers(bufs, 4, 2, elem_size(dt))) != MI_OK) return st;
    const int vec = pick_vec(D, elem_size(dt), bufs, 4);
    const size_t need = linear_fwd_workspace_bytes(B, T, D, dt, vec);
    if (need == 0) return MI_ERR_UNSUPPORTED;  // the grid does not fit the ticket space
    if (need > (size_t)MI_NOALLOC_SCRATCH_BYTES) return MI_ERR_CAPACITY;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != MI_OK) return st;
    return launch_linear_fwd(a, b, A, Bc, B, T, D, dt, vec, ws, need, stream);
}
