// common.hpp -- device-side building blocks shared by the scan kernels:
// storage <-> fp32 packing, vector row IO, the cross-workgroup carry protocol
// (dynamic chunk tickets + decoupled look-back flags) and the workspace layout.
//
// Target: gfx950 only (wave64, agent-scope release/acquire through the L2s of
// all XCDs).  Arithmetic is IEEE fp32; bf16 is a storage format only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "miscan.h"

namespace miscan {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 f = {lo, hi};
    bf16x2 r = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// Pack<T, VEC>: VEC consecutive elements of storage type T held as one raw
// register value, loaded/stored with a single VEC*sizeof(T)-byte access.
// ---------------------------------------------------------------------------
template <typename T, int VEC> struct Pack;

template <> struct Pack<float, 4> {
    typedef f32x4 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w; }
    static __device__ __forceinline__ raw_t pack(const float *f) { raw_t r = {f[0], f[1], f[2], f[3]}; return r; }
};
template <> struct Pack<float, 2> {
    typedef f32x2 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = r.x; f[1] = r.y; }
    static __device__ __forceinline__ raw_t pack(const float *f) { raw_t r = {f[0], f[1]}; return r; }
};
template <> struct Pack<float, 1> {
    typedef float raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = r; }
    static __device__ __forceinline__ raw_t pack(const float *f) { return f[0]; }
};
template <> struct Pack<bf16_t, 8> {
    typedef u32x4 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
    static __device__ __forceinline__ raw_t pack(const float *f) {
        raw_t r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                   pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
        return r;
    }
};
template <> struct Pack<bf16_t, 4> {
    typedef u32x2 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) {
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
    }
    static __device__ __forceinline__ raw_t pack(const float *f) {
        raw_t r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        return r;
    }
};
template <> struct Pack<bf16_t, 2> {
    typedef uint32_t raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = bf16_lo(r); f[1] = bf16_hi(r); }
    static __device__ __forceinline__ raw_t pack(const float *f) { return pack_bf16x2(f[0], f[1]); }
};
template <> struct Pack<bf16_t, 1> {
    typedef uint16_t raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = __uint_as_float((uint32_t)r << 16); }
    static __device__ __forceinline__ raw_t pack(const float *f) { return (uint16_t)(pack_bf16x2(f[0], 0.f) & 0xffffu); }
};

template <typename T, int VEC>
__device__ __forceinline__ typename Pack<T, VEC>::raw_t load_vec(const T *p) {
    return *reinterpret_cast<const typename Pack<T, VEC>::raw_t *>(p);
}

// Outputs are written once and never re-read by the kernel: stream them past
// the caches (nontemporal hint).
template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T *p, typename Pack<T, VEC>::raw_t r) {
    __builtin_nontemporal_store(r, reinterpret_cast<typename Pack<T, VEC>::raw_t *>(p));
}

template <typename T, int VEC>
__device__ __forceinline__ typename Pack<T, VEC>::raw_t splat(float x) {
    float f[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = x;
    return Pack<T, VEC>::pack(f);
}

// ---------------------------------------------------------------------------
// Cross-workgroup carry protocol.
//
// Work items (a channel tile x a time chunk) take a ticket from a global
// counter when they start, and the ticket -- not blockIdx -- decides which
// chunk they scan.  Tickets are handed out chunk-major in scan order, so an
// item only ever waits on items that already hold a ticket and are running:
// forward progress does not depend on the hardware's dispatch order.
//
// Each item publishes, per channel, first its local aggregate (flag AGG),
// then its inclusive prefix (flag INC).  A successor walks back over its
// predecessors' slots, folding aggregates until it meets an inclusive prefix
// (decoupled look-back).  Payload stores are ordered before the flag store by
// an agent-scope release; payload loads after the flag load by an agent-scope
// acquire (both span the separate L2s of the XCDs).
// ---------------------------------------------------------------------------
enum : uint32_t { FLAG_EMPTY = 0, FLAG_AGG = 1, FLAG_INC = 2 };

// About 2^22 polls of >= 64 cycles each (~0.1 s): only a broken protocol gets
// here.  The wait then gives up, counts the event in the workspace header and
// lets the kernel finish, so a bug shows up as a wrong result plus a non-zero
// counter instead of a hung GPU.
constexpr uint32_t SPIN_LIMIT = 1u << 22;

__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void publish_flag(uint32_t *flag, uint32_t v) {
    __hip_atomic_store(flag, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until the slot's flag is non-empty; returns FLAG_AGG or FLAG_INC.
__device__ __forceinline__ uint32_t wait_flag(const uint32_t *flag, uint32_t *timeouts) {
    uint32_t spins = 0;
    uint32_t f;
    while ((f = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)) == FLAG_EMPTY) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= SPIN_LIMIT) {
            __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return FLAG_INC;
        }
    }
    return f;
}

// ---------------------------------------------------------------------------
// Workspace layout (bytes), identical for every op:
//   [0, 256)                 header: u32 ticket counter, u32 timeout counter
//   [256, 256 + F)           u32 flag per slot, F rounded up to 256
//   [.., + P)                fp32 aggregate payload, `payload` floats per slot
//   [.., + P)                fp32 inclusive-prefix payload, same size
// ---------------------------------------------------------------------------
constexpr size_t WS_HEADER = 256;

__host__ __device__ inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

struct WsLayout {
    size_t flags_off, agg_off, inc_off, total;
    __host__ WsLayout(size_t n_slots, size_t payload_floats) {
        flags_off = WS_HEADER;
        agg_off = flags_off + round_up(n_slots * sizeof(uint32_t), 256);
        size_t pbytes = round_up(n_slots * payload_floats * sizeof(float), 256);
        inc_off = agg_off + pbytes;
        total = inc_off + pbytes;
    }
};

struct WsPtrs {
    uint32_t *hdr;    // [0] ticket, [1] timeouts
    uint32_t *flags;  // one per slot
    float *agg;
    float *inc;
};

inline WsPtrs ws_ptrs(void *ws, const WsLayout &l) {
    char *base = static_cast<char *>(ws);
    WsPtrs p;
    p.hdr = reinterpret_cast<uint32_t *>(base);
    p.flags = reinterpret_cast<uint32_t *>(base + l.flags_off);
    p.agg = reinterpret_cast<float *>(base + l.agg_off);
    p.inc = reinterpret_cast<float *>(base + l.inc_off);
    return p;
}

// Clears the header and the flags of `n_slots` slots before a scan launch
// (a plain kernel rather than a memset node, so the pair stays capturable).
mi_status clear_workspace(const WsPtrs &w, size_t n_slots, hipStream_t stream);

inline mi_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MI_OK : MI_ERR_LAUNCH;
}

}  // namespace miscan
