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
typedef _Float16 f16_t;   // IEEE binary16 (storage only; arithmetic stays fp32)

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

// fp16 <-> fp32: widening is exact (v_cvt_f32_f16); narrowing rounds to
// nearest even (v_cvt_f16_f32 under the default rounding mode), with fp16
// subnormals kept.
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(f16_t, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16_t, (uint16_t)(w >> 16)); }
__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (f16_t)x); }
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return (uint32_t)f16_bits(lo) | ((uint32_t)f16_bits(hi) << 16);
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

template <> struct Pack<f16_t, 8> {
    typedef u32x4 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) {
        f[0] = f16_lo(r.x); f[1] = f16_hi(r.x); f[2] = f16_lo(r.y); f[3] = f16_hi(r.y);
        f[4] = f16_lo(r.z); f[5] = f16_hi(r.z); f[6] = f16_lo(r.w); f[7] = f16_hi(r.w);
    }
    static __device__ __forceinline__ raw_t pack(const float *f) {
        raw_t r = {pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3]),
                   pack_f16x2(f[4], f[5]), pack_f16x2(f[6], f[7])};
        return r;
    }
};
template <> struct Pack<f16_t, 4> {
    typedef u32x2 raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) {
        f[0] = f16_lo(r.x); f[1] = f16_hi(r.x); f[2] = f16_lo(r.y); f[3] = f16_hi(r.y);
    }
    static __device__ __forceinline__ raw_t pack(const float *f) {
        raw_t r = {pack_f16x2(f[0], f[1]), pack_f16x2(f[2], f[3])};
        return r;
    }
};
template <> struct Pack<f16_t, 2> {
    typedef uint32_t raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = f16_lo(r); f[1] = f16_hi(r); }
    static __device__ __forceinline__ raw_t pack(const float *f) { return pack_f16x2(f[0], f[1]); }
};
template <> struct Pack<f16_t, 1> {
    typedef uint16_t raw_t;
    static __device__ __forceinline__ void unpack(raw_t r, float *f) { f[0] = (float)__builtin_bit_cast(f16_t, r); }
    static __device__ __forceinline__ raw_t pack(const float *f) { return f16_bits(f[0]); }
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

// ---------------------------------------------------------------------------
// Row access through buffer resources.  A work item sets up one descriptor
// per tensor, based at the first row it touches; a lane then needs a single
// 32-bit byte offset (its channels), and the row offset is a wave-uniform
// scalar.  No 64-bit address per row lives in vector registers.  Callers
// keep every offset inside the tensor themselves; the descriptor's size
// (accesses past it read zeros and are dropped) is a second line of defence.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw-buffer descriptor word 3 for gfx9-class GPUs (32-bit data format; the
// raw loads and stores used here ignore the format).
constexpr int RSRC_WORD3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rows(const void *base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : bytes >= (int64_t)0xffffffffll ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, RSRC_WORD3);
}

// Cache policy of the streaming row loads: non-temporal (NT).  Every row is
// read once (a halo row twice, soon after), so the loads should not displace
// cached lines; measured on the channel scans, NT loads run 4-6% faster than
// the default policy and 27% faster on a cold-cache log-space forward.
#ifndef MISCAN_LOAD_CPOL
#define MISCAN_LOAD_CPOL 2
#endif
template <typename T, int VEC>
__device__ __forceinline__ typename Pack<T, VEC>::raw_t buf_load(rsrc_t r, uint32_t voff, uint32_t soff) {
    using raw_t = typename Pack<T, VEC>::raw_t;
    constexpr int BYTES = (int)sizeof(T) * VEC;
    constexpr int CP = MISCAN_LOAD_CPOL;
    if constexpr (BYTES == 16) return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP));
    else if constexpr (BYTES == 8) return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CP));
    else if constexpr (BYTES == 4) return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CP));
    else return __builtin_bit_cast(raw_t, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, CP));
}

// Descriptor for the rows [first_row, T) of batch row `b` of a (B, T, D)
// tensor; accesses at or past row T read zeros and are dropped.
template <typename T>
__device__ __forceinline__ rsrc_t batch_rows(const void *tensor, int b, int64_t first_row, int64_t Tn,
                                             int64_t D) {
    const T *base = static_cast<const T *>(tensor) + ((int64_t)b * Tn + first_row) * D;
    return make_rows(base, (Tn - first_row) * D * (int64_t)sizeof(T));
}

// Row base of batch row `b`, time `row` of a (B, T, D) tensor.  With
// wave-uniform arguments the result is a scalar address.
template <typename T>
__device__ __forceinline__ char *row_ptr(void *tensor, int b, int64_t row, int64_t Tn, int64_t D) {
    return reinterpret_cast<char *>(static_cast<T *>(tensor) + ((int64_t)b * Tn + row) * D);
}

// Streaming store (nontemporal; outputs are written once, never re-read) of
// one lane's vector at byte offset `voff` from a wave-uniform row base: a
// global store with a scalar base and a 32-bit lane offset.
//
// Outputs deliberately do not use buffer stores.  On gfx950 a buffer store of
// more than 8 bytes that takes its row offset from an SGPR can still be
// reading its data registers when the next VALU instruction overwrites them,
// and the compiler inserts no wait state for that form; 16-byte bf16 stores
// were seen to lose their first dword that way.  The compiler does protect
// wide global stores.
template <typename T, int VEC>
__device__ __forceinline__ void row_store(typename Pack<T, VEC>::raw_t v, char *row, uint32_t voff) {
    __builtin_nontemporal_store(v, reinterpret_cast<typename Pack<T, VEC>::raw_t *>(row + voff));
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load of the calling wave (vmcnt(0)), which would
// drain rows prefetched for the next work item; the kernels exchange only LDS
// data across their barriers, so waiting for this wave's LDS operations
// (lgkmcnt(0)) is enough.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Makes the compiler treat a held raw row as freshly produced, so a second
// pass over rows kept in registers re-widens them from the packed storage
// instead of keeping a widened fp32 copy of every row alive in between.
template <typename R>
__device__ __forceinline__ void opaque(R &r) {
    asm volatile("" : "+v"(r));
}

template <typename T, int VEC>
__device__ __forceinline__ typename Pack<T, VEC>::raw_t splat(float x) {
    float f[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) f[i] = x;
    return Pack<T, VEC>::pack(f);
}

// ---------------------------------------------------------------------------
// Cross-workgroup carry protocol: a windowed look-back with a fixed
// association, so that every run rounds identically.
//
// Work items (a channel tile or head group x a time chunk) take a ticket from
// a global counter when they start, and the ticket -- not blockIdx -- decides
// which chunk they scan.  Tickets are handed out chunk-major in scan order, so
// an item only ever waits on items that already hold a ticket and are
// running: forward progress does not depend on the hardware's dispatch order.
//
// The chunks of one tile are numbered in scan order ord = 0, 1, ... (time
// order for a forward scan, reverse time for an adjoint).  Every chunk
// publishes two payloads in its slot: first its aggregate (the transform of
// its own rows), before it waits for anything, then its inclusive state.
// Chunk ord takes as its carry-in
//     the inclusive state of chunk ord - W (the scan's initial state if
//     ord < W), followed by the aggregates of the chunks after it, up to
//     ord - 1, applied in time order,
// with W a power of two that the host derives from the shape alone.  That
// expression depends on ord alone, never on which predecessor happened to
// publish first, so results are bitwise reproducible.  The inclusive states
// form W interleaved chains along time, each link W chunks long: the chunk a
// link waits for started W chunk rows earlier, so it has usually published.
//
// Visibility across the XCDs (each has its own L2) uses device-scope memory
// operations only, never cache maintenance: payload words and flags are
// written and read with agent-scope relaxed atomics, which gfx950 performs at
// the device coherence point (the sc1 bit).  The writer waits until its
// payload stores are acknowledged (s_waitcnt vmcnt(0)) before it stores the
// flag; the reader's payload loads are issued only after its flag loads have
// returned (the branch on their values waits for them).  An agent-scope
// release/acquire pair would add an L2 writeback on every publish and an L2
// invalidate on every poll, which the streaming kernels around it cannot
// afford.
// ---------------------------------------------------------------------------
enum : uint32_t { FLAG_EMPTY = 0, FLAG_AGG = 1, FLAG_INC = 2 };

// Position of a chunk in the look-back.
struct LbPos {
    int n_wait;    // predecessors folded: min(ord, W)
    bool has_inc;  // the farthest of them (ord - W) contributes its inclusive state
};
__host__ __device__ inline LbPos lb_pos(int ord, int W) {
    LbPos q;
    q.has_inc = ord >= W;
    q.n_wait = q.has_inc ? W : ord;
    return q;
}

// Window from the shape: about RESIDENT work items run at once, i.e.
// RESIDENT / tiles consecutive chunks of every tile.  A power of two in
// [2, wmax] (wmax <= 64: a wait polls one flag a lane).  It depends on the
// shape only, so equal shapes always fold in the same order.
#ifndef MISCAN_LB_RESIDENT
#define MISCAN_LB_RESIDENT 256
#endif
#ifndef MISCAN_LB_WMAX
#define MISCAN_LB_WMAX 16
#endif
inline int lb_window(int64_t tiles, int64_t resident = MISCAN_LB_RESIDENT, int wmax = MISCAN_LB_WMAX) {
    const int64_t want = tiles > 0 ? (resident + tiles - 1) / tiles : 1;
    int W = 2;
    while (W < want && W < wmax) W *= 2;
    return W;
}

// About 2^22 polls, each a device-coherent load (a round trip to the memory
// side, about a microsecond under load) plus a short sleep: seconds, so only a
// broken protocol gets here.  The wait then gives up, counts the event in the
// workspace header and lets the kernel finish, so a bug shows up as a wrong
// result plus a non-zero counter instead of a hung GPU.
constexpr uint32_t SPIN_LIMIT = 1u << 22;

__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Payload words: device-coherent stores and loads.
__device__ __forceinline__ void carry_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float carry_load(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Vector form of carry_load for N = 1, 2 or 4 consecutive floats at byte
// offset `voff` of a buffer resource: the same cache policy (sc1) as the
// relaxed device-scope atomic loads, so it observes payload words published
// under the flag protocol.
constexpr int CPOL_SC1 = 16;
// The same for a poll that a loop repeats: the volatile bit keeps the
// compiler from treating the repeated load as invariant.
constexpr int CPOL_SC1_VOLATILE = (int)(16u | 0x80000000u);
template <int N>
__device__ __forceinline__ void carry_load_vec(float *dst, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
    if constexpr (N == 4) {
        const f32x4 q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, CPOL_SC1));
        dst[0] = q.x; dst[1] = q.y; dst[2] = q.z; dst[3] = q.w;
    } else if constexpr (N == 2) {
        const f32x2 q = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, CPOL_SC1));
        dst[0] = q.x; dst[1] = q.y;
    } else {
        static_assert(N == 1, "N must be 1, 2 or 4");
        dst[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, CPOL_SC1));
    }
}

// One payload word at byte offset voff + soff of a buffer resource, with the
// device-coherent policy of carry_load (soff wave-uniform).
__device__ __forceinline__ float carry_load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, CPOL_SC1));
}

// Store the flag once this lane's earlier payload stores are acknowledged.
__device__ __forceinline__ void publish_flag(uint32_t *flag, uint32_t v) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-cooperative wait for a chunk's look-back window: the n_wait (<= 64)
// slots slot + dir, ..., slot + n_wait dir must have published their
// aggregate, and the farthest one its inclusive state if q.has_inc.  Lane d
// polls slot + (d + 1) dir, so one coalesced load reads every flag.  If `own`
// is non-null the caller's aggregate flag is stored right after the first
// poll returns: the wait for the caller's payload acknowledgements then
// overlaps that first round trip.  Every lane of the wave must call this.
__device__ __forceinline__ void wait_window(const uint32_t *flags, int64_t slot, int dir, const LbPos &q,
                                            uint32_t *timeouts, uint32_t *own) {
    const int lane = threadIdx.x & 63;
    const bool valid = lane < q.n_wait;
    const uint32_t need = (q.has_inc && lane == q.n_wait - 1) ? FLAG_INC : FLAG_AGG;
    // the window's flags through one descriptor based at its lowest slot: a
    // 32-bit offset per lane (device-coherent loads, as carry_load)
    const int64_t lo = dir < 0 ? slot - q.n_wait : slot + 1;
    const rsrc_t r = make_rows(flags + lo, (int64_t)q.n_wait * 4);
    const uint32_t voff = valid ? 4u * (uint32_t)(dir < 0 ? q.n_wait - 1 - lane : lane) : 0u;
    uint32_t spins = 0;
    while (true) {
        uint32_t f = FLAG_INC;
        if (valid) f = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, CPOL_SC1_VOLATILE);
        const uint64_t empty = __ballot(f < need);
        if (own) {
            publish_flag(own, FLAG_AGG);
            own = nullptr;
        }
        if (empty == 0) {
            asm volatile("" ::: "memory");  // payload loads stay after the flag loads
            return;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= SPIN_LIMIT) {
            if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
}

// ---------------------------------------------------------------------------
// Workspace layout (bytes), identical for every op:
//   [0, 256)                 header: u32 ticket counter, u32 timeout counter
//   [256, 256 + F)           u32 flag per slot, F rounded up to 256
//   [.., + P)                fp32 aggregate payload, `payload` floats per slot
//   [.., + P)                fp32 inclusive-state payload, same size
// ---------------------------------------------------------------------------
constexpr size_t WS_HEADER = 256;

__host__ __device__ inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

struct WsLayout {
    size_t flags_off, agg_off, inc_off, total;
    __host__ WsLayout(size_t n_slots, size_t payload_floats) {
        flags_off = WS_HEADER;
        agg_off = flags_off + round_up(n_slots * sizeof(uint32_t), 256);
        const size_t pbytes = round_up(n_slots * payload_floats * sizeof(float), 256);
        inc_off = agg_off + pbytes;
        total = inc_off + pbytes;
    }
};

struct WsPtrs {
    uint32_t *hdr;    // [0] ticket, [1] timeouts
    uint32_t *flags;  // one per slot
    float *agg;       // per slot: the chunk's aggregate
    float *inc;       // per slot: the inclusive state after the chunk
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

// ---------------------------------------------------------------------------
// Workgroup-wide look-back for the channel scans.  A work item is a tile of
// TILE channels x one time chunk, run by NT threads.  Thread t owns channels
// t, t + NT, ... (< TILE); `c` holds this chunk's aggregate for them and `in`
// enters as the scan's initial state (the identity unless the scan starts
// from a given state) and leaves as the carry-in of this chunk.
//
//  1. every thread stores its channels' aggregate (component-major payload,
//     so the stores and the loads below coalesce); wave 0 publishes it;
//  2. wave 0 waits for the chunk's look-back window (wait_window);
//  3. every thread folds, in time order, the inclusive state of chunk
//     ord - W (which replaces `in`) or, for ord < W, nothing, then the
//     aggregates of the window, issuing up to BATCH predecessors' loads at a
//     time: one round trip per BATCH payloads;
//  4. every thread stores its channels' inclusive state in (+) c; the caller
//     then stages `in` in LDS and calls wg_publish.
//
// Op describes the carry algebra: NC floats per channel, and
// then(r, x, y): r = x followed by y (x is applied to the state first).
// ---------------------------------------------------------------------------
template <class Op, int TILE, int NT, int BATCH = 8>
__device__ __forceinline__ void wg_lookback(const WsPtrs &ws, int64_t slot, int dir, const LbPos &q,
                                            const float (&c)[(TILE + NT - 1) / NT][Op::NC],
                                            float (&in)[(TILE + NT - 1) / NT][Op::NC]) {
    constexpr int NC = Op::NC, CPT = (TILE + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int64_t pay = (int64_t)NC * TILE;  // payload floats per slot
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = tid + u * NT;
        if (ch < TILE)
#pragma unroll
            for (int m = 0; m < NC; ++m) carry_store(ws.agg + slot * pay + m * TILE + ch, c[u][m]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every wave's aggregate is acknowledged
    lds_barrier();
    if (tid < 64) wait_window(ws.flags, slot, dir, q, ws.hdr + 1, ws.flags + slot);
    if (q.n_wait == 0) return;  // wave 0 has published; no carry to fold
    lds_barrier();
    // Fold index j = 0 is the farthest predecessor (slot + n_wait dir), j =
    // n_wait - 1 the nearest.  The predecessors' slots are consecutive: one
    // descriptor per payload array covers them, each lane keeps one offset
    // (its channel) and each predecessor and component is a wave-uniform
    // offset.
    const int64_t lo = dir < 0 ? slot - q.n_wait : slot + 1;  // lowest slot of the window
    const rsrc_t ra = make_rows(ws.agg + lo * pay, (int64_t)q.n_wait * pay * 4);
    const rsrc_t ri = make_rows(ws.inc + lo * pay, (int64_t)q.n_wait * pay * 4);
    for (int j0 = 0; j0 < q.n_wait; j0 += BATCH) {
        float x[BATCH][CPT][NC];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int j = j0 + u;
            if (j < q.n_wait) {
                const int a = dir < 0 ? j : q.n_wait - 1 - j;  // slot lo + a
                const bool from_inc = j == 0 && q.has_inc;
#pragma unroll
                for (int v = 0; v < CPT; ++v) {
                    const int ch = tid + v * NT;
                    const uint32_t voff = 4u * (uint32_t)(ch < TILE ? ch : 0);
#pragma unroll
                    for (int m = 0; m < NC; ++m)
                        x[u][v][m] = carry_load_buf(from_inc ? ri : ra, voff, 4u * (uint32_t)(a * pay + m * TILE));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int j = j0 + u;
            if (j < q.n_wait) {
#pragma unroll
                for (int v = 0; v < CPT; ++v) {
                    if (j == 0 && q.has_inc) {
#pragma unroll
                        for (int m = 0; m < NC; ++m) in[v][m] = x[u][v][m];  // chunk ord - W's inclusive state
                    } else {
                        float r[NC];
                        Op::then(r, in[v], x[u][v]);  // the state so far, then predecessor j's rows
#pragma unroll
                        for (int m = 0; m < NC; ++m) in[v][m] = r[m];
                    }
                }
            }
        }
    }
}

// Every chunk stores its inclusive state (in followed by c) for its channels.
template <class Op, int TILE, int NT>
__device__ __forceinline__ void wg_store_inclusive(const WsPtrs &ws, int64_t slot,
                                                   const float (&c)[(TILE + NT - 1) / NT][Op::NC],
                                                   const float (&in)[(TILE + NT - 1) / NT][Op::NC]) {
    constexpr int NC = Op::NC, CPT = (TILE + NT - 1) / NT;
    const int64_t pay = (int64_t)NC * TILE;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
        const int ch = threadIdx.x + u * NT;
        if (ch < TILE) {
            float r[NC];
            Op::then(r, in[u], c[u]);
#pragma unroll
            for (int m = 0; m < NC; ++m) carry_store(ws.inc + slot * pay + m * TILE + ch, r[m]);
        }
    }
}

// The barrier after the caller has staged its carry in LDS; the inclusive
// state is published once every wave's payload stores are acknowledged.
__device__ __forceinline__ void wg_publish(const WsPtrs &ws, int64_t slot) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (threadIdx.x < 64)
        __hip_atomic_store(ws.flags + slot, (uint32_t)FLAG_INC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace miscan
