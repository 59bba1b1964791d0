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
// (decoupled look-back).
//
// Visibility across the XCDs (each has its own L2) uses device-scope memory
// operations only, never cache maintenance: payload words and flags are
// written and read with agent-scope relaxed atomics, which gfx950 performs at
// the device coherence point (the sc1 bit).  The writer waits until its
// payload stores are acknowledged (s_waitcnt vmcnt(0)) before it stores the
// flag; the reader's payload loads are issued only after its flag load has
// returned a non-empty value (the branch on that value waits for it).  An
// agent-scope release/acquire pair would add an L2 writeback on every publish
// and an L2 invalidate on every poll, which the streaming kernels around it
// cannot afford.
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

// Payload words: device-coherent stores and loads.
__device__ __forceinline__ void carry_store(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float carry_load(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
__device__ __forceinline__ void carry_store_n(float *dst, const float *src) {
#pragma unroll
    for (int i = 0; i < N; ++i) carry_store(dst + i, src[i]);
}
template <int N>
__device__ __forceinline__ void carry_load_n(float *dst, const float *src) {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = carry_load(src + i);
}

// Vector form of carry_load for N = 1, 2 or 4 consecutive floats at byte
// offset `voff` of a buffer resource: the same cache policy (sc1) as the
// relaxed device-scope atomic loads, so it observes payload words published
// under the flag protocol.
constexpr int CPOL_SC1 = 16;
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

// Store the flag once this lane's earlier payload stores are acknowledged.
__device__ __forceinline__ void publish_flag(uint32_t *flag, uint32_t v) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-cooperative look-back wait.  Predecessor d (d = 0 is the nearest) owns
// slot slot0 + dir*d, for d < n_pred; the farthest predecessor always
// publishes an inclusive prefix without waiting on anyone.  Lane l polls
// predecessor base + l, so one coalesced load reads 64 flags.  Returns the
// distance k of the nearest predecessor whose inclusive prefix is published
// with every nearer one at least aggregate-ready: the caller then folds
// aggregates 0..k-1 and the inclusive prefix k.
//
// If `pending` is non-null the caller's own flag is stored (value
// `pending_val`) right after the first poll returns: the wait for the
// caller's payload acknowledgements then overlaps that first round trip.
// Every lane of the wave must call this.
__device__ __forceinline__ int wait_ready(const uint32_t *flags, int64_t slot0, int dir, int n_pred,
                                          uint32_t *timeouts, uint32_t *pending = nullptr,
                                          uint32_t pending_val = 0) {
    const int lane = threadIdx.x & 63;
    int base = 0;
    uint32_t spins = 0;
    while (true) {
        const int d = base + lane;
        const bool valid = d < n_pred;
        uint32_t f = FLAG_EMPTY;
        if (valid)
            f = __hip_atomic_load(flags + slot0 + (int64_t)dir * d, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t incm = __ballot(valid && f == FLAG_INC);
        const uint64_t empm = __ballot(valid && f == FLAG_EMPTY);
        if (pending) {
            publish_flag(pending, pending_val);
            pending = nullptr;
        }
        const int first_inc = incm ? __builtin_ctzll(incm) : 64;
        const int first_emp = empm ? __builtin_ctzll(empm) : 64;
        if (first_inc < first_emp) {
            asm volatile("" ::: "memory");  // payload loads stay after the flag loads
            return base + first_inc;
        }
        if (first_emp == 64 && base + 64 < n_pred) {  // whole window ready, none inclusive
            base += 64;
            continue;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++spins >= SPIN_LIMIT) {
            if (lane == 0) __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return n_pred - 1;
        }
    }
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

// Workgroups of a persistent kernel: as many as can be resident on the
// current device at once (they loop over tickets), never more than the work
// items.  Residency changes nothing for correctness -- a workgroup that is not
// yet running holds no ticket -- it only sizes the loop.
inline size_t persistent_grid(const void *kernel, int block, size_t n_items) {
    int dev = 0, n_cu = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess ||
        n_cu <= 0 || per_cu <= 0) {
        n_cu = 256;
        per_cu = 1;
    }
    const size_t cap = (size_t)n_cu * (size_t)per_cu;
    return n_items < cap ? n_items : cap;
}

inline mi_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MI_OK : MI_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// Workgroup-wide look-back for the channel scans.  A work item is a tile of
// TILE channels x one time chunk, run by NT threads.  Thread t owns channels
// t, t + NT, ... (< TILE); `c` holds this chunk's aggregate for them and `in`
// enters as the state before the first chunk (the identity unless the scan
// starts from a given state) and leaves as the carry-in of this chunk.
//
//  1. every thread stores its channels' aggregate (component-major payload,
//     so the stores and the loads below coalesce);
//  2. wave 0 finds the nearest predecessor with a published inclusive prefix
//     (wait_ready), publishing this chunk's aggregate flag on the way;
//  3. every thread folds the k aggregates and the inclusive prefix of its
//     channels, issuing up to BATCH predecessors' loads at a time -- so the walk
//     costs one round trip per BATCH predecessors rather than one each.  When
//     the workgroup has G >= 2 threads per channel, G groups fold disjoint
//     runs of predecessors at once and combine their partials through LDS;
//  4. every thread stores its channels' inclusive prefix in (+) c.
// The caller then stages `in` in LDS and calls wg_publish_inc.
//
// Op describes the carry algebra: NC floats per channel, and
// then(r, x, y): r = x followed by y (x is applied to the state first).
// ---------------------------------------------------------------------------
template <class Op, int TILE, int NT, int BATCH = 8>
__device__ __forceinline__ void wg_lookback(const WsPtrs &ws, int64_t slot, int dir, int n_pred,
                                            const float (&c)[(TILE + NT - 1) / NT][Op::NC],
                                            float (&in)[(TILE + NT - 1) / NT][Op::NC], int *s_k) {
    constexpr int NC = Op::NC, CPT = (TILE + NT - 1) / NT;
    constexpr int G = NT >= 2 * TILE ? NT / TILE : 1;  // predecessor-folding groups
    const int tid = threadIdx.x;
    const int64_t pay = (int64_t)NC * TILE;  // payload floats per slot
    if (n_pred > 0) {
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = tid + q * NT;
            if (ch < TILE)
#pragma unroll
                for (int m = 0; m < NC; ++m) carry_store(ws.agg + slot * pay + m * TILE + ch, c[q][m]);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // every wave's aggregate is acknowledged
        lds_barrier();
        if (tid < 64) {
            const int k = wait_ready(ws.flags, slot + dir, dir, n_pred, ws.hdr + 1, ws.flags + slot, FLAG_AGG);
            if (tid == 0) *s_k = k;
        }
        lds_barrier();
        const int k = *s_k;
        if constexpr (G == 1) {
            for (int j0 = 0; j0 <= k; j0 += BATCH) {
                float x[BATCH][CPT][NC];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int j = j0 + u;
                    if (j <= k) {
                        const float *src = (j == k ? ws.inc : ws.agg) + (slot + (int64_t)dir * (j + 1)) * pay;
#pragma unroll
                        for (int q = 0; q < CPT; ++q) {
                            const int ch = tid + q * NT;
#pragma unroll
                            for (int m = 0; m < NC; ++m)
                                x[u][q][m] = ch < TILE ? carry_load(src + m * TILE + ch) : 0.f;
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    if (j0 + u <= k) {
#pragma unroll
                        for (int q = 0; q < CPT; ++q) {
                            float r[NC];
                            Op::then(r, x[u][q], in[q]);  // predecessor j comes before all folded so far
#pragma unroll
                            for (int m = 0; m < NC; ++m) in[q][m] = r[m];
                        }
                    }
                }
            }
        } else {
            // G groups of TILE threads (CPT == 1).  Group g folds predecessors
            // [g * per, (g + 1) * per) into a partial transform, nearest
            // first; group 0 then applies the partials of the later groups,
            // which lie further back in time.
            __shared__ float s_part[G - 1][NC][TILE];
            const int grp = tid / TILE, ch = tid - grp * TILE;
            const int per = (k + 1 + G - 1) / G;
            const int lo = grp * per;
            const int hi = lo + per < k + 1 ? lo + per : k + 1;
            float part[NC];
            bool have = false;
            if (grp < G) {
                for (int j0 = lo; j0 < hi; j0 += BATCH) {
                    float x[BATCH][NC];
#pragma unroll
                    for (int u = 0; u < BATCH; ++u) {
                        const int j = j0 + u;
                        if (j < hi) {
                            const float *src = (j == k ? ws.inc : ws.agg) + (slot + (int64_t)dir * (j + 1)) * pay;
#pragma unroll
                            for (int m = 0; m < NC; ++m) x[u][m] = carry_load(src + m * TILE + ch);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < BATCH; ++u) {
                        if (j0 + u < hi) {
                            if (!have) {
#pragma unroll
                                for (int m = 0; m < NC; ++m) part[m] = x[u][m];
                                have = true;
                            } else {
                                float r[NC];
                                Op::then(r, x[u], part);
#pragma unroll
                                for (int m = 0; m < NC; ++m) part[m] = r[m];
                            }
                        }
                    }
                }
                if (grp > 0 && have)
#pragma unroll
                    for (int m = 0; m < NC; ++m) s_part[grp - 1][m][ch] = part[m];
            }
            lds_barrier();
            if (grp == 0) {
                if (have) {
                    float r[NC];
                    Op::then(r, part, in[0]);
#pragma unroll
                    for (int m = 0; m < NC; ++m) in[0][m] = r[m];
                }
                for (int g = 1; g < G && g * per < k + 1; ++g) {
                    float x[NC], r[NC];
#pragma unroll
                    for (int m = 0; m < NC; ++m) x[m] = s_part[g - 1][m][ch];
                    Op::then(r, x, in[0]);
#pragma unroll
                    for (int m = 0; m < NC; ++m) in[0][m] = r[m];
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
        const int ch = tid + q * NT;
        if (ch < TILE) {
            float r[NC];
            Op::then(r, in[q], c[q]);
#pragma unroll
            for (int m = 0; m < NC; ++m) carry_store(ws.inc + slot * pay + m * TILE + ch, r[m]);
        }
    }
}

// Publish the chunk's inclusive prefix once every wave's payload stores are
// acknowledged; the barrier also makes the caller's staged LDS carry visible.
__device__ __forceinline__ void wg_publish_inc(const WsPtrs &ws, int64_t slot) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    if (threadIdx.x < 64)
        __hip_atomic_store(ws.flags + slot, (uint32_t)FLAG_INC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace miscan
