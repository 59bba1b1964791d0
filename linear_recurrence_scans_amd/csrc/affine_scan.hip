// affine_scan.hip -- k x k matrix-affine scan H_t = A_t @ H_{t-1} + B_t, its
// running product, and its adjoint.
//
// Operations: minGRU docs, "Triton kernels" page, Kernel entry points,
// affine_scan_fwd (Abar_t = A_t @ ... @ A_1, composition A_current @ A_earlier;
// Bbar_t the H_0 = 0 solution) and affine_scan_bwd (grads w.r.t. A and Bm
// from A, Abar, Bbar, gAbar, gBbar).
//
// Layout: A, Abar (B,T,n,k,k) and Bm, Bbar (B,T,n,k,v), row-major; the n heads
// of one (b, t) are contiguous.
//
// Forward.  X_t = [Abar_t | H_t] is k x (k+v) and X_t = A_t X_{t-1} + [0 | B_t]
// with X_0 = [I | 0]: every column of X evolves on its own under the same
// A_t.  A lane therefore owns CPL columns of one head and keeps them (k*CPL
// fp32) in registers; the G = (k+v)/CPL lanes of a head share A_t, and a wave
// has HPW = 64/G such slots.  The k x k products are tiny and per step, not a
// dense contraction: they run on the vector ALU.
//
// In the forward the HPW slots hold HH heads x SEG time segments (HPW =
// HH * SEG): a workgroup covers HH heads for a chunk of SEG segments of
// NW * L steps.  Splitting a chunk into segments instead of filling the slots
// with other heads makes chunks SEG times longer at the same registers and
// LDS, so the chain of look-backs along time is SEG times shorter.  Pass 1 composes
// transforms [Abar | H] from [I | 0] (per wave, then over waves and over
// segments); the decoupled look-back (common.hpp) yields the state entering
// the chunk; pass 2 rescans from registers and writes the true states.  The
// look-back needs whole k x k blocks of other lanes' columns: those come from
// the published payloads in memory, or from LDS for the workgroup's own.
//
// Backward.  Y_t = [M_t | Lam_t] = [gAbar_t | gBbar_t] + A_{t+1}^T Y_{t+1}
// runs in reverse time, again column by column, with HPW adjacent heads per
// wave (loads and stores at one step hit one contiguous run of each tensor).
// A chunk's reverse transform
// also needs P_c = A_{t0+1}^T ... A_{t1+1}^T, so pass 1 carries k extra
// columns Z = [P | M | Lam] started from [I | 0 | 0].  Pass 2 produces
// dB_t = Lam_t directly and dA_t = Y_t X_{t-1}^T, a sum over the columns of
// several lanes, reduced through LDS.
#include "common.hpp"
#include "internal.hpp"

namespace miscan {
namespace {

enum : int { C_PAD = 0, C_ABAR = 1, C_H = 2 };         // forward column kinds
enum : int { Z_PAD = 0, Z_P = 1, Z_M = 2, Z_L = 3 };   // backward column kinds

template <int N>
__device__ __forceinline__ void ldv(float *dst, const float *src) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            f32x4 q = *reinterpret_cast<const f32x4 *>(src + i);
            dst[i] = q.x; dst[i + 1] = q.y; dst[i + 2] = q.z; dst[i + 3] = q.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            f32x2 q = *reinterpret_cast<const f32x2 *>(src + i);
            dst[i] = q.x; dst[i + 1] = q.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}

template <int N, bool NT>
__device__ __forceinline__ void stv(float *dst, const float *src) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            f32x4 q = {src[i], src[i + 1], src[i + 2], src[i + 3]};
            if constexpr (NT) __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(dst + i));
            else *reinterpret_cast<f32x4 *>(dst + i) = q;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            f32x2 q = {src[i], src[i + 1]};
            if constexpr (NT) __builtin_nontemporal_store(q, reinterpret_cast<f32x2 *>(dst + i));
            else *reinterpret_cast<f32x2 *>(dst + i) = q;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if constexpr (NT) __builtin_nontemporal_store(src[i], dst + i);
            else dst[i] = src[i];
        }
    }
}

// Global tensors are stored as TS (float or bf16); arithmetic is fp32.
// ld_g / st_g move N consecutive elements (a vector access when the width
// allows), widening bf16 on loads and rounding to nearest even on stores.
// (Default cache policy: unlike the channel scans, these kernels measured
// 10-20% slower with non-temporal loads.)
template <typename TS, int N>
__device__ __forceinline__ void ld_g(float *dst, const TS *src) {
    constexpr int W = (int)(16 / sizeof(TS)) < N ? (int)(16 / sizeof(TS)) : N;  // elements per access
    static_assert(N % W == 0, "vector width");
    using PK = Pack<TS, W>;
#pragma unroll
    for (int i = 0; i < N; i += W)
        PK::unpack(*reinterpret_cast<const typename PK::raw_t *>(src + i), dst + i);
}
template <typename TS, int N, bool NT>
__device__ __forceinline__ void st_g(TS *dst, const float *src) {
    constexpr int W = (int)(16 / sizeof(TS)) < N ? (int)(16 / sizeof(TS)) : N;
    static_assert(N % W == 0, "vector width");
    using PK = Pack<TS, W>;
#pragma unroll
    for (int i = 0; i < N; i += W) {
        const typename PK::raw_t r = PK::pack(src + i);
        if constexpr (NT) __builtin_nontemporal_store(r, reinterpret_cast<typename PK::raw_t *>(dst + i));
        else *reinterpret_cast<typename PK::raw_t *>(dst + i) = r;
    }
}
template <typename TS>
__device__ __forceinline__ float ld1(const TS *src) {
    float f[1];
    ld_g<TS, 1>(f, src);
    return f[0];
}
template <typename TS>
__device__ __forceinline__ void st1(TS *dst, float v) {
    const float f[1] = {v};
    st_g<TS, 1, false>(dst, f);
}

// Sixteen zero bytes in device memory, never written: lanes with nothing to
// load (padding and P columns, steps past T) read their CPL values here with a
// row stride of 0, so the loads need no select afterwards.
__device__ __align__(16) uint32_t g_aff_zeros[4];
template <typename TS>
__device__ __forceinline__ const TS *aff_zeros() {
    return reinterpret_cast<const TS *>(g_aff_zeros);
}

// Tensor pointers are untyped here; the kernels read them as TS.
struct FwdArgs {
    const void *A, *Bm;
    void *Abar, *Bbar;
    const void *H0;  // initial state (B, n, k, v) for the H0 kernels; NULL = zero
    int64_t T, heads;
    int n, k, v;
    int G, HPW, NCP, n_groups, n_chunks, NW;
    int HH;  // heads per workgroup; SEG = HPW / HH time segments per chunk
    int DB;  // payload blocks the look-back stages in LDS per round trip
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

struct BwdArgs {
    const void *A, *Abar, *Bbar, *gAbar, *gBbar;
    void *dA, *dB;
    const void *H0;  // initial state (B, n, k, v) for the H0 kernels; NULL = zero
    void *dH0;       // its gradient, written by the H0 kernels
    int64_t T, heads;
    int n, k, v;
    int G, HPW, NCP, n_groups, n_chunks, NW;
    int HH;  // heads per workgroup; SEG = HPW / HH time segments per chunk
    int DB;  // payload blocks the look-back stages in LDS per round trip
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

// Wave 0's look-back (publish, wait, fold, publish) is a link of the chain
// of inclusive states that later chunks wait on.  In the backward (three
// workgroups a CU, a window of two, the chain sets the pace) the wave issues
// ahead of the other waves on its SIMD while it runs: measured 664 -> 650 us
// (fp32) and 549 -> 535 us (bf16) on B=4, T=4096, n=32, k=8, v=32.  The
// forward gains nothing from it (bf16 runs 3% slower).
#ifndef MISCAN_AFF_LB_PRIO
#define MISCAN_AFF_LB_PRIO 0
#endif
#ifndef MISCAN_AFF_BWD_LB_PRIO
#define MISCAN_AFF_BWD_LB_PRIO 3
#endif
template <int PRIO>
__device__ __forceinline__ void lb_prio(bool on) {
    if constexpr (PRIO > 0) {
        if (on) __builtin_amdgcn_s_setprio(PRIO);
        else __builtin_amdgcn_s_setprio(0);
    }
}

// Column kinds of a lane.  With VIO all CPL columns share one kind (k and v
// are multiples of CPL).
template <int CPL>
struct Cols {
    int kind[CPL];
    int col[CPL];  // column index inside its own tensor
};

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// Time steps a wave holds in registers: L steps of the lane's B columns,
// L * KP * CPL floats, kept near 64 (see aff_breg_floats).  More steps per
// wave mean fewer pieces for the chunk's prefix rounds, whose block products
// are overhead on top of the two per step (compose, rescan); measured on the
// k = 4 and k = 8 forward, 64 beats 32, 48 and 96.
#ifndef MISCAN_AFF_BREGS
#define MISCAN_AFF_BREGS 64
#endif
#ifndef MISCAN_AFF_NWMAX
#define MISCAN_AFF_NWMAX 8
#endif
// The forward at padded k >= 8 needs over 128 VGPRs a lane: with four waves
// per workgroup two workgroups share a CU and overlap each other's loads,
// barriers and look-back, where one eight-wave workgroup would stall alone.
#ifndef MISCAN_AFF_NWMAX_K8
#define MISCAN_AFF_NWMAX_K8 4
#endif
// The backward holds the G_t columns of its steps and more state per lane
// (2k + v columns); it runs best with half the forward's budget.
#ifndef MISCAN_AFF_BWD_BREGS
#define MISCAN_AFF_BWD_BREGS 32
#endif
#ifndef MISCAN_AFF_BWD_NWMAX
#define MISCAN_AFF_BWD_NWMAX 4
#endif
// Floats of B (forward) or G (backward) columns a lane holds over its steps.
// The forward doubles its budget only at padded k = 8 with two columns a lane
// (measured faster, 256 VGPRs, no spill); four columns there, or padded
// k = 16, would spill with it.  The backward doubles it at padded k >= 8.
__host__ __device__ constexpr int aff_breg_floats(int KP, int CPL, bool bwd) {
    return bwd ? MISCAN_AFF_BWD_BREGS * (KP >= 8 ? 2 : 1)
               : MISCAN_AFF_BREGS * (KP >= 8 && KP * CPL <= 16 ? 2 : 1);
}
__host__ __device__ constexpr int aff_steps(int KP, int CPL, bool bwd) {
    return aff_breg_floats(KP, CPL, bwd) / (KP * CPL) < 1 ? 1
           : aff_breg_floats(KP, CPL, bwd) / (KP * CPL) > 16 ? 16
           : aff_breg_floats(KP, CPL, bwd) / (KP * CPL);
}
template <int KP, int CPL, bool BWD = false> struct AffL {
    static constexpr int L = aff_steps(KP, CPL, BWD);
};

// The lane's columns of B_t (zero for Abar and padding columns, or when !ok).
template <typename TS, int KP, int CPL, bool VIO>
__device__ __forceinline__ void load_b(float (&b)[KP][CPL], const FwdArgs &p, const Cols<CPL> &cl, int64_t m,
                                       bool ok) {
    const int k = VIO ? KP : p.k, v = p.v;
    const TS *Bm = static_cast<const TS *>(p.Bm);
    if constexpr (VIO) {
        // every lane loads, other kinds (and steps past T) zeros: no branch
        // around the loads and no select after them
        const bool use = ok && cl.kind[0] == C_H;
        const TS *src = use ? Bm + m * k * v + cl.col[0] : aff_zeros<TS>();
        const int ld = use ? v : 0;
#pragma unroll
        for (int i = 0; i < KP; ++i) ld_g<TS, CPL>(b[i], src + i * ld);
    } else {
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                b[i][cc] = (ok && cl.kind[cc] == C_H && i < k) ? ld1(Bm + m * k * v + i * v + cl.col[cc]) : 0.f;
    }
}

// Store the lane's columns of X_t = [Abar_t | H_t].
template <typename TS, int KP, int CPL, bool VIO>
__device__ __forceinline__ void store_x(const FwdArgs &p, const Cols<CPL> &cl, int64_t m, const float (&x)[KP][CPL]) {
    const int k = VIO ? KP : p.k, v = p.v;
    TS *Abar = static_cast<TS *>(p.Abar);
    TS *Bbar = static_cast<TS *>(p.Bbar);
    if constexpr (VIO) {
        if (cl.kind[0] != C_PAD) {
            TS *dst = (cl.kind[0] == C_ABAR) ? Abar + m * k * k + cl.col[0] : Bbar + m * k * v + cl.col[0];
            const int ld = (cl.kind[0] == C_ABAR) ? k : v;
#pragma unroll
            for (int i = 0; i < KP; ++i) st_g<TS, CPL, true>(dst + i * ld, x[i]);
        }
    } else {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
            for (int i = 0; i < KP; ++i) {
                if (i < k && cl.kind[cc] == C_ABAR) st1(Abar + m * k * k + i * k + cl.col[cc], x[i][cc]);
                if (i < k && cl.kind[cc] == C_H) st1(Bbar + m * k * v + i * v + cl.col[cc], x[i][cc]);
            }
    }
}

// LDS strides of per-head blocks, padded to 4 (mod 32) floats: the lanes of
// one head read the same address (a broadcast), and with this padding up to 8
// heads' blocks start in distinct banks.
__host__ __device__ constexpr int pad_bank(int f) { return f < 4 ? f : f + ((4 - f % 32) + 32) % 32; }

// Slot s of a wave holds head s % HH of the workgroup's group and segment
// s / HH of its chunk; row q (0 <= q < CHW = NW * L) of a segment is time step
// t_c + (s / HH) * CHW + q.
// Batch index and head of a global head index (b * n + h).  The plan admits
// fewer than 2^31 heads, so the division runs in 32 bits: a 64-bit division
// is a long instruction sequence, and the A staging divides once per element.
__device__ __forceinline__ void split_head(int64_t gh, int n, int64_t &b, int64_t &h) {
    const uint32_t g32 = (uint32_t)gh, q = g32 / (uint32_t)n;
    b = (int64_t)q;
    h = (int64_t)(g32 - q * (uint32_t)n);
}

struct SlotMap {
    int HH, CHW;
    __device__ __forceinline__ int64_t t(int64_t t_c, int s, int q) const { return t_c + (int64_t)(s / HH) * CHW + q; }
    __device__ __forceinline__ int64_t head(int grp, int s) const { return (int64_t)grp * HH + s % HH; }
};

// Loads a thread issues before its first LDS write when staging A: a batch
// of loads in flight together instead of a round trip each.  Sized to what a
// thread stages at padded k = 8 (six float4s on 3 heads x 32 steps) and half
// that at k = 4; the backward's chunks are shorter (two float4s a thread on
// 2 heads x 16 steps), and a batch of two keeps it at three waves per SIMD.  Other tiles keep one load at a
// time: they stage little A per thread (k <= 2) or have no registers to
// spare (k = 16).
#ifndef MISCAN_AFF_STAGE_BATCH
#define MISCAN_AFF_STAGE_BATCH 8
#endif
#ifndef MISCAN_AFF_BWD_STAGE_BATCH
#define MISCAN_AFF_BWD_STAGE_BATCH 2
#endif
__host__ __device__ constexpr int aff_stage_batch(int KP, bool bwd) {
    if (KP < 4 || KP > 8) return 1;
    return bwd ? MISCAN_AFF_BWD_STAGE_BATCH : KP == 8 ? MISCAN_AFF_STAGE_BATCH : MISCAN_AFF_STAGE_BATCH / 2;
}

// A_t of every slot for the CHW rows of its segment into LDS, laid out
// [row][slot][AS] with AS = pad_bank(KP * KP) (each block zero padded to
// KP x KP; identity for steps past T and for heads past the last).
// Cooperative, coalesced: consecutive threads take consecutive float4s (or
// floats) of the source blocks.  Each thread issues a batch of loads before
// it writes any of them.
template <typename TS, int KP, bool VIO>
__device__ __forceinline__ void stage_a(float *s_A, const FwdArgs &p, const SlotMap &sm, int grp, int64_t t_c) {
    const TS *Ag = static_cast<const TS *>(p.A);
    constexpr int KK = KP * KP;
    constexpr int AS = pad_bank(KK);
    constexpr int NB = aff_stage_batch(KP, false);
    constexpr int EPT = (VIO && KK % 4 == 0) ? 4 : 1;  // elements a thread moves per access
    using PK = Pack<TS, EPT>;
    const int per_row = p.HPW * KK;
    const int total = sm.CHW * per_row;
    const int step = (int)blockDim.x * EPT;
    const int k = VIO ? KP : p.k;
    // One batch: NB accesses starting at e0, every `step` elements.  Every
    // access loads (elements outside the tensor from its first element) and
    // the identity is selected at the write: no branch around a load, so the
    // batch's loads are all in flight before the first write waits.  The
    // first batch is straight-line code: in a loop the compiler waits for
    // every load in flight (the caller's too) before the loop's first load.
    auto batch = [&](int e0) {
        typename PK::raw_t raw[NB];
        int dst[NB], off[NB];
        bool in[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int e = e0 + u * step;
            const bool valid = e < total;
            const int ec = valid ? e : 0;
            const int q = ec / per_row;
            const int rem = ec - q * per_row;
            const int hs = rem / KK;
            const int o = rem - hs * KK;
            const int64_t t = sm.t(t_c, hs, q);
            const int64_t gh = sm.head(grp, hs);
            const int i = o / KP, j = o - (o / KP) * KP;
            in[u] = valid && t < p.T && gh < p.heads && (EPT == 4 || (i < k && j < k));
            int64_t b, h;
            split_head(in[u] ? gh : 0, p.n, b, h);
            const TS *src = Ag;
            if (in[u]) src = EPT == 4 ? Ag + ((b * p.T + t) * p.n + h) * KK + o
                                      : Ag + ((b * p.T + t) * p.n + h) * k * k + i * k + j;
            raw[u] = load_vec<TS, EPT>(src);
            dst[u] = valid ? (q * p.HPW + hs) * AS + o : -1;
            off[u] = o;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (dst[u] < 0) continue;
            float w[EPT];
            PK::unpack(raw[u], w);
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                const int o = off[u] + c;
                w[c] = in[u] ? w[c] : (o / KP == o % KP ? 1.f : 0.f);  // identity padding
            }
            if constexpr (EPT == 4)
                *reinterpret_cast<f32x4 *>(s_A + dst[u]) = f32x4{w[0], w[1], w[2], w[3]};
            else
                s_A[dst[u]] = w[0];
        }
    };
    const int e_first = (int)threadIdx.x * EPT;
    batch(e_first);
    for (int e0 = e_first + NB * step; e0 < total; e0 += NB * step) batch(e0);
}

// x <- A x + b for the lane's columns, A a KP x KP block in LDS.  b is zero
// outside the lane's H columns.
template <int KP, int CPL>
__device__ __forceinline__ void step_lds(float (&x)[KP][CPL], const float *Ablk, const float (&b)[KP][CPL]) {
    float nx[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        float arow[KP];
        ldv<KP>(arow, Ablk + i * KP);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float s = b[i][cc];
#pragma unroll
            for (int j = 0; j < KP; ++j) s = fmaf(arow[j], x[j][cc], s);
            nx[i][cc] = s;
        }
    }
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[i][cc] = nx[i][cc];
}

// The lane's columns of a [KP][NCP] block in LDS.
// (Rows start 16-byte aligned and c0 is a multiple of CPL: vector accesses.)
template <int KP, int CPL>
__device__ __forceinline__ void put_cols(float *blk, int NCP, int c0, const float (&x)[KP][CPL]) {
#pragma unroll
    for (int i = 0; i < KP; ++i) stv<CPL, false>(blk + i * NCP + c0, x[i]);
}
template <int KP, int CPL>
__device__ __forceinline__ void get_cols(float (&x)[KP][CPL], const float *blk, int NCP, int c0) {
#pragma unroll
    for (int i = 0; i < KP; ++i) ldv<CPL>(x[i], blk + i * NCP + c0);
}

// Own columns of one head's payload block, row-major (KP rows of NCP floats),
// moved with device-coherent word accesses (see common.hpp).
template <int KP, int CPL>
__device__ __forceinline__ void payload_store(float *blk, int NCP, int c0, const float (&x)[KP][CPL]) {
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) carry_store(blk + i * NCP + c0 + cc, x[i][cc]);
}
// S <- M S + [0 | H] for a transform block [M | H] (row-major, row stride
// NCP, the leading k x k block is M): the add term of each of the lane's H
// columns comes from the same block, so no copy of it is held in registers.
// `rows(i, m, h)` fetches row i: its first KP entries into m and the lane's
// CPL columns into h.  Fetches are unconditional (every address is inside
// the block) and out-of-range entries are zeroed by selects: a load under a
// per-lane branch costs a wait of its own.
template <int KP, int CPL, class Rows>
__device__ __forceinline__ void apply_rows(float (&S)[KP][CPL], Rows rows, int k, const bool (&is_h)[CPL]) {
    float ns[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        float mrow[KP], hrow[CPL];
        rows(i, mrow, hrow);
#pragma unroll
        for (int j = 0; j < KP; ++j) mrow[j] = (i < k && j < k) ? mrow[j] : 0.f;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float s = is_h[cc] ? hrow[cc] : 0.f;
#pragma unroll
            for (int j = 0; j < KP; ++j) s = fmaf(mrow[j], S[j][cc], s);
            ns[i][cc] = s;
        }
    }
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) S[i][cc] = ns[i][cc];
}

// The block in LDS (rows and the lane's columns 16-byte aligned).
template <int KP, int CPL>
__device__ __forceinline__ void block_apply(float (&S)[KP][CPL], const float *blk, int NCP, int k, int c0,
                                            const bool (&is_h)[CPL]) {
    apply_rows<KP, CPL>(S, [&](int i, float (&m)[KP], float (&h)[CPL]) {
        ldv<KP>(m, blk + i * NCP);
        ldv<CPL>(h, blk + i * NCP + c0);
    }, k, is_h);
}

// Float4s of look-back payload a thread loads per round trip, from each of
// the two arrays: the forward at padded k = 8 stages about three a thread
// (3 heads x 8 x 40 floats, 3 aggregates); smaller k stage under one, and the
// batch's registers would cost those kernels a wave per SIMD.
#ifndef MISCAN_AFF_PAYLOAD_BATCH
#define MISCAN_AFF_PAYLOAD_BATCH 4
#endif
#ifndef MISCAN_AFF_BWD_PAYLOAD_BATCH
#define MISCAN_AFF_BWD_PAYLOAD_BATCH 1
#endif
__host__ __device__ constexpr int aff_payload_batch(int KP, bool bwd) {
    return bwd ? MISCAN_AFF_BWD_PAYLOAD_BATCH : KP == 8 ? MISCAN_AFF_PAYLOAD_BATCH : 1;
}

// Look-back payloads into LDS, cooperatively: one round trip for a batch of
// up to DB published blocks instead of one per block.  A chunk folds n_wait
// predecessors; fold index q = 0 is the farthest (slot + n_wait dir) and, if
// q.has_inc, contributes its inclusive state (the `inc` array), the others
// their aggregates (the `agg` array); q = n_wait - 1 is the nearest (slot +
// dir).  That is time order for the forward (dir = -1) and reverse time
// order for the adjoint (dir = +1).  The batch holds fold indices b0 .. b0 +
// nb - 1, index q at s_stage + (q - b0) * slot_sz.  Its slots are
// consecutive, so each array is read through one descriptor; the loads from
// both arrays go out together before any is written to LDS.
template <int NB>
__device__ __forceinline__ void stage_payloads(float *s_stage, const WsPtrs &ws, int64_t slot, int dir,
                                               const LbPos &lq, int b0, int nb, int slot_sz) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n_wait = lq.n_wait;
    const bool inc = b0 == 0 && lq.has_inc;  // fold index 0: the inclusive state of slot + n_wait dir
    const int first = inc ? 1 : b0;
    const int last = b0 + nb - 1;
    const int na = last - first + 1;  // aggregates in this batch
    const int inc_len = inc ? slot_sz : 0;
    const int agg_len = na > 0 ? na * slot_sz : 0;
    const int64_t lo = dir < 0 ? slot - n_wait + first : slot + n_wait - last;  // lowest aggregate slot
    const rsrc_t ri = make_rows(ws.inc + (slot + (int64_t)dir * n_wait) * slot_sz, (int64_t)inc_len * 4);
    const rsrc_t ra = make_rows(ws.agg + (na > 0 ? lo : slot) * slot_sz, (int64_t)agg_len * 4);
    for (int e0 = tid * 4; e0 < inc_len || e0 < agg_len; e0 += nt * 4 * NB) {
        float vi[NB][4], va[NB][4];
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (e0 + u * nt * 4 < inc_len) carry_load_vec<4>(vi[u], ri, 4u * (uint32_t)(e0 + u * nt * 4));
#pragma unroll
        for (int u = 0; u < NB; ++u)
            if (e0 + u * nt * 4 < agg_len) carry_load_vec<4>(va[u], ra, 4u * (uint32_t)(e0 + u * nt * 4));
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int e = e0 + u * nt * 4;
            if (e < inc_len) *reinterpret_cast<f32x4 *>(s_stage + e) = f32x4{vi[u][0], vi[u][1], vi[u][2], vi[u][3]};
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int e = e0 + u * nt * 4;
            if (e < agg_len) {
                const int a = e / slot_sz, off = e - a * slot_sz;  // slot lo + a
                const int q = dir < 0 ? first + a : last - a;       // its fold index
                *reinterpret_cast<f32x4 *>(s_stage + (q - b0) * slot_sz + off) =
                    f32x4{va[u][0], va[u][1], va[u][2], va[u][3]};
            }
        }
    }
}

// One workgroup = NW waves; each wave holds HPW slots = HH heads x SEG
// segments, and wave w owns rows [w L, (w + 1) L) of every segment, so a chunk
// is SEG * NW * L steps of HH heads:
//  1. every wave loads its L steps of B (its columns) into registers, and the
//     workgroup stages the A_t blocks of every slot in LDS;
//  2. each wave composes its steps' transform [Abar_w | H_w] from [I | 0];
//  3. an inclusive prefix over the chunk's SEG * NW pieces (segment-major,
//     wave-minor: time order) of each head, through LDS, in log2(SEG * NW)
//     rounds;
//  4. wave 0 runs the look-back for the state entering the chunk and
//     publishes the chunk's inclusive state (the last prefix applied to it);
//  5. each piece applies the prefix of the pieces before it to that state,
//     rescans its steps from registers and stores Abar_t, Bbar_t.
// The chunk is read from memory once.
// H0: the scan starts from X_0 = [I | H0] (Bbar then holds the states from
// H0): the state entering chunk 0 is that instead of [I | 0].
template <typename TS, int KP, int CPL, bool VIO, bool H0 = false>
__global__ __launch_bounds__(512) void affine_fwd_kernel(FwdArgs p) {
    constexpr int L = AffL<KP, CPL>::L;
    extern __shared__ __align__(16) float s_dyn[];
    __shared__ uint32_t s_ticket;
    const int NW = p.NW, HPW = p.HPW, NCP = p.NCP, HH = p.HH;
    const int SEG = HPW / HH;
    constexpr int AS = pad_bank(KP * KP);  // LDS stride of an A_t block
    const int CHW = NW * L;                 // steps per segment
    const int CH = SEG * CHW;               // steps per chunk
    const SlotMap sm{HH, CHW};
    const int blk = KP * NCP;               // floats of one head's [KP][NCP] payload block
    const int bs = pad_bank(blk);           // LDS stride of such a block
    float *s_A = s_dyn;                     // [CHW][HPW][AS]
    float *s_X = s_A + (CHW * HPW * AS + 3) / 4 * 4;  // [NW][HPW][bs]: wave transforms (16-byte aligned)
    float *s_S = s_X + NW * HPW * bs;       // [HH][bs]: state entering the chunk, per head
    float *s_stage = s_S + HH * bs;         // [DB][HH * blk]: predecessor payloads

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)__builtin_amdgcn_readfirstlane(s_ticket);
    const int chunk = ticket / p.n_groups;
    const int grp = ticket - chunk * p.n_groups;
    const int hs = lane / p.G;
    const int g = lane - hs * p.G;
    const bool slot_lane = hs < HPW;  // lane maps to a slot
    const int hsc = slot_lane ? hs : 0;
    const int sg = hsc / HH;          // the slot's segment
    const int hh = hsc - sg * HH;     // and head within the group
    const int64_t gh = sm.head(grp, hsc);
    const bool active = slot_lane && gh < p.heads;
    int64_t bidx, hn;
    split_head(active ? gh : 0, p.n, bidx, hn);
    // With vector IO k equals KP: a compile-time k removes every bounds test
    // (and the branches around the loads) from the block products.
    const int k = VIO ? KP : p.k;
    const int c0 = g * CPL;

    Cols<CPL> cl;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int c = c0 + cc;
        if (!active || c >= k + p.v) { cl.kind[cc] = C_PAD; cl.col[cc] = 0; }
        else if (c < k) { cl.kind[cc] = C_ABAR; cl.col[cc] = c; }
        else { cl.kind[cc] = C_H; cl.col[cc] = c - k; }
    }
    bool is_h[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) is_h[cc] = cl.kind[cc] == C_H;

    const int64_t t_c = (int64_t)chunk * CH;  // first step of the chunk
    const int64_t t_w = sm.t(t_c, hsc, wave * L);  // first step of the lane's rows
    const int64_t m0 = bidx * p.T * p.n + hn;  // matrix index of (b, t = 0, h); + t n per step

    float x[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[i][cc] = (cl.kind[cc] == C_ABAR && i == cl.col[cc]) ? 1.f : 0.f;
    // 1. B of the wave's steps (registers) and the A_t blocks (LDS).
    //    With vector IO a lane's B columns and X_t destination are a base at
    //    the wave's first step plus one stride a step (n matrices): a step
    //    costs a 64-bit add, not a recomputed matrix index.
    float rb[L][KP][CPL];
    const TS *bsrc = nullptr;
    TS *xdst = nullptr;
    int64_t bstep = 0, xstep = 0;
    int xld = 0;
    if constexpr (VIO) {
        const int64_t mw = m0 + t_w * p.n;  // matrix index at the wave's first step
        const bool bh = active && cl.kind[0] == C_H;
        bsrc = bh ? static_cast<const TS *>(p.Bm) + mw * k * p.v + cl.col[0] : aff_zeros<TS>();
        bstep = bh ? p.n * (int64_t)k * p.v : 0;
        const bool xa = cl.kind[0] == C_ABAR;
        xdst = xa ? static_cast<TS *>(p.Abar) + mw * k * k + cl.col[0] : static_cast<TS *>(p.Bbar) + mw * k * p.v + cl.col[0];
        xstep = p.n * (int64_t)k * (xa ? k : p.v);
        xld = xa ? k : p.v;
        const int bld = bh ? p.v : 0;
        const TS *src = bsrc;
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const TS *sr = (t_w + r < p.T) ? src : aff_zeros<TS>();
            const int ldr = (t_w + r < p.T) ? bld : 0;
#pragma unroll
            for (int i = 0; i < KP; ++i) ld_g<TS, CPL>(rb[r][i], sr + i * ldr);
            src += bstep;
        }
    } else {
#pragma unroll
        for (int r = 0; r < L; ++r)
            load_b<TS, KP, CPL, VIO>(rb[r], p, cl, m0 + (t_w + r) * p.n, active && t_w + r < p.T);
    }
    stage_a<TS, KP, VIO>(s_A, p, sm, grp, t_c);
    lds_barrier();

    // 2. The wave's transform from [I | 0].
#pragma unroll
    for (int r = 0; r < L; ++r) step_lds<KP, CPL>(x, s_A + ((wave * L + r) * HPW + hsc) * AS, rb[r]);
    // 3. Inclusive prefix (Hillis-Steele) over the chunk's SEG * NW pieces in
    //    time order, e = segment * NW + wave; piece e of a head is wave e % NW
    //    in slot (e / NW) * HH + head.  After the round with offset o, piece e
    //    holds T_e o ... o T_{max(0, e - 2o + 1)}.  Each round applies the
    //    block of piece e - o to the piece's own transform:
    //    X <- X o P  means  [A_X A_P | A_X H_P + H_X], i.e. the lane's columns
    //    of P under A_X, plus H_X on the H columns.
    const int E = SEG * NW;
    const int e = sg * NW + wave;
    auto piece = [&](int q) { return s_X + ((q % NW) * HPW + (q / NW) * HH + hh) * bs; };
    if (slot_lane) put_cols<KP, CPL>(s_X + (wave * HPW + hs) * bs, NCP, c0, x);
    lds_barrier();
    for (int o = 1; o < E; o *= 2) {
        const bool upd = e >= o;
        float P[KP][CPL];
        get_cols<KP, CPL>(P, piece(upd ? e - o : e), NCP, c0);
        block_apply<KP, CPL>(P, s_X + (wave * HPW + hsc) * bs, NCP, k, c0, is_h);
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) x[i][cc] = upd ? P[i][cc] : x[i][cc];
        lds_barrier();  // every read of this round is done
        if (upd && slot_lane) put_cols<KP, CPL>(s_X + (wave * HPW + hs) * bs, NCP, c0, x);
        lds_barrier();
    }

    // 4. Look-back and publication (windowed look-back, common.hpp).  Wave 0
    //    publishes the chunk's transform and waits for the chunk's look-back
    //    window; the workgroup stages the window's payloads in LDS, a batch
    //    per round trip; wave 0 folds them in time order onto the initial
    //    state (or the inclusive state of chunk - W) and publishes the
    //    chunk's inclusive state.  The chunk transform of head hh is the
    //    prefix through its last piece.
    const float *s_C = piece(E - 1);
    const int slot_sz = HH * blk;
    const int hoff = hh * blk;
    const int64_t slot = (int64_t)grp * p.n_chunks + chunk;
    const LbPos lq = lb_pos(chunk, p.lb_window);
    float S[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) S[i][cc] = (cl.kind[cc] == C_ABAR && i == cl.col[cc]) ? 1.f : 0.f;
    if constexpr (H0) {
        if (!lq.has_inc && p.H0 != nullptr && active) {  // H columns of the initial state: H0
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    if (i < k && cl.kind[cc] == C_H)
                        S[i][cc] = ld1(static_cast<const TS *>(p.H0) + gh * k * p.v + i * p.v + cl.col[cc]);
        }
    }
    // Every segment's lanes of a head hold the same look-back values (same
    // loads, same operations) and store them to the same addresses.
    if (wave == 0) lb_prio<MISCAN_AFF_LB_PRIO>(true);
    if (wave == 0) {
        if (slot_lane) {
            float C[KP][CPL];
            get_cols<KP, CPL>(C, s_C, NCP, c0);
            payload_store<KP, CPL>(p.ws.agg + slot * slot_sz + hoff, NCP, c0, C);
        }
        wait_window(p.ws.flags, slot, -1, lq, p.ws.hdr + 1, p.ws.flags + slot);
    }
    if (lq.n_wait > 0) {
        lds_barrier();
        for (int b0 = 0; b0 < lq.n_wait; b0 += p.DB) {
            const int nb = lq.n_wait - b0 < p.DB ? lq.n_wait - b0 : p.DB;
            stage_payloads<aff_payload_batch(KP, false)>(s_stage, p.ws, slot, -1, lq, b0, nb, slot_sz);
            lds_barrier();
            if (wave == 0) {
                int q = b0;
                if (q == 0 && lq.has_inc) {  // the inclusive state of chunk - W
                    get_cols<KP, CPL>(S, s_stage + hoff, NCP, c0);
                    q = 1;
                }
                for (; q < b0 + nb; ++q) block_apply<KP, CPL>(S, s_stage + (q - b0) * slot_sz + hoff, NCP, k, c0, is_h);
            }
            if (b0 + p.DB < lq.n_wait) lds_barrier();  // the next batch overwrites the stage
        }
    }
    if (wave == 0) {
        if (slot_lane) put_cols<KP, CPL>(s_S + hh * bs, NCP, c0, S);
        block_apply<KP, CPL>(S, s_C, NCP, k, c0, is_h);  // S becomes the inclusive state
        if (slot_lane) payload_store<KP, CPL>(p.ws.inc + slot * slot_sz + hoff, NCP, c0, S);
        publish_flag(p.ws.flags + slot, FLAG_INC);
        lb_prio<MISCAN_AFF_LB_PRIO>(false);
    }
    lds_barrier();

    // 5. State entering this piece (the chunk's, then the prefix of the pieces
    //    before it), rescan, store.
    get_cols<KP, CPL>(S, s_S + hh * bs, NCP, c0);
    if (e > 0) block_apply<KP, CPL>(S, piece(e - 1), NCP, k, c0, is_h);
    const bool xst = active && cl.kind[0] != C_PAD;  // vector IO: the lane stores
#pragma unroll
    for (int r = 0; r < L; ++r) {
        step_lds<KP, CPL>(S, s_A + ((wave * L + r) * HPW + hsc) * AS, rb[r]);
        if constexpr (VIO) {
            if (xst && t_w + r < p.T) {
#pragma unroll
                for (int i = 0; i < KP; ++i) st_g<TS, CPL, true>(xdst + i * xld, S[i]);
            }
            xdst += xstep;
        } else {
            if (active && t_w + r < p.T) store_x<TS, KP, CPL, VIO>(p, cl, m0 + (t_w + r) * p.n, S);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

// Rows of dA partial sums exchanged through LDS per round.  Four keep the
// buffer small enough for three backward workgroups per CU at k = 8.
#ifndef MISCAN_AFF_RBMAX
#define MISCAN_AFF_RBMAX 4
#endif
template <int KP> struct AffRB {
    static constexpr int RB = KP < MISCAN_AFF_RBMAX ? KP : MISCAN_AFF_RBMAX;
};
// Floats between two lanes' dA partial sums (RB rows of KP) in LDS.  A stride
// that is a multiple of 8 floats put the 16-byte writes of every lane of a
// wave in the same 4 of the 32 banks; 4 more floats spread 8 consecutive
// lanes over all 32.
__host__ __device__ constexpr int aff_part_stride(int rbkp) { return rbkp >= 8 ? rbkp + 4 : rbkp; }

// dA_t with vector IO and k a multiple of 4 goes through rows instead: each
// head's Y_t and X_{t-1} rows in LDS (2 KP rows of the NCP columns), row
// stride an odd number of float4s so that the KP rows a wave reads at once
// fall in different banks.
__host__ __device__ constexpr bool aff_da_rows(int KP, bool VIO) { return VIO && KP % 4 == 0; }
__host__ __device__ constexpr int aff_row_stride(int NCP) { return (NCP / 4) % 2 == 0 ? NCP + 4 : NCP; }
// Floats of one wave's dA buffer (HPW heads).
// Floats between two heads' rows: 16 past the 2 KP rows, so that where one
// pass of a row write covers lanes of two heads (24 lanes a head at k = 8,
// v = 32) their words fall in opposite halves of the 32 banks.
__host__ __device__ constexpr int aff_row_head(int KP, int NCP) { return 2 * KP * aff_row_stride(NCP) + 16; }
__host__ __device__ constexpr int aff_da_wave_floats(int KP, int CPL, bool VIO, int HPW, int G, int NCP) {
    return aff_da_rows(KP, VIO) ? (HPW * aff_row_head(KP, NCP) + 3) / 4 * 4
                                : (HPW * G * aff_part_stride((KP < MISCAN_AFF_RBMAX ? KP : MISCAN_AFF_RBMAX) * KP) + 3) / 4 * 4;
}

// Source of the lane's columns of one of two (k x k | k x v) tensor pairs at
// matrix index m: the k x k tensor for Z_M columns, the k x v tensor for Z_L
// columns.  Lanes of other kinds (and !ok) read zeros (row stride 0): every
// lane loads, so no branch sits around the loads and no select follows them.
template <typename TS, int CPL>
__device__ __forceinline__ const TS *y_src(const void *kk_, const void *kv_, const Cols<CPL> &cl, int64_t m,
                                           int k, int v, bool ok, int &ld) {
    const TS *kk = static_cast<const TS *>(kk_), *kv = static_cast<const TS *>(kv_);
    const bool is_m = ok && cl.kind[0] == Z_M, is_l = ok && cl.kind[0] == Z_L;
    ld = is_l ? v : is_m ? k : 0;
    return is_m ? kk + m * k * k + cl.col[0] : is_l ? kv + m * k * v + cl.col[0] : aff_zeros<TS>();
}

// The lane's columns of G_t = [gAbar_t | gBbar_t] (zero for P and padding
// columns, or when !ok).
template <typename TS, int KP, int CPL, bool VIO>
__device__ __forceinline__ void load_g(float (&g)[KP][CPL], const BwdArgs &p, const Cols<CPL> &cl, int64_t m,
                                       bool ok) {
    const int k = VIO ? KP : p.k, v = p.v;
    if constexpr (VIO) {
        int ld;
        const TS *src = y_src<TS, CPL>(p.gAbar, p.gBbar, cl, m, k, v, ok, ld);
#pragma unroll
        for (int i = 0; i < KP; ++i) ld_g<TS, CPL>(g[i], src + i * ld);
    } else {
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                float gv = 0.f;
                if (ok && i < k) {
                    if (cl.kind[cc] == Z_M) gv = ld1(static_cast<const TS *>(p.gAbar) + m * k * k + i * k + cl.col[cc]);
                    else if (cl.kind[cc] == Z_L) gv = ld1(static_cast<const TS *>(p.gBbar) + m * k * v + i * v + cl.col[cc]);
                }
                g[i][cc] = gv;
            }
    }
}

// The lane's columns of X_{t-1} = [Abar_{t-1} | Bbar_{t-1}] matching its Y
// columns ([I | 0] at t = 0; zero when !ok), element-wise IO (vector IO uses
// xprev_issue / xprev_finish below).
template <typename TS, int KP, int CPL, bool H0 = false>
__device__ __forceinline__ void load_xprev(float (&x)[KP][CPL], const BwdArgs &p, const Cols<CPL> &cl, int64_t m,
                                           int64_t t, bool ok, int64_t gh = 0) {
    const int k = p.k, v = p.v;
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float xv = 0.f;
            if (ok && i < k) {
                if (cl.kind[cc] == Z_M)
                    xv = (t > 0) ? ld1(static_cast<const TS *>(p.Abar) + (m - p.n) * k * k + i * k + cl.col[cc])
                                 : (i == cl.col[cc] ? 1.f : 0.f);
                else if (cl.kind[cc] == Z_L && t > 0)
                    xv = ld1(static_cast<const TS *>(p.Bbar) + (m - p.n) * k * v + i * v + cl.col[cc]);
            }
            x[i][cc] = xv;
        }
    if constexpr (H0) {  // X_{-1} = [I | H0]: its H columns at t = 0
        if (ok && t == 0 && p.H0 != nullptr) {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    if (i < k && cl.kind[cc] == Z_L)
                        x[i][cc] = ld1(static_cast<const TS *>(p.H0) + gh * k * v + i * v + cl.col[cc]);
        }
    }
}

// load_xprev in two parts for vector IO: xprev_issue only loads (raw; lanes
// without X columns, and t = 0, read zeros) and xprev_finish widens, when the
// step uses the columns, and sets the identity at t = 0.  Work on the loaded
// values right after the loads would wait for them, so a load issued a step
// ahead would not stay in flight.
template <typename TS, int KP, int CPL>
struct XRaw {
    typename Pack<TS, CPL>::raw_t r[KP];
};
template <typename TS, int KP, int CPL>
__device__ __forceinline__ void xprev_issue(XRaw<TS, KP, CPL> &xr, const TS *src, int ld) {
#pragma unroll
    for (int i = 0; i < KP; ++i) xr.r[i] = load_vec<TS, CPL>(src + i * ld);
}
template <typename TS, int KP, int CPL, bool H0>
__device__ __forceinline__ void xprev_finish(float (&x)[KP][CPL], const XRaw<TS, KP, CPL> &xr, const BwdArgs &p,
                                             const Cols<CPL> &cl, int64_t t, bool ok, int64_t gh) {
#pragma unroll
    for (int i = 0; i < KP; ++i) Pack<TS, CPL>::unpack(xr.r[i], x[i]);
    if (t == 0) {  // wave-uniform: X_0 = [I | 0] on the lane's M columns (zeros were loaded)
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                x[i][cc] = (ok && cl.kind[cc] == Z_M && i == cl.col[cc]) ? 1.f : 0.f;
    }
    if constexpr (H0) {  // X_{-1} = [I | H0]: its H columns at t = 0
        if (ok && t == 0 && p.H0 != nullptr) {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
                    if (cl.kind[cc] == Z_L) x[i][cc] = ld1(static_cast<const TS *>(p.H0) + gh * KP * p.v + i * p.v + cl.col[cc]);
        }
    }
}

// A_{t+1}^T for the CH steps t of the chunk into LDS, [step][head][AS] like
// stage_a: zero for t = T - 1 (A_{T+1} = 0 in the page's 1-based time) and the
// identity for steps past T or heads past the last.  Sources are read as
// float4 rows and written transposed.  Batched like stage_a.
template <typename TS, int KP, bool VIO>
__device__ __forceinline__ void stage_at(float *s_A, const BwdArgs &p, int grp, int64_t t_c, int CH) {
    const TS *Ag = static_cast<const TS *>(p.A);
    constexpr int KK = KP * KP;
    constexpr int AS = pad_bank(KK);
    constexpr int NB = aff_stage_batch(KP, true);
    constexpr int EPT = (VIO && KP % 4 == 0) ? 4 : 1;  // elements a thread moves per access
    using PK = Pack<TS, EPT>;
    const int per_step = p.HPW * KK;
    const int total = CH * per_step;
    const int k = VIO ? KP : p.k;
    const int step = (int)blockDim.x * EPT;
    auto batch = [&](int e0) {  // as in stage_a
        typename PK::raw_t raw[NB];
        int dst[NB], jr[NB], i0[NB];
        float d[NB];
        bool in[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int e = e0 + u * step;
            const bool valid = e < total;
            const int ec = valid ? e : 0;
            const int st = ec / per_step;
            const int rem = ec - st * per_step;
            const int hs = rem / KK;
            const int q = rem - hs * KK;
            const int64_t t = t_c + st;
            const int64_t gh = (int64_t)grp * p.HPW + hs;
            // EPT == 4: source row jr, columns i0 .. i0 + 3, written transposed;
            // EPT == 1: element (i0, jr) of A^T = A[jr][i0]
            jr[u] = EPT == 4 ? q / KP : q - (q / KP) * KP;
            i0[u] = EPT == 4 ? q - (q / KP) * KP : q / KP;
            in[u] = valid && t + 1 < p.T && gh < p.heads && (EPT == 4 || (i0[u] < k && jr[u] < k));
            // diagonal where nothing loads: 0 at a head's last step (A_{T+1} = 0),
            // 1 elsewhere (steps past T, heads past the last, padding of k)
            d[u] = (gh < p.heads && t == p.T - 1) ? 0.f : 1.f;
            int64_t b, h;
            split_head(in[u] ? gh : 0, p.n, b, h);
            const TS *src = Ag;
            if (in[u]) src = EPT == 4 ? Ag + ((b * p.T + t + 1) * p.n + h) * KK + q
                                      : Ag + ((b * p.T + t + 1) * p.n + h) * k * k + jr[u] * k + i0[u];
            raw[u] = load_vec<TS, EPT>(src);
            dst[u] = valid ? (st * p.HPW + hs) * AS + (EPT == 4 ? i0[u] * KP + jr[u] : q) : -1;
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (dst[u] < 0) continue;
            float w[EPT];
            PK::unpack(raw[u], w);
#pragma unroll
            for (int c = 0; c < EPT; ++c) {
                const bool diag = EPT == 4 ? i0[u] + c == jr[u] : i0[u] == jr[u];
                w[c] = in[u] ? w[c] : (diag ? d[u] : 0.f);
                s_A[dst[u] + c * KP] = w[c];
            }
        }
    };
    const int e_first = (int)threadIdx.x * EPT;
    batch(e_first);
    for (int e0 = e_first + NB * step; e0 < total; e0 += NB * step) batch(e0);
}

// Reverse time.  Y_t = [M_t | Lam_t] = G_t + A_{t+1}^T Y_{t+1}; a chunk's
// reverse transform is Z = [P | Q]: Y at its first step = P Y_in + Q, with
// P = A_{t0+1}^T ... A_{t1}^T.  The lane's columns of Z are P (k), M (k) and
// Lam (v); the algebra is the forward's with Z for X and reverse order.
// One workgroup = NW waves = HPW heads x one chunk of CH = NW * L steps:
//  1. every wave loads its steps' G columns into registers; the workgroup
//     stages the chunk's A_{t+1}^T in LDS;
//  2. each wave composes its steps' reverse transform from [I | 0 | 0];
//  3. an inclusive suffix over the waves (reverse Hillis-Steele) through LDS;
//  4. the look-back over later chunks; wave 0 publishes the state at the
//     chunk's first step;
//  5. each wave applies the suffix of the waves after it to the state from
//     later time, rescans its steps backwards, stores dB_t = Lam_t and forms
//     dA_t = Y_t X_{t-1}^T from the X_{t-1} columns it loads step by step:
//     per-lane partial sums over its columns, added across the head's lanes
//     through a per-wave LDS buffer (RB rows a round).
// H0: the forward started from [I | H0]: X_{-1} = [I | H0] in dA at the first
// step, and dH0 = A_1^T Lam_1 is written as well.
template <typename TS, int KP, int CPL, bool VIO, bool H0 = false>
__global__ __launch_bounds__(512) void affine_bwd_kernel(BwdArgs p) {
    constexpr int L = AffL<KP, CPL, true>::L;
    constexpr int RB = AffRB<KP>::RB;
    constexpr int AS = pad_bank(KP * KP);
    extern __shared__ __align__(16) float s_dyn[];
    __shared__ uint32_t s_ticket;
    const int NW = p.NW, HPW = p.HPW, NCP = p.NCP, G = p.G;
    const int CH = NW * L;
    const int blk = KP * NCP;
    const int bs = pad_bank(blk);
    constexpr int PS = aff_part_stride(RB * KP);      // floats per lane in it
    const int pw = aff_da_wave_floats(KP, CPL, VIO, HPW, G, NCP);  // one wave's dA buffer
    const int YS = aff_row_stride(NCP);               // its row stride (row path)
    float *s_A = s_dyn;                                 // [CH][HPW][AS]: A_{t+1}^T
    float *s_X = s_A + (CH * HPW * AS + 3) / 4 * 4;     // [NW][HPW][bs]: wave transforms / suffixes
    float *s_S = s_X + NW * HPW * bs;                   // [HPW][bs]: Y entering the chunk from later
    float *s_part = s_S + HPW * bs;                     // [NW][pw]; first the look-back's payload stage

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)__builtin_amdgcn_readfirstlane(s_ticket);
    const int rchunk = ticket / p.n_groups;
    const int grp = ticket - rchunk * p.n_groups;
    const int chunk = p.n_chunks - 1 - rchunk;
    const int hs = lane / G;
    const int g = lane - hs * G;
    const bool slot_lane = hs < HPW;
    const int hsc = slot_lane ? hs : 0;
    const int64_t gh = (int64_t)grp * HPW + hs;
    const bool active = slot_lane && gh < p.heads;
    int64_t bidx, hh;
    split_head(active ? gh : 0, p.n, bidx, hh);
    const int k = VIO ? KP : p.k;
    const int v = p.v;
    const int c0 = g * CPL;

    Cols<CPL> cl;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
        const int c = c0 + cc;
        if (!active || c >= 2 * k + v) { cl.kind[cc] = Z_PAD; cl.col[cc] = 0; }
        else if (c < k) { cl.kind[cc] = Z_P; cl.col[cc] = c; }
        else if (c < 2 * k) { cl.kind[cc] = Z_M; cl.col[cc] = c - k; }
        else { cl.kind[cc] = Z_L; cl.col[cc] = c - 2 * k; }
    }
    bool is_y[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) is_y[cc] = cl.kind[cc] == Z_M || cl.kind[cc] == Z_L;

    const int64_t t_c = (int64_t)chunk * CH;
    const int64_t t_w = t_c + (int64_t)wave * L;
    const int64_t m0 = bidx * p.T * p.n + hh;

    // 1. G columns (registers), A_{t+1}^T (LDS).
    //    With vector IO a lane's G and X_{t-1} sources and dB, dA destinations
    //    are a base at the wave's first step plus one stride a step.
    float rg[L][KP][CPL];
    const int64_t mw = m0 + t_w * p.n;  // matrix index at the wave's first step
    const bool yl = active && (cl.kind[0] == Z_M || cl.kind[0] == Z_L);  // vector IO: Y columns
    const int64_t ystep = yl ? p.n * (int64_t)k * (cl.kind[0] == Z_M ? k : v) : 0;
    const int yld = yl ? (cl.kind[0] == Z_M ? k : v) : 0;
    if constexpr (VIO) {
        int ld0;
        const TS *src = y_src<TS, CPL>(p.gAbar, p.gBbar, cl, mw, k, v, active, ld0);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const bool ok = t_w + r < p.T;
            const TS *sr = ok ? src : aff_zeros<TS>();
            const int ldr = ok ? yld : 0;
#pragma unroll
            for (int i = 0; i < KP; ++i) ld_g<TS, CPL>(rg[r][i], sr + i * ldr);
            src += ystep;
        }
    } else {
#pragma unroll
        for (int r = 0; r < L; ++r) load_g<TS, KP, CPL, VIO>(rg[r], p, cl, m0 + (t_w + r) * p.n, active && t_w + r < p.T);
    }
    stage_at<TS, KP, VIO>(s_A, p, grp, t_c, CH);
    lds_barrier();

    // 2. The wave's reverse transform from [I | 0 | 0].
    {
        float z[KP][CPL];
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) z[i][cc] = (cl.kind[cc] == Z_P && i == cl.col[cc]) ? 1.f : 0.f;
#pragma unroll
        for (int r = L - 1; r >= 0; --r) step_lds<KP, CPL>(z, s_A + ((wave * L + r) * HPW + hsc) * AS, rg[r]);
        if (slot_lane) put_cols<KP, CPL>(s_X + (wave * HPW + hs) * bs, NCP, c0, z);
    }
    lds_barrier();


    // 3. Inclusive suffix: after the round with offset o, wave w holds
    //    T_w o T_{w+1} o ... (T of later waves applied first).
    for (int o = 1; o < NW; o *= 2) {
        float x[KP][CPL];
        if (wave + o < NW) {
            get_cols<KP, CPL>(x, s_X + ((wave + o) * HPW + hsc) * bs, NCP, c0);
            block_apply<KP, CPL>(x, s_X + (wave * HPW + hsc) * bs, NCP, k, c0, is_y);
        }
        lds_barrier();
        if (wave + o < NW && slot_lane) put_cols<KP, CPL>(s_X + (wave * HPW + hs) * bs, NCP, c0, x);
        lds_barrier();
    }

    // 4. Look-back over later chunks (windowed look-back, common.hpp): Y
    //    entering the chunk from later time (zero after the last chunk), then
    //    Y at the chunk's first step.  Wave 0 publishes the chunk's reverse
    //    transform and waits for the chunk's look-back window; the workgroup
    //    stages the window's payloads in LDS (in the dA buffer, idle until
    //    step 5), a batch per round trip; wave 0 folds them in reverse time
    //    order onto zero (or the state of chunk + W) and publishes the state
    //    at the chunk's first step.
    const int slot_sz = HPW * blk;
    const int hoff = hsc * blk;
    const int64_t slot = (int64_t)grp * p.n_chunks + chunk;
    const LbPos lq = lb_pos(rchunk, p.lb_window);
    float S[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) S[i][cc] = 0.f;
    if (wave == 0) lb_prio<MISCAN_AFF_BWD_LB_PRIO>(true);
    if (wave == 0) {
        if (slot_lane) {
            float Z[KP][CPL];
            get_cols<KP, CPL>(Z, s_X + hs * bs, NCP, c0);
            payload_store<KP, CPL>(p.ws.agg + slot * slot_sz + hoff, NCP, c0, Z);
        }
        wait_window(p.ws.flags, slot, +1, lq, p.ws.hdr + 1, p.ws.flags + slot);
    }
    if (lq.n_wait > 0) {
        lds_barrier();
        for (int b0 = 0; b0 < lq.n_wait; b0 += p.DB) {
            const int nb = lq.n_wait - b0 < p.DB ? lq.n_wait - b0 : p.DB;
            stage_payloads<aff_payload_batch(KP, true)>(s_part, p.ws, slot, +1, lq, b0, nb, slot_sz);
            lds_barrier();
            if (wave == 0) {
                int q = b0;
                if (q == 0 && lq.has_inc) {  // the state of chunk + W (its Y columns)
                    get_cols<KP, CPL>(S, s_part + hoff, NCP, c0);
#pragma unroll
                    for (int i = 0; i < KP; ++i)
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) S[i][cc] = is_y[cc] ? S[i][cc] : 0.f;
                    q = 1;
                }
                for (; q < b0 + nb; ++q) block_apply<KP, CPL>(S, s_part + (q - b0) * slot_sz + hoff, NCP, k, c0, is_y);
            }
            if (b0 + p.DB < lq.n_wait) lds_barrier();  // the next batch overwrites the stage
        }
    }
    if (wave == 0) {
        if (slot_lane) put_cols<KP, CPL>(s_S + hs * bs, NCP, c0, S);
        block_apply<KP, CPL>(S, s_X + hsc * bs, NCP, k, c0, is_y);  // through the whole chunk
        if (slot_lane) payload_store<KP, CPL>(p.ws.inc + slot * slot_sz + hoff, NCP, c0, S);
        publish_flag(p.ws.flags + slot, FLAG_INC);
        lb_prio<MISCAN_AFF_BWD_LB_PRIO>(false);
    }
    lds_barrier();

    // 5. Y entering this wave from later time, reverse rescan, outputs.
    get_cols<KP, CPL>(S, s_S + hsc * bs, NCP, c0);
    if (wave + 1 < NW) block_apply<KP, CPL>(S, s_X + ((wave + 1) * HPW + hsc) * bs, NCP, k, c0, is_y);
    float *part = s_part + wave * pw;
    if constexpr (aff_da_rows(KP, VIO)) {
        // the last group of four columns reads past 2k + v when it is not a
        // multiple of 4: those columns are never written, so zero them once
        // (the buffer held the look-back's stage until the barrier above)
        if (slot_lane && g == G - 1) {
            float *hb = part + hsc * aff_row_head(KP, NCP);
            for (int r2 = 0; r2 < 2 * KP; ++r2)
                for (int c = c0 + CPL; c < NCP; ++c) hb[r2 * YS + c] = 0.f;
        }
    }
    // X_{t-1} columns for dA, loaded one step ahead of their use: holding all
    // L steps would cost L * KP * CPL registers and a workgroup per CU, while
    // loading each in the step that uses it exposes the load latency.
    float rxn[KP][CPL];   // element-wise IO: the next step's columns
    XRaw<TS, KP, CPL> xn;  // vector IO: the next step's loads, still in flight
    // vector IO: X_{t-1} of step r (t = t_w + r) sits at matrix index t_w + r - 1
    int ldx0;
    const TS *xb = y_src<TS, CPL>(p.Abar, p.Bbar, cl, mw, k, v, active, ldx0);
    auto x_src = [&](int r, int &ldr) -> const TS * {
        const int64_t tr = t_w + r;
        const bool ok = yl && tr > 0 && tr < p.T;
        ldr = ok ? yld : 0;
        return ok ? xb + (int64_t)(r - 1) * ystep : aff_zeros<TS>();
    };
    if constexpr (VIO) {
        int ldr;
        const TS *sr = x_src(L - 1, ldr);
        xprev_issue<TS, KP, CPL>(xn, sr, ldr);
    } else
        load_xprev<TS, KP, CPL, H0>(rxn, p, cl, m0 + (t_w + L - 1) * p.n, t_w + L - 1,
                                         active && t_w + L - 1 < p.T, gh);
#pragma unroll
    for (int r = L - 1; r >= 0; --r) {
        const int64_t t = t_w + r;
        float rxr[KP][CPL];
        if constexpr (VIO) {
            xprev_finish<TS, KP, CPL, H0>(rxr, xn, p, cl, t, active && t < p.T, gh);
            if (r > 0) {
                int ldr;
                const TS *sr = x_src(r - 1, ldr);
                xprev_issue<TS, KP, CPL>(xn, sr, ldr);
            }
        } else {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) rxr[i][cc] = rxn[i][cc];
            if (r > 0)
                load_xprev<TS, KP, CPL, H0>(rxn, p, cl, m0 + (t_w + r - 1) * p.n, t_w + r - 1,
                                                 active && t_w + r - 1 < p.T, gh);
        }
        step_lds<KP, CPL>(S, s_A + ((wave * L + r) * HPW + hsc) * AS, rg[r]);  // S = Y_t
        if (t >= p.T) continue;  // wave-uniform
        const int64_t m = m0 + t * p.n;
        if constexpr (H0) {
            if (t == 0 && active) {  // dH0 = A_1^T Lam_1 for the lane's Lam columns
                float dh[KP][CPL];
#pragma unroll
                for (int i = 0; i < KP; ++i)
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) dh[i][cc] = 0.f;
#pragma unroll
                for (int j = 0; j < KP; ++j) {
                    float arow[KP];  // row j of A_1
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        arow[i] = (j < k && i < k) ? ld1(static_cast<const TS *>(p.A) + m * k * k + j * k + i) : 0.f;
#pragma unroll
                    for (int i = 0; i < KP; ++i)
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) dh[i][cc] = fmaf(arow[i], S[j][cc], dh[i][cc]);
                }
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        if (i < k && cl.kind[cc] == Z_L) st1(static_cast<TS *>(p.dH0) + gh * k * v + i * v + cl.col[cc], dh[i][cc]);
            }
        }
        // dB_t = Lam_t
        if (active) {
            if constexpr (VIO) {
                if (cl.kind[0] == Z_L) {
                    TS *db = static_cast<TS *>(p.dB) + (mw * k * v + cl.col[0]) + (int64_t)r * ystep;
#pragma unroll
                    for (int i = 0; i < KP; ++i) st_g<TS, CPL, true>(db + i * v, S[i]);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        if (i < k && cl.kind[cc] == Z_L) st1(static_cast<TS *>(p.dB) + m * k * v + i * v + cl.col[cc], S[i][cc]);
            }
        }
        if constexpr (aff_da_rows(KP, VIO)) {
            // dA_t = Y_t X_{t-1}^T as dot products over the k + v Y columns:
            // every lane writes its columns of Y_t and X_{t-1} into the head's
            // rows (no cross-lane sums), then lanes g < KP^2 / 4 of the head
            // each form a 2 x 2 block of dA_t (two Y rows and two X rows a
            // column group: four LDS reads for 16 FMA).  P columns (c < k)
            // are written but not read.
            float *hb = part + hsc * aff_row_head(KP, NCP);
            if (slot_lane) {
#pragma unroll
                for (int i = 0; i < KP; ++i) stv<CPL, false>(hb + i * YS + c0, S[i]);
#pragma unroll
                for (int j = 0; j < KP; ++j) stv<CPL, false>(hb + (KP + j) * YS + c0, rxr[j]);
            }
            // the wave's own rows are in LDS before any lane reads them
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // groups e = g, g + G, ...: at most MAXIT a lane (a head has at
            // least GMIN lanes, v >= CPL).  The loop over groups is unrolled:
            // with a global store in a loop of run-time length the compiler
            // waits for every load in flight, the next step's X_{t-1} too.
            TS *const dA_w = static_cast<TS *>(p.dA) + mw * k * k;  // dA at the wave's first step
            const int64_t dastep = p.n * (int64_t)k * k;
            constexpr int NG = KP * KP / 4;
            constexpr int GMIN = (2 * KP + CPL) / CPL;
            constexpr int MAXIT = (NG + GMIN - 1) / GMIN;
#pragma unroll
            for (int it = 0; it < MAXIT; ++it) {
                const int e = g + it * G;
                if (active && e < NG) {
                    const int i0 = e / (KP / 2) * 2, j0 = (e - e / (KP / 2) * (KP / 2)) * 2;
                    const float *yr = hb + i0 * YS;
                    const float *xr = hb + (KP + j0) * YS;
                    float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
                    for (int c = k; c < 2 * k + v; c += 4) {
                        float y[2][4], x[2][4];
#pragma unroll
                        for (int u = 0; u < 2; ++u) ldv<4>(y[u], yr + u * YS + c);
#pragma unroll
                        for (int u = 0; u < 2; ++u) ldv<4>(x[u], xr + u * YS + c);
#pragma unroll
                        for (int a = 0; a < 2; ++a)
#pragma unroll
                            for (int b = 0; b < 2; ++b)
#pragma unroll
                                for (int w = 0; w < 4; ++w) acc[a][b] = fmaf(y[a][w], x[b][w], acc[a][b]);
                    }
#pragma unroll
                    for (int a = 0; a < 2; ++a) st_g<TS, 2, true>(dA_w + (int64_t)r * dastep + (i0 + a) * k + j0, acc[a]);
                }
            }
            // LDS operations of one wave complete in order: the next step's
            // writes land after these reads; this keeps the compiler's order too.
            asm volatile("" ::: "memory");
        } else {
            // dA_t = Y_t X_{t-1}^T, RB rows a round.  Lanes that hold only P
            // columns (g < k / CPL) contribute zeros: they store no partial sums
            // and the readers skip their slots.
            const int g_first = k / CPL;
#pragma unroll
            for (int ib = 0; ib < KP; ib += RB) {
                if (slot_lane && g >= g_first) {
#pragma unroll
                    for (int ii = 0; ii < RB; ++ii) {
                        float row[KP];
#pragma unroll
                        for (int j = 0; j < KP; ++j) row[j] = 0.f;
#pragma unroll
                        for (int cc = 0; cc < CPL; ++cc) {
                            const float y = is_y[cc] ? S[ib + ii][cc] : 0.f;
#pragma unroll
                            for (int j = 0; j < KP; ++j) row[j] = fmaf(y, rxr[j][cc], row[j]);
                        }
                        stv<KP, false>(part + (hs * G + g) * PS + ii * KP, row);
                    }
                }
                // the wave's own partial sums are in LDS before any lane reads them
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (active) {
                    if constexpr (KP % 4 == 0) {
                        // groups of 4 consecutive entries of a row: vector LDS reads
                        for (int e = 4 * g; e < RB * KP; e += 4 * G) {
                            const int ii = e / KP, j0 = e - (e / KP) * KP;
                            const int i = ib + ii;
                            float acc[4] = {0.f, 0.f, 0.f, 0.f};
                            for (int gg = g_first; gg < G; ++gg) {
                                float q[4];
                                ldv<4>(q, part + (hs * G + gg) * PS + ii * KP + j0);
#pragma unroll
                                for (int u = 0; u < 4; ++u) acc[u] += q[u];
                            }
                            if constexpr (VIO) {
                                if (i < k) st_g<TS, 4, true>(static_cast<TS *>(p.dA) + m * k * k + (int64_t)i * k + j0, acc);
                            } else {
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    if (i < k && j0 + u < k) st1(static_cast<TS *>(p.dA) + m * k * k + (int64_t)i * k + j0 + u, acc[u]);
                            }
                        }
                    } else {
                        for (int e = g; e < RB * KP; e += G) {
                            const int ii = e / KP, j = e - (e / KP) * KP;
                            const int i = ib + ii;
                            float acc = 0.f;
                            for (int gg = g_first; gg < G; ++gg) acc += part[(hs * G + gg) * PS + ii * KP + j];
                            if (i < k && j < k) st1(static_cast<TS *>(p.dA) + m * k * k + (int64_t)i * k + j, acc);
                        }
                    }
                }
                // LDS operations of one wave complete in order: the next round's
                // writes land after these reads; this keeps the compiler's order too.
                asm volatile("" ::: "memory");
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: tile selection and launch.
// ---------------------------------------------------------------------------
struct AffPlan {
    int KP, CPL;
    bool VIO;
    bool h0;    // launch the initial-state (H0) kernels
    mi_dtype dt;  // storage type (arithmetic is fp32)
    int G, HPW, NCP, n_groups, n_chunks, LC, NW;
    int HH, SEG;  // heads per workgroup, time segments per chunk (HH * SEG = HPW)
    int DB;       // look-back payload blocks staged per round trip
    int W;        // look-back window
    size_t n_slots, payload, lds_bytes;
    bool ok;  // the work-item count fits the int32 ticket space, the LDS the workgroup
};

inline int next_pow2_16(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

// LDS per workgroup: the forward keeps two workgroups per CU possible; the
// backward (its registers allow one workgroup per CU at the larger k anyway)
// may take all 160 KiB for its dA partial-sum buffers.
constexpr size_t FWD_LDS_MAX = 65536;
#ifndef MISCAN_AFF_BWD_LDS
#define MISCAN_AFF_BWD_LDS 163840
#endif
constexpr size_t BWD_LDS_MAX = MISCAN_AFF_BWD_LDS;
// Shapes that need more than the budget even with one wave (large padded k
// with element-wise IO) take up to the device's 160 KiB per workgroup.
constexpr size_t LDS_DEVICE_MAX = 163840;

// Look-back: payload blocks staged in LDS per round trip, at most this many
// and (forward) within this many floats of LDS.  The backward stages them in
// its dA buffer.
#ifndef MISCAN_AFF_DBMAX
#define MISCAN_AFF_DBMAX 16
#endif
#ifndef MISCAN_AFF_STAGE_FLOATS
#define MISCAN_AFF_STAGE_FLOATS 4096
#endif

// Work items that run at once, for the look-back window (lb_window): the k x k
// fold costs a block product per payload on one wave, so its window is kept
// short (2 to 4 chunks at the workloads' head counts).
#ifndef MISCAN_AFF_RESIDENT
#define MISCAN_AFF_RESIDENT 128
#endif
#ifndef MISCAN_AFF_BWD_RESIDENT
#define MISCAN_AFF_BWD_RESIDENT MISCAN_AFF_RESIDENT
#endif

// Time segments per forward chunk: the largest divisor of HPW up to this
// bound.  Segments shorten the look-back chain but add prefix rounds; with
// the longer per-wave runs above, two segments at most measured fastest.
#ifndef MISCAN_AFF_SEGMAX
#define MISCAN_AFF_SEGMAX 2
#endif

inline int aff_L(int KP, int CPL, bool bwd) { return aff_steps(KP, CPL, bwd); }

// Tiling: G lanes x CPL columns per head (k + v columns forward, 2k + v
// backward), HPW slots per wave = HH heads x SEG time segments, L steps per
// wave and segment (AffL), NW waves per workgroup (as many as the LDS budget
// allows), chunks of SEG * NW * L steps.
inline AffPlan make_plan(int64_t B, int64_t T, int64_t n, int k, int v, bool bwd, int CPL, bool VIO) {
    AffPlan pl;
    pl.KP = next_pow2_16(k);
    pl.CPL = CPL;
    pl.VIO = VIO;
    pl.h0 = false;
    pl.dt = MI_F32;
    const int ncols = bwd ? 2 * k + v : k + v;
    pl.G = (ncols + CPL - 1) / CPL;
    if (pl.G > 64) {  // a head must fit one wave: this tiling is not usable
        pl.HPW = 0; pl.NCP = 0; pl.n_groups = 0; pl.n_chunks = 0; pl.LC = 0; pl.NW = 0;
        pl.HH = 0; pl.SEG = 0; pl.DB = 0; pl.W = 2;
        pl.n_slots = 0; pl.payload = 0; pl.lds_bytes = 0; pl.ok = false;
        return pl;
    }
    pl.HPW = 64 / pl.G;
    pl.SEG = 1;  // the backward holds HPW heads per wave (one segment)
    if (!bwd)
        for (int sgc = 1; sgc <= pl.HPW && sgc <= MISCAN_AFF_SEGMAX; ++sgc)
            if (pl.HPW % sgc == 0) pl.SEG = sgc;
    pl.HH = pl.HPW / pl.SEG;
    pl.NCP = (int)round_up((size_t)pl.G * CPL, 4);
    const int L = aff_L(pl.KP, CPL, bwd);
    const size_t a_ld = (size_t)pad_bank(pl.KP * pl.KP);  // LDS strides (see pad_bank)
    const size_t x_ld = (size_t)pad_bank(pl.KP * pl.NCP);
    const size_t part = (size_t)aff_da_wave_floats(pl.KP, CPL, VIO, pl.HPW, pl.G, pl.NCP);
    const size_t limit = bwd ? BWD_LDS_MAX : FWD_LDS_MAX;
    const size_t payload = (size_t)pl.HH * pl.KP * pl.NCP;  // floats of one look-back slot
    // Look-back window (payloads a chunk folds) and staged payloads per round
    // trip: no more than the window, so the forward's stage takes no more LDS
    // than one round needs.
    const int64_t heads = B * n;
    pl.W = lb_window((heads + pl.HH - 1) / pl.HH, bwd ? MISCAN_AFF_BWD_RESIDENT : MISCAN_AFF_RESIDENT);
    const size_t fwd_db = MISCAN_AFF_STAGE_FLOATS / payload;
    const int fdb_cap = pl.W < MISCAN_AFF_DBMAX ? pl.W : MISCAN_AFF_DBMAX;
    const int fdb = fwd_db < 1 ? 1 : fwd_db > (size_t)fdb_cap ? fdb_cap : (int)fwd_db;
    auto lds_floats = [&](int nw) {
        const size_t common = round_up((size_t)nw * L * pl.HPW * a_ld, 4) + (size_t)nw * pl.HPW * x_ld;
        // the backward's dA buffer also holds at least one staged payload
        const size_t dab = (size_t)nw * part > payload ? (size_t)nw * part : payload;
        return bwd ? common + (size_t)pl.HH * x_ld + dab : common + (size_t)pl.HH * x_ld + (size_t)fdb * payload;
    };
    pl.NW = 1;
    const int nwmax = bwd ? MISCAN_AFF_BWD_NWMAX : pl.KP >= 8 ? MISCAN_AFF_NWMAX_K8 : MISCAN_AFF_NWMAX;
    for (int nw = nwmax; nw >= 1; nw /= 2)
        if (lds_floats(nw) * sizeof(float) <= limit) { pl.NW = nw; break; }
    pl.LC = pl.SEG * pl.NW * L;
    pl.lds_bytes = lds_floats(pl.NW) * sizeof(float);
    const int64_t ng = (heads + pl.HH - 1) / pl.HH;
    const int64_t nc = (T + pl.LC - 1) / pl.LC;
    pl.ok = ng <= INT32_MAX && nc <= INT32_MAX && ng * nc <= (int64_t)INT32_MAX && heads <= INT32_MAX &&
            pl.lds_bytes <= LDS_DEVICE_MAX;
    pl.n_groups = (int)ng;
    pl.n_chunks = (int)nc;
    pl.n_slots = pl.ok ? (size_t)ng * (size_t)nc : 0;
    pl.payload = payload;
    if (bwd) {
        const size_t db = ((size_t)pl.NW * part > payload ? (size_t)pl.NW * part : payload) / payload;
        pl.DB = db > (size_t)fdb_cap ? fdb_cap : (int)db;
    } else {
        pl.DB = fdb;
    }
    return pl;
}

// Column tiling: of the vector tilings the alignment allows (k a power of two
// so that rows load as vectors, k and v multiples of CPL so that column groups
// never straddle tensors, 16-byte aligned pointers), the one whose waves cover
// the most steps (fewer look-back steps and payload bytes per step of data),
// four columns per lane on a tie; otherwise four columns with element accesses.
inline AffPlan choose_plan(int64_t B, int64_t T, int64_t n, int k, int v, bool bwd, bool ptrs16) {
    const bool kpow2 = next_pow2_16(k) == k;
    AffPlan best;
    bool have = false;
    const int cands[2] = {4, 2};
    for (int cpl : cands) {
        if (!(ptrs16 && kpow2 && k % cpl == 0 && v % cpl == 0)) continue;
        AffPlan pl = make_plan(B, T, n, k, v, bwd, cpl, true);
        if (!pl.ok) continue;
        // compare the time each wave covers (NW * L): segments lengthen chunks
        // of either width alike, while the wider tiling costs registers
        if (!have || pl.LC / pl.SEG > best.LC / best.SEG) { best = pl; have = true; }
    }
    if (!have) best = make_plan(B, T, n, k, v, bwd, 4, false);
    return best;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

// More than 64 KiB of dynamic LDS (the device allows 160 KiB per workgroup).
template <class K>
inline mi_status allow_lds(K kernel, size_t bytes) {
    if (bytes <= 65536) return MI_OK;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess ? MI_OK : MI_ERR_LAUNCH;
}

template <typename TS, int KP, int CPL, bool VIO, bool H0>
mi_status fwd_launch_h(const AffPlan &pl, FwdArgs &a, hipStream_t s) {
    if (pl.LC != pl.SEG * pl.NW * AffL<KP, CPL>::L || pl.HH * pl.SEG != pl.HPW)  // host and kernel tilings agree
        return MI_ERR_UNSUPPORTED;
    if (allow_lds(&affine_fwd_kernel<TS, KP, CPL, VIO, H0>, pl.lds_bytes) != MI_OK) return MI_ERR_LAUNCH;
    hipLaunchKernelGGL((affine_fwd_kernel<TS, KP, CPL, VIO, H0>), dim3((unsigned)pl.n_slots), dim3(64 * pl.NW),
                       pl.lds_bytes, s, a);
    return launch_status();
}
// Storage type and initial-state kernels from the plan.
template <int KP, int CPL, bool VIO>
mi_status fwd_launch(const AffPlan &pl, FwdArgs &a, hipStream_t s) {
    if (pl.dt == MI_BF16)
        return pl.h0 ? fwd_launch_h<bf16_t, KP, CPL, VIO, true>(pl, a, s)
                     : fwd_launch_h<bf16_t, KP, CPL, VIO, false>(pl, a, s);
    if (pl.dt == MI_F16)
        return pl.h0 ? fwd_launch_h<f16_t, KP, CPL, VIO, true>(pl, a, s)
                     : fwd_launch_h<f16_t, KP, CPL, VIO, false>(pl, a, s);
    return pl.h0 ? fwd_launch_h<float, KP, CPL, VIO, true>(pl, a, s) : fwd_launch_h<float, KP, CPL, VIO, false>(pl, a, s);
}
template <typename TS, int KP, int CPL, bool VIO, bool H0>
mi_status bwd_launch_h(const AffPlan &pl, BwdArgs &a, hipStream_t s) {
    if (pl.LC != pl.SEG * pl.NW * AffL<KP, CPL, true>::L || pl.HH * pl.SEG != pl.HPW) return MI_ERR_UNSUPPORTED;
    if (allow_lds(&affine_bwd_kernel<TS, KP, CPL, VIO, H0>, pl.lds_bytes) != MI_OK) return MI_ERR_LAUNCH;
    hipLaunchKernelGGL((affine_bwd_kernel<TS, KP, CPL, VIO, H0>), dim3((unsigned)pl.n_slots), dim3(64 * pl.NW),
                       pl.lds_bytes, s, a);
    return launch_status();
}
template <int KP, int CPL, bool VIO>
mi_status bwd_launch(const AffPlan &pl, BwdArgs &a, hipStream_t s) {
    if (pl.dt == MI_BF16)
        return pl.h0 ? bwd_launch_h<bf16_t, KP, CPL, VIO, true>(pl, a, s)
                     : bwd_launch_h<bf16_t, KP, CPL, VIO, false>(pl, a, s);
    if (pl.dt == MI_F16)
        return pl.h0 ? bwd_launch_h<f16_t, KP, CPL, VIO, true>(pl, a, s)
                     : bwd_launch_h<f16_t, KP, CPL, VIO, false>(pl, a, s);
    return pl.h0 ? bwd_launch_h<float, KP, CPL, VIO, true>(pl, a, s) : bwd_launch_h<float, KP, CPL, VIO, false>(pl, a, s);
}

// Instantiated tiles: vector IO for k in {4,8,16} (CPL 4) and {2,4,8,16}
// (CPL 2); element-wise IO with CPL 4 for every padded k.
#define MISCAN_AFF_DISPATCH(FN, PL, ARGS, S)                          \
    do {                                                              \
        const int kp_ = (PL).KP;                                      \
        if ((PL).VIO && (PL).CPL == 4) {                              \
            if (kp_ == 4) return FN<4, 4, true>(PL, ARGS, S);         \
            if (kp_ == 8) return FN<8, 4, true>(PL, ARGS, S);         \
            if (kp_ == 16) return FN<16, 4, true>(PL, ARGS, S);       \
        } else if ((PL).VIO && (PL).CPL == 2) {                       \
            if (kp_ == 2) return FN<2, 2, true>(PL, ARGS, S);         \
            if (kp_ == 4) return FN<4, 2, true>(PL, ARGS, S);         \
            if (kp_ == 8) return FN<8, 2, true>(PL, ARGS, S);         \
            if (kp_ == 16) return FN<16, 2, true>(PL, ARGS, S);       \
        } else {                                                      \
            if (kp_ == 1) return FN<1, 4, false>(PL, ARGS, S);        \
            if (kp_ == 2) return FN<2, 4, false>(PL, ARGS, S);        \
            if (kp_ == 4) return FN<4, 4, false>(PL, ARGS, S);        \
            if (kp_ == 8) return FN<8, 4, false>(PL, ARGS, S);        \
            if (kp_ == 16) return FN<16, 4, false>(PL, ARGS, S);      \
        }                                                             \
        return MI_ERR_UNSUPPORTED;                                    \
    } while (0)

mi_status dispatch_fwd(const AffPlan &pl, FwdArgs &a, hipStream_t s) { MISCAN_AFF_DISPATCH(fwd_launch, pl, a, s); }
mi_status dispatch_bwd(const AffPlan &pl, BwdArgs &a, hipStream_t s) { MISCAN_AFF_DISPATCH(bwd_launch, pl, a, s); }

}  // namespace

size_t affine_workspace_bytes(int64_t B, int64_t T, int64_t n, int64_t k, int64_t v) {
    // The column tiling depends on pointer alignment, known only at the call:
    // size for the largest of the tilings either alignment can select.
    size_t m = 0;
    for (int a16 = 0; a16 < 2; ++a16)
        for (int bwd = 0; bwd < 2; ++bwd) {
            const AffPlan pl = choose_plan(B, T, n, (int)k, (int)v, bwd != 0, a16 != 0);
            const size_t w = WsLayout(pl.n_slots, pl.payload).total;
            m = w > m ? w : m;
        }
    return m;
}

mi_status launch_affine_fwd(const void *A, const void *Bm, void *Abar, void *Bbar, int64_t B,
                            int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt, void *ws,
                            size_t ws_bytes, hipStream_t s, bool h0_kernels, const void *H0) {
    const bool p16 = aligned16(A) && aligned16(Bm) && aligned16(Abar) && aligned16(Bbar);
    AffPlan pl = choose_plan(B, T, n, (int)k, (int)v, false, p16);
    if (!pl.ok) return MI_ERR_UNSUPPORTED;
    pl.h0 = h0_kernels;
    pl.dt = dt;
    WsLayout lay(pl.n_slots, pl.payload);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    FwdArgs a;
    a.A = A; a.Bm = Bm; a.Abar = Abar; a.Bbar = Bbar; a.H0 = H0;
    a.T = T; a.heads = B * n; a.n = (int)n; a.k = (int)k; a.v = (int)v;
    a.G = pl.G; a.HPW = pl.HPW; a.NCP = pl.NCP; a.n_groups = pl.n_groups;
    a.n_chunks = pl.n_chunks; a.NW = pl.NW; a.HH = pl.HH; a.DB = pl.DB;
    a.lb_window = pl.W;
    a.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(a.ws, pl.n_slots, s);
    if (st != MI_OK) return st;
    return dispatch_fwd(pl, a, s);
}

mi_status launch_affine_bwd(const void *A, const void *Abar, const void *Bbar,
                            const void *gAbar, const void *gBbar, void *dA, void *dB,
                            int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, mi_dtype dt, void *ws,
                            size_t ws_bytes, hipStream_t s, bool h0_kernels, const void *H0, void *dH0) {
    const void *ptrs[7] = {A, Abar, Bbar, gAbar, gBbar, dA, dB};
    bool p16 = true;
    for (const void *q : ptrs) p16 = p16 && aligned16(q);
    AffPlan pl = choose_plan(B, T, n, (int)k, (int)v, true, p16);
    if (!pl.ok) return MI_ERR_UNSUPPORTED;
    pl.h0 = h0_kernels;
    pl.dt = dt;
    WsLayout lay(pl.n_slots, pl.payload);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    BwdArgs a;
    a.H0 = H0; a.dH0 = dH0;
    a.A = A; a.Abar = Abar; a.Bbar = Bbar; a.gAbar = gAbar; a.gBbar = gBbar; a.dA = dA; a.dB = dB;
    a.T = T; a.heads = B * n; a.n = (int)n; a.k = (int)k; a.v = (int)v;
    a.G = pl.G; a.HPW = pl.HPW; a.NCP = pl.NCP; a.n_groups = pl.n_groups;
    a.n_chunks = pl.n_chunks; a.NW = pl.NW; a.HH = pl.HH; a.DB = pl.DB;
    a.lb_window = pl.W;
    a.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(a.ws, pl.n_slots, s);
    if (st != MI_OK) return st;
    return dispatch_bwd(pl, a, s);
}

}  // namespace miscan
