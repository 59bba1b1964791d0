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
// fp32) in registers; the G = (k+v)/CPL lanes of a head share A_t.  A wave
// holds HPW = 64/G heads that are adjacent in memory, so its loads and stores
// at one time step hit one contiguous run of each tensor.  The k x k products
// are tiny and per step, not a dense contraction: they run on the vector ALU.
//
// One wave is one work item: HPW heads x one chunk of LC time steps.  Pass 1
// composes the chunk's transform [Abar_c | H_c] from [I | 0]; the decoupled
// look-back (common.hpp) yields the state entering the chunk; pass 2 re-reads
// the chunk (the re-read is served by the caches) and writes the true states.
// The look-back needs whole k x k blocks of other lanes' columns: those come
// from the published payloads in memory, or from LDS for the wave's own.
//
// Backward.  Y_t = [M_t | Lam_t] = [gAbar_t | gBbar_t] + A_{t+1}^T Y_{t+1}
// runs in reverse time, again column by column.  A chunk's reverse transform
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

// k x k block (row-major, row stride `ld`) into a KP x KP register tile, zero
// padded.  VIO: k == KP and the rows are vector-aligned.
template <int KP, bool VIO>
__device__ __forceinline__ void load_block(float (&m)[KP][KP], const float *src, int k, int64_t ld) {
    if constexpr (VIO) {
#pragma unroll
        for (int i = 0; i < KP; ++i) ldv<KP>(m[i], src + i * ld);
    } else {
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int j = 0; j < KP; ++j) m[i][j] = (i < k && j < k) ? src[i * ld + j] : 0.f;
    }
}

// One row of a k x k block into KP registers, zero padded; `ok` false gives zeros.
template <int KP, bool VIO>
__device__ __forceinline__ void load_row(float (&r)[KP], const float *src, bool ok, int k) {
    if (ok) {
        if constexpr (VIO) {
            ldv<KP>(r, src);
        } else {
#pragma unroll
            for (int j = 0; j < KP; ++j) r[j] = (j < k) ? src[j] : 0.f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < KP; ++j) r[j] = 0.f;
    }
}

struct FwdArgs {
    const float *A, *Bm;
    float *Abar, *Bbar;
    int64_t T, heads;
    int n, k, v;
    int G, HPW, NCP, n_groups, n_chunks, LC;
    WsPtrs ws;
};

struct BwdArgs {
    const float *A, *Abar, *Bbar, *gAbar, *gBbar;
    float *dA, *dB;
    int64_t T, heads;
    int n, k, v;
    int G, HPW, NCP, n_groups, n_chunks, LC;
    WsPtrs ws;
};

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
template <int KP, int CPL, bool VIO>
__device__ __forceinline__ void fwd_step(float (&x)[KP][CPL], const FwdArgs &p, const Cols<CPL> &cl,
                                         int64_t m, bool active, bool store) {
    const int k = p.k, v = p.v;
    const float *At = p.A + m * k * k;
    const float *Bt = p.Bm + m * k * v;
    float nx[KP][CPL];
    // nx = [0 | B_t] for the lane's columns
    if constexpr (VIO) {
        if (active && cl.kind[0] == C_H) {
#pragma unroll
            for (int i = 0; i < KP; ++i) ldv<CPL>(nx[i], Bt + i * v + cl.col[0]);
        } else {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) nx[i][cc] = 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc)
                nx[i][cc] = (active && cl.kind[cc] == C_H && i < k) ? Bt[i * v + cl.col[cc]] : 0.f;
    }
    // nx[i] += sum_j A_t[i][j] x[j], one row of A_t at a time
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        float arow[KP];
        load_row<KP, VIO>(arow, At + i * k, active && i < k, k);
#pragma unroll
        for (int j = 0; j < KP; ++j)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) nx[i][cc] = fmaf(arow[j], x[j][cc], nx[i][cc]);
    }
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[i][cc] = nx[i][cc];

    if (store && active) {
        if constexpr (VIO) {
            if (cl.kind[0] != C_PAD) {
                float *dst = (cl.kind[0] == C_ABAR) ? p.Abar + m * k * k + cl.col[0]
                                                    : p.Bbar + m * k * v + cl.col[0];
                const int ld = (cl.kind[0] == C_ABAR) ? k : v;
#pragma unroll
                for (int i = 0; i < KP; ++i) stv<CPL, true>(dst + i * ld, x[i]);
            }
        } else {
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
#pragma unroll
                for (int i = 0; i < KP; ++i) {
                    if (i < k && cl.kind[cc] == C_ABAR) p.Abar[m * k * k + i * k + cl.col[cc]] = x[i][cc];
                    if (i < k && cl.kind[cc] == C_H) p.Bbar[m * k * v + i * v + cl.col[cc]] = x[i][cc];
                }
            }
        }
    }
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
template <int KP, int CPL>
__device__ __forceinline__ void payload_load(float (&x)[KP][CPL], const float *blk, int NCP, int c0) {
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) x[i][cc] = carry_load(blk + i * NCP + c0 + cc);
}

// S <- M S (+ add where addmask), column by column.  M is the leading k x k
// block (zero padded to KP) of a row-major matrix with row stride `ld`, read
// either from a published payload (PAYLOAD: device-coherent word loads) or
// from LDS.
template <int KP, int CPL, bool PAYLOAD>
__device__ __forceinline__ void mat_apply(float (&S)[KP][CPL], const float *Msrc, int64_t ld, int k,
                                          const float (&add)[KP][CPL], const bool (&addmask)[CPL]) {
    float ns[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i) {
        float mrow[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) {
            const bool in = i < k && j < k;
            if constexpr (PAYLOAD) mrow[j] = in ? carry_load(Msrc + i * ld + j) : 0.f;
            else mrow[j] = in ? Msrc[i * ld + j] : 0.f;
        }
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
            float s = addmask[cc] ? add[i][cc] : 0.f;
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

template <int KP, int CPL, bool VIO>
__global__ __launch_bounds__(64) void affine_fwd_kernel(FwdArgs p) {
    extern __shared__ float s_dyn[];
    float *s_abar = s_dyn;  // [HPW][KP][KP]: this chunk's Abar_c per head, zero padded

    const int lane = threadIdx.x;
    uint32_t tk = 0;
    if (lane == 0) tk = take_ticket(p.ws.hdr);
    const int ticket = __shfl((int)tk, 0);
    const int chunk = ticket / p.n_groups;
    const int grp = ticket - chunk * p.n_groups;
    const int hs = lane / p.G;
    const int g = lane - hs * p.G;
    const bool slot_lane = hs < p.HPW;  // lane maps to a head slot of this wave
    const int hsc = slot_lane ? hs : 0;
    const int64_t gh = (int64_t)grp * p.HPW + hs;
    const bool active = slot_lane && gh < p.heads;
    const int64_t bidx = active ? gh / p.n : 0;
    const int64_t hh = active ? gh % p.n : 0;
    const int k = p.k;
    const int c0 = g * CPL;

    for (int i = lane; i < p.HPW * KP * KP; i += 64) s_abar[i] = 0.f;

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

    const int64_t t_begin = (int64_t)chunk * p.LC;
    const int64_t t_end = (t_begin + p.LC < p.T) ? t_begin + p.LC : p.T;
    const int64_t m0 = bidx * p.T * p.n + hh;  // matrix index of (b, t=0, h); + t*n per step

    // Pass 1: the chunk's transform [Abar_c | H_c] from [I | 0].
    float x[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
            x[i][cc] = (cl.kind[cc] == C_ABAR && i == cl.col[cc]) ? 1.f : 0.f;
    for (int64_t t = t_begin; t < t_end; ++t)
        fwd_step<KP, CPL, VIO>(x, p, cl, m0 + t * p.n, active, false);

    // Abar_c of each head to LDS, written by the lanes that own its columns.
    __syncthreads();
    if (slot_lane) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
            if (cl.kind[cc] == C_ABAR)
#pragma unroll
                for (int i = 0; i < KP; ++i) s_abar[(hs * KP + i) * KP + cl.col[cc]] = x[i][cc];
    }
    __syncthreads();

    // Look-back: the state S entering the chunk ([I | 0] before chunk 0).
    const int64_t slot_sz = (int64_t)p.HPW * KP * p.NCP;
    const int64_t hoff = (int64_t)hsc * KP * p.NCP;
    const int64_t slot = (int64_t)grp * p.n_chunks + chunk;
    float S[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
            S[i][cc] = (cl.kind[cc] == C_ABAR && i == cl.col[cc]) ? 1.f : 0.f;
    if (chunk > 0) {
        if (slot_lane) payload_store<KP, CPL>(p.ws.agg + slot * slot_sz + hoff, p.NCP, c0, x);
        const int dist = wait_ready(p.ws.flags, slot - 1, -1, chunk, p.ws.hdr + 1, p.ws.flags + slot, FLAG_AGG);
        const int j0 = chunk - 1 - dist;
        // slot j0 holds an inclusive state; chunks j0+1 .. chunk-1 hold transforms
        payload_load<KP, CPL>(S, p.ws.inc + ((int64_t)grp * p.n_chunks + j0) * slot_sz + hoff,
                                   p.NCP, c0);
        for (int jj = j0 + 1; jj < chunk; ++jj) {
            const float *blk = p.ws.agg + ((int64_t)grp * p.n_chunks + jj) * slot_sz + hoff;
            float Hx[KP][CPL];
            payload_load<KP, CPL>(Hx, blk, p.NCP, c0);
            mat_apply<KP, CPL, true>(S, blk, p.NCP, k, Hx, is_h);
        }
    }
    // Inclusive state after this chunk: [Abar_c | H_c] applied to S.
    {
        float inc[KP][CPL];
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) inc[i][cc] = S[i][cc];
        mat_apply<KP, CPL, false>(inc, s_abar + hsc * KP * KP, KP, KP, x, is_h);
        if (slot_lane) payload_store<KP, CPL>(p.ws.inc + slot * slot_sz + hoff, p.NCP, c0, inc);
        publish_flag(p.ws.flags + slot, FLAG_INC);
    }

    // Pass 2: rescan the chunk from S and store Abar_t, Bbar_t.
    for (int64_t t = t_begin; t < t_end; ++t)
        fwd_step<KP, CPL, VIO>(S, p, cl, m0 + t * p.n, active, true);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------

// z <- G_t + A_{t+1}^T z for the lane's columns; A_{T+1} = 0.
template <int KP, int CPL, bool VIO>
__device__ __forceinline__ void bwd_scan_step(float (&z)[KP][CPL], const BwdArgs &p, const Cols<CPL> &cl,
                                              int64_t m, int64_t t, bool active) {
    const int k = p.k, v = p.v;
    float nz[KP][CPL];
    if constexpr (VIO) {
        if (active && cl.kind[0] == Z_M) {
#pragma unroll
            for (int i = 0; i < KP; ++i) ldv<CPL>(nz[i], p.gAbar + m * k * k + i * k + cl.col[0]);
        } else if (active && cl.kind[0] == Z_L) {
#pragma unroll
            for (int i = 0; i < KP; ++i) ldv<CPL>(nz[i], p.gBbar + m * k * v + i * v + cl.col[0]);
        } else {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) nz[i][cc] = 0.f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) {
                float gv = 0.f;
                if (active && i < k) {
                    if (cl.kind[cc] == Z_M) gv = p.gAbar[m * k * k + i * k + cl.col[cc]];
                    else if (cl.kind[cc] == Z_L) gv = p.gBbar[m * k * v + i * v + cl.col[cc]];
                }
                nz[i][cc] = gv;
            }
    }
    // nz[i] += sum_j A_{t+1}[j][i] z[j], one row j of A_{t+1} at a time
    const bool has_next = active && t + 1 < p.T;
    const float *An = p.A + (m + p.n) * k * k;
#pragma unroll
    for (int j = 0; j < KP; ++j) {
        float arow[KP];
        load_row<KP, VIO>(arow, An + j * k, has_next && j < k, k);
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) nz[i][cc] = fmaf(arow[i], z[j][cc], nz[i][cc]);
    }
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) z[i][cc] = nz[i][cc];
}

template <int KP> struct RowBlock { static constexpr int RB = KP < 8 ? KP : 8; };

template <int KP, int CPL, bool VIO>
__global__ __launch_bounds__(64) void affine_bwd_kernel(BwdArgs p) {
    constexpr int RB = RowBlock<KP>::RB;
    extern __shared__ float s_dyn[];
    float *s_P = s_dyn;                        // [HPW][KP][KP]: this chunk's P_c
    float *s_part = s_dyn + p.HPW * KP * KP;   // [HPW][G][RB][KP]: dA partial sums

    const int lane = threadIdx.x;
    uint32_t tk = 0;
    if (lane == 0) tk = take_ticket(p.ws.hdr);
    const int ticket = __shfl((int)tk, 0);
    const int rchunk = ticket / p.n_groups;
    const int grp = ticket - rchunk * p.n_groups;
    const int chunk = p.n_chunks - 1 - rchunk;
    const int hs = lane / p.G;
    const int g = lane - hs * p.G;
    const bool slot_lane = hs < p.HPW;
    const int hsc = slot_lane ? hs : 0;
    const int64_t gh = (int64_t)grp * p.HPW + hs;
    const bool active = slot_lane && gh < p.heads;
    const int64_t bidx = active ? gh / p.n : 0;
    const int64_t hh = active ? gh % p.n : 0;
    const int k = p.k, v = p.v;
    const int c0 = g * CPL;

    for (int i = lane; i < p.HPW * KP * KP; i += 64) s_P[i] = 0.f;

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

    const int64_t t_begin = (int64_t)chunk * p.LC;
    const int64_t t_end = (t_begin + p.LC < p.T) ? t_begin + p.LC : p.T;
    const int64_t m0 = bidx * p.T * p.n + hh;

    // Pass 1 (reverse): Z_c = [P_c | Y_c] from [I | 0 | 0].
    float z[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) z[i][cc] = (cl.kind[cc] == Z_P && i == cl.col[cc]) ? 1.f : 0.f;
    for (int64_t t = t_end - 1; t >= t_begin; --t)
        bwd_scan_step<KP, CPL, VIO>(z, p, cl, m0 + t * p.n, t, active);

    __syncthreads();
    if (slot_lane) {
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
            if (cl.kind[cc] == Z_P)
#pragma unroll
                for (int i = 0; i < KP; ++i) s_P[(hs * KP + i) * KP + cl.col[cc]] = z[i][cc];
    }
    __syncthreads();

    // Look-back over later chunks: Y entering this chunk from the future
    // (zero after the last chunk).
    const int64_t slot_sz = (int64_t)p.HPW * KP * p.NCP;
    const int64_t hoff = (int64_t)hsc * KP * p.NCP;
    const int64_t slot = (int64_t)grp * p.n_chunks + chunk;
    const int last = p.n_chunks - 1;
    float S[KP][CPL];
#pragma unroll
    for (int i = 0; i < KP; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) S[i][cc] = 0.f;
    if (chunk < last) {
        if (slot_lane) payload_store<KP, CPL>(p.ws.agg + slot * slot_sz + hoff, p.NCP, c0, z);
        const int dist = wait_ready(p.ws.flags, slot + 1, +1, last - chunk, p.ws.hdr + 1, p.ws.flags + slot,
                                    FLAG_AGG);
        const int j0 = chunk + 1 + dist;
        payload_load<KP, CPL>(S, p.ws.inc + ((int64_t)grp * p.n_chunks + j0) * slot_sz + hoff,
                                   p.NCP, c0);
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) S[i][cc] = is_y[cc] ? S[i][cc] : 0.f;
        for (int jj = j0 - 1; jj > chunk; --jj) {
            const float *blk = p.ws.agg + ((int64_t)grp * p.n_chunks + jj) * slot_sz + hoff;
            float Yl[KP][CPL];
            payload_load<KP, CPL>(Yl, blk, p.NCP, c0);
            mat_apply<KP, CPL, true>(S, blk, p.NCP, k, Yl, is_y);
        }
    }
    {
        float inc[KP][CPL];
#pragma unroll
        for (int i = 0; i < KP; ++i)
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) inc[i][cc] = S[i][cc];
        mat_apply<KP, CPL, false>(inc, s_P + hsc * KP * KP, KP, KP, z, is_y);
        if (slot_lane) payload_store<KP, CPL>(p.ws.inc + slot * slot_sz + hoff, p.NCP, c0, inc);
        publish_flag(p.ws.flags + slot, FLAG_INC);
    }

    // Pass 2 (reverse): true Y_t from S; dB_t = Lam_t; dA_t = Y_t X_{t-1}^T.
    float *part_mine = s_part + ((int64_t)(hsc * p.G + g) * RB) * KP;
    const float *part_head = s_part + (int64_t)hsc * p.G * RB * KP;
    for (int64_t t = t_end - 1; t >= t_begin; --t) {
        const int64_t m = m0 + t * p.n;
        bwd_scan_step<KP, CPL, VIO>(S, p, cl, m, t, active);

        // X_{t-1} columns matching the lane's Y columns ([I | 0] at t = 0).
        float xp[KP][CPL];
        if constexpr (VIO) {
            if (active && t > 0 && cl.kind[0] == Z_M) {
#pragma unroll
                for (int i = 0; i < KP; ++i) ldv<CPL>(xp[i], p.Abar + (m - p.n) * k * k + i * k + cl.col[0]);
            } else if (active && t > 0 && cl.kind[0] == Z_L) {
#pragma unroll
                for (int i = 0; i < KP; ++i) ldv<CPL>(xp[i], p.Bbar + (m - p.n) * k * v + i * v + cl.col[0]);
            } else {
#pragma unroll
                for (int i = 0; i < KP; ++i)
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc)
                        xp[i][cc] = (t == 0 && cl.kind[cc] == Z_M && i == cl.col[cc]) ? 1.f : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < KP; ++i)
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc) {
                    float xv = 0.f;
                    if (active && i < k) {
                        if (cl.kind[cc] == Z_M)
                            xv = (t > 0) ? p.Abar[(m - p.n) * k * k + i * k + cl.col[cc]]
                                         : (i == cl.col[cc] ? 1.f : 0.f);
                        else if (cl.kind[cc] == Z_L && t > 0)
                            xv = p.Bbar[(m - p.n) * k * v + i * v + cl.col[cc]];
                    }
                    xp[i][cc] = xv;
                }
        }

        // dB_t = Lam_t (own Lam columns).
        if (active) {
            if constexpr (VIO) {
                if (cl.kind[0] == Z_L) {
#pragma unroll
                    for (int i = 0; i < KP; ++i) stv<CPL, true>(p.dB + m * k * v + i * v + cl.col[0], S[i]);
                }
            } else {
#pragma unroll
                for (int cc = 0; cc < CPL; ++cc)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        if (i < k && cl.kind[cc] == Z_L) p.dB[m * k * v + i * v + cl.col[cc]] = S[i][cc];
            }
        }

        // dA_t rows in blocks of RB: partial sums over the lane's own columns,
        // then the head's lanes add the G partials of each row through LDS.
#pragma unroll
        for (int ib = 0; ib < KP; ib += RB) {
            if (slot_lane) {
#pragma unroll
                for (int ii = 0; ii < RB; ++ii) {
                    float row[KP];
#pragma unroll
                    for (int j = 0; j < KP; ++j) row[j] = 0.f;
#pragma unroll
                    for (int cc = 0; cc < CPL; ++cc) {
                        const float y = is_y[cc] ? S[ib + ii][cc] : 0.f;
#pragma unroll
                        for (int j = 0; j < KP; ++j) row[j] = fmaf(y, xp[j][cc], row[j]);
                    }
                    stv<KP, false>(part_mine + ii * KP, row);
                }
            }
            __syncthreads();
            if (active) {
                for (int ii = g; ii < RB; ii += p.G) {
                    const int i = ib + ii;
                    if (i < k) {
                        float acc[KP];
#pragma unroll
                        for (int j = 0; j < KP; ++j) acc[j] = 0.f;
                        for (int gg = 0; gg < p.G; ++gg) {
                            float q[KP];
                            ldv<KP>(q, part_head + ((int64_t)gg * RB + ii) * KP);
#pragma unroll
                            for (int j = 0; j < KP; ++j) acc[j] += q[j];
                        }
                        float *dst = p.dA + m * k * k + (int64_t)i * k;
                        if constexpr (VIO) {
                            stv<KP, true>(dst, acc);
                        } else {
#pragma unroll
                            for (int j = 0; j < KP; ++j)
                                if (j < k) dst[j] = acc[j];
                        }
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: tile selection and launch.
// ---------------------------------------------------------------------------
#ifndef MISCAN_AFF_LC
#define MISCAN_AFF_LC 32
#endif
constexpr int LC_STEPS = MISCAN_AFF_LC;  // time steps per work item

struct AffPlan {
    int KP, CPL;
    bool VIO;
    int G, HPW, NCP, n_groups, n_chunks, LC, RB;
    size_t n_slots, payload, lds_bytes;
    bool ok;  // the work-item count fits the int32 ticket space
};

inline int next_pow2_16(int k) { return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16; }

inline AffPlan make_plan(int64_t B, int64_t T, int64_t n, int k, int ncols, bool bwd, int CPL, bool VIO) {
    AffPlan pl;
    pl.KP = next_pow2_16(k);
    pl.CPL = CPL;
    pl.VIO = VIO;
    pl.G = (ncols + CPL - 1) / CPL;
    pl.HPW = 64 / pl.G;
    pl.NCP = (int)round_up((size_t)pl.G * CPL, 4);
    const int64_t heads = B * n;
    const int64_t ng = (heads + pl.HPW - 1) / pl.HPW;
    pl.LC = LC_STEPS;
    const int64_t nc = (T + pl.LC - 1) / pl.LC;
    pl.ok = ng <= INT32_MAX && nc <= INT32_MAX && ng * nc <= (int64_t)INT32_MAX;
    pl.n_groups = (int)ng;
    pl.n_chunks = (int)nc;
    pl.RB = pl.KP < 8 ? pl.KP : 8;
    pl.n_slots = pl.ok ? (size_t)ng * (size_t)nc : 0;
    pl.payload = (size_t)pl.HPW * pl.KP * pl.NCP;
    pl.lds_bytes = sizeof(float) * (size_t)pl.HPW * pl.KP * pl.KP;
    if (bwd) pl.lds_bytes += sizeof(float) * (size_t)pl.HPW * pl.G * pl.RB * pl.KP;
    return pl;
}

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

// Vector IO needs k to be a power of two (rows load as vectors), k and v to be
// multiples of CPL (column groups never straddle tensors), 16-byte aligned
// base pointers, and a head to fit one wave (G <= 64).  Otherwise four
// columns per lane with element-wise accesses.
inline void choose_cols(int k, int v, int ncols, bool ptrs16, int &CPL, bool &VIO) {
    const bool kpow2 = next_pow2_16(k) == k;
    if (ptrs16 && kpow2 && k % 4 == 0 && v % 4 == 0) { CPL = 4; VIO = true; return; }
    if (ptrs16 && kpow2 && k % 2 == 0 && v % 2 == 0 && (ncols + 1) / 2 <= 64) { CPL = 2; VIO = true; return; }
    CPL = 4;
    VIO = false;
}

template <int KP, int CPL, bool VIO>
mi_status fwd_launch(const AffPlan &pl, FwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((affine_fwd_kernel<KP, CPL, VIO>), dim3((unsigned)pl.n_slots), dim3(64),
                       pl.lds_bytes, s, a);
    return launch_status();
}
template <int KP, int CPL, bool VIO>
mi_status bwd_launch(const AffPlan &pl, BwdArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((affine_bwd_kernel<KP, CPL, VIO>), dim3((unsigned)pl.n_slots), dim3(64),
                       pl.lds_bytes, s, a);
    return launch_status();
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
    for (int bwd = 0; bwd < 2; ++bwd) {
        const int nc = (int)(bwd ? 2 * k + v : k + v);
        for (int a16 = 0; a16 < 2; ++a16) {
            int CPL;
            bool VIO;
            choose_cols((int)k, (int)v, nc, a16 != 0, CPL, VIO);
            AffPlan pl = make_plan(B, T, n, (int)k, nc, bwd != 0, CPL, VIO);
            const size_t w = WsLayout(pl.n_slots, pl.payload).total;
            m = w > m ? w : m;
        }
    }
    return m;
}

mi_status launch_affine_fwd(const void *A, const void *Bm, void *Abar, void *Bbar, int64_t B,
                            int64_t T, int64_t n, int64_t k, int64_t v, void *ws,
                            size_t ws_bytes, hipStream_t s) {
    const bool p16 = aligned16(A) && aligned16(Bm) && aligned16(Abar) && aligned16(Bbar);
    const int nc = (int)(k + v);
    int CPL;
    bool VIO;
    choose_cols((int)k, (int)v, nc, p16, CPL, VIO);
    AffPlan pl = make_plan(B, T, n, (int)k, nc, false, CPL, VIO);
    if (!pl.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(pl.n_slots, pl.payload);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    FwdArgs a;
    a.A = static_cast<const float *>(A); a.Bm = static_cast<const float *>(Bm);
    a.Abar = static_cast<float *>(Abar); a.Bbar = static_cast<float *>(Bbar);
    a.T = T; a.heads = B * n; a.n = (int)n; a.k = (int)k; a.v = (int)v;
    a.G = pl.G; a.HPW = pl.HPW; a.NCP = pl.NCP; a.n_groups = pl.n_groups;
    a.n_chunks = pl.n_chunks; a.LC = pl.LC;
    a.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(a.ws, pl.n_slots, s);
    if (st != MI_OK) return st;
    return dispatch_fwd(pl, a, s);
}

mi_status launch_affine_bwd(const void *A, const void *Abar, const void *Bbar,
                            const void *gAbar, const void *gBbar, void *dA, void *dB,
                            int64_t B, int64_t T, int64_t n, int64_t k, int64_t v, void *ws,
                            size_t ws_bytes, hipStream_t s) {
    const void *ptrs[7] = {A, Abar, Bbar, gAbar, gBbar, dA, dB};
    bool p16 = true;
    for (const void *q : ptrs) p16 = p16 && aligned16(q);
    const int nc = (int)(2 * k + v);
    int CPL;
    bool VIO;
    choose_cols((int)k, (int)v, nc, p16, CPL, VIO);
    AffPlan pl = make_plan(B, T, n, (int)k, nc, true, CPL, VIO);
    if (!pl.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(pl.n_slots, pl.payload);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    BwdArgs a;
    a.A = static_cast<const float *>(A); a.Abar = static_cast<const float *>(Abar);
    a.Bbar = static_cast<const float *>(Bbar); a.gAbar = static_cast<const float *>(gAbar);
    a.gBbar = static_cast<const float *>(gBbar);
    a.dA = static_cast<float *>(dA); a.dB = static_cast<float *>(dB);
    a.T = T; a.heads = B * n; a.n = (int)n; a.k = (int)k; a.v = (int)v;
    a.G = pl.G; a.HPW = pl.HPW; a.NCP = pl.NCP; a.n_groups = pl.n_groups;
    a.n_chunks = pl.n_chunks; a.LC = pl.LC;
    a.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(a.ws, pl.n_slots, s);
    if (st != MI_OK) return st;
    return dispatch_bwd(pl, a, s);
}

}  // namespace miscan
