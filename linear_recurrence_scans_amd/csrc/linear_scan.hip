// linear_scan.hip -- k = 1 channel scan h_t = a_t h_{t-1} + b_t and its adjoint.
//
// Operations: minGRU docs, "Triton kernels" page, Kernel entry points,
// linear_scan_fwd (A = running product of a, Bc = h_0 = 0 solution) and
// linear_scan_bwd (grads w.r.t. a and b from a, A, Bc, gA, gBc).
//
// Layout: (B, T, D) row-major; D is innermost, so one time row of one batch is
// D contiguous elements.  Mapping (one workgroup = one work item):
//   - lanes run along channels: lane l of every wave owns channels
//     [tile*64*VEC + l*VEC, +VEC) and moves them with one VEC-wide access per
//     row (16 bytes for fp32 x4 and bf16 x8), so each wave-wide load or store
//     covers 64*VEC contiguous channels;
//   - waves run along time: wave w of the workgroup owns rows
//     [chunk*NW*L + w*L, +L) and scans them serially in registers;
//   - the NW wave aggregates are combined through LDS, the chunk's carry-in
//     comes from the decoupled look-back over earlier chunks of the same tile
//     (common.hpp), and each wave then rescans its rows from registers with
//     its carry-in and stores the results.
// HBM traffic is one read of every input and one write of every output, plus
// per chunk the carry payload (2 or 3 fp32 per channel) and, in the backward,
// one halo row of a, A and Bc.
#include "common.hpp"
#include "internal.hpp"

namespace miscan {
namespace {

struct FwdArgs {
    const void *a, *b;
    void *A, *Bc;
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    WsPtrs ws;
};

struct BwdArgs {
    const void *a, *A, *Bc, *gA, *gBc;
    void *da, *db;
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    WsPtrs ws;
};

template <int N>
__device__ __forceinline__ void store_floats(float *dst, const float *src) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            f32x4 v = {src[i], src[i + 1], src[i + 2], src[i + 3]};
            *reinterpret_cast<f32x4 *>(dst + i) = v;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            f32x2 v = {src[i], src[i + 1]};
            *reinterpret_cast<f32x2 *>(dst + i) = v;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}

template <int N>
__device__ __forceinline__ void load_floats(float *dst, const float *src) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(src + i);
            dst[i] = v.x; dst[i + 1] = v.y; dst[i + 2] = v.z; dst[i + 3] = v.w;
        }
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            f32x2 v = *reinterpret_cast<const f32x2 *>(src + i);
            dst[i] = v.x; dst[i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = src[i];
    }
}

// ---------------------------------------------------------------------------
// Forward.  Per channel the segment transform is (A, h): h_out = A*h_in + h.
// Composition, earlier segment 1 then later segment 2:
//     (A1, h1) then (A2, h2) = (A2*A1, A2*h1 + h2).
// ---------------------------------------------------------------------------
template <typename T, int VEC, int L, int NW>
__global__ __launch_bounds__(NW * 64) void linear_fwd_kernel(FwdArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC;
    constexpr int CHUNK = NW * L;
    constexpr int NV = 2 * VEC;  // payload floats per lane: A[VEC], h[VEC]

    __shared__ float s_A[NW][TILE];
    __shared__ float s_H[NW][TILE];
    __shared__ float s_cA[TILE];
    __shared__ float s_cH[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)s_ticket;
    const int chunk = ticket / p.n_tiles;
    const int tile = ticket - chunk * p.n_tiles;
    const int bidx = tile / p.n_dtiles;
    const int dtile = tile - bidx * p.n_dtiles;

    const int64_t d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    const bool lane_ok = d < p.D;
    const int64_t t0 = (int64_t)chunk * CHUNK + (int64_t)wave * L;
    const int64_t base = ((int64_t)bidx * p.T + t0) * p.D + d;
    const T *a = static_cast<const T *>(p.a) + base;
    const T *b = static_cast<const T *>(p.b) + base;

    // 1. Load this wave's L rows (identity step (1, 0) past T or past D).
    raw_t ra[L], rb[L];
#pragma unroll
    for (int r = 0; r < L; ++r) {
        if (lane_ok && t0 + r < p.T) {
            ra[r] = load_vec<T, VEC>(a + r * p.D);
            rb[r] = load_vec<T, VEC>(b + r * p.D);
        } else {
            ra[r] = splat<T, VEC>(1.f);
            rb[r] = splat<T, VEC>(0.f);
        }
    }

    // 2. Serial scan of the wave's rows from (1, 0): the wave aggregate.
    float gA[VEC], gH[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { gA[v] = 1.f; gH[v] = 0.f; }
#pragma unroll
    for (int r = 0; r < L; ++r) {
        float fa[VEC], fb[VEC];
        PK::unpack(ra[r], fa);
        PK::unpack(rb[r], fb);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            gH[v] = fmaf(fa[v], gH[v], fb[v]);
            gA[v] = fa[v] * gA[v];
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        s_A[wave][lane * VEC + v] = gA[v];
        s_H[wave][lane * VEC + v] = gH[v];
    }
    __syncthreads();

    // 3. Wave 0: chunk aggregate, publish, look back, publish inclusive prefix.
    if (wave == 0) {
        float c[NV];  // chunk aggregate: c[0..VEC) = A, c[VEC..2VEC) = h
#pragma unroll
        for (int v = 0; v < VEC; ++v) { c[v] = 1.f; c[VEC + v] = 0.f; }
        for (int w = 0; w < NW; ++w) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float xA = s_A[w][lane * VEC + v], xH = s_H[w][lane * VEC + v];
                c[VEC + v] = fmaf(xA, c[VEC + v], xH);
                c[v] = xA * c[v];
            }
        }
        float in[NV];  // carry-in = inclusive prefix of all earlier chunks
#pragma unroll
        for (int v = 0; v < VEC; ++v) { in[v] = 1.f; in[VEC + v] = 0.f; }
        const int64_t slot = (int64_t)tile * p.n_chunks + chunk;
        const int64_t lane_off = (int64_t)lane * NV;
        if (chunk > 0) {
            store_floats<NV>(p.ws.agg + slot * (64 * NV) + lane_off, c);
            publish_flag(p.ws.flags + slot, FLAG_AGG);
            for (int j = chunk - 1; j >= 0; --j) {
                const int64_t sj = (int64_t)tile * p.n_chunks + j;
                const uint32_t f = wait_flag(p.ws.flags + sj, p.ws.hdr + 1);
                const float *src = (f == FLAG_INC ? p.ws.inc : p.ws.agg) + sj * (64 * NV) + lane_off;
                float x[NV];
                load_floats<NV>(x, src);
                // slot j comes before everything folded so far
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    in[VEC + v] = fmaf(in[v], x[VEC + v], in[VEC + v]);
                    in[v] = in[v] * x[v];
                }
                if (f == FLAG_INC) break;
            }
        }
        float inc[NV];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            inc[v] = c[v] * in[v];
            inc[VEC + v] = fmaf(c[v], in[VEC + v], c[VEC + v]);
        }
        store_floats<NV>(p.ws.inc + slot * (64 * NV) + lane_off, inc);
        publish_flag(p.ws.flags + slot, FLAG_INC);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            s_cA[lane * VEC + v] = in[v];
            s_cH[lane * VEC + v] = in[VEC + v];
        }
    }
    __syncthreads();

    // 4. Carry into this wave: chunk carry-in, then waves 0..wave-1.
    float hA[VEC], hH[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { hA[v] = s_cA[lane * VEC + v]; hH[v] = s_cH[lane * VEC + v]; }
    for (int w = 0; w < wave; ++w) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float xA = s_A[w][lane * VEC + v], xH = s_H[w][lane * VEC + v];
            hH[v] = fmaf(xA, hH[v], xH);
            hA[v] = xA * hA[v];
        }
    }

    // 5. Rescan the rows from registers and store A_t, Bc_t.
    if (!lane_ok) return;
    T *Ao = static_cast<T *>(p.A) + base;
    T *Bo = static_cast<T *>(p.Bc) + base;
#pragma unroll
    for (int r = 0; r < L; ++r) {
        if (t0 + r < p.T) {
            float fa[VEC], fb[VEC];
            PK::unpack(ra[r], fa);
            PK::unpack(rb[r], fb);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                hA[v] = fa[v] * hA[v];
                hH[v] = fmaf(fa[v], hH[v], fb[v]);
            }
            store_vec<T, VEC>(Ao + r * p.D, PK::pack(hA));
            store_vec<T, VEC>(Bo + r * p.D, PK::pack(hH));
        }
    }
}

// ---------------------------------------------------------------------------
// Backward.  Reverse time with c_t = a_{t+1} (c_T = 0):
//     lam_t = gBc_t + c_t lam_{t+1},  mu_t = gA_t + c_t mu_{t+1},
//     db_t = lam_t,  da_t = lam_t Bc_{t-1} + mu_t A_{t-1}  (A_0 = 1, Bc_0 = 0).
// A reverse segment is (P, l, m): lam_out = P*lam_in + l, mu_out = P*mu_in + m.
// Applying later segment 2 first, then earlier segment 1:
//     (P1*P2, P1*l2 + l1, P1*m2 + m1).
// ---------------------------------------------------------------------------
template <typename T, int VEC, int L, int NW>
__global__ __launch_bounds__(NW * 64) void linear_bwd_kernel(BwdArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC;
    constexpr int CHUNK = NW * L;
    constexpr int NV = 3 * VEC;  // payload floats per lane: P[VEC], lam[VEC], mu[VEC]

    __shared__ float s_P[NW][TILE];
    __shared__ float s_L[NW][TILE];
    __shared__ float s_M[NW][TILE];
    __shared__ float s_cP[TILE];
    __shared__ float s_cL[TILE];
    __shared__ float s_cM[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)s_ticket;
    const int rchunk = ticket / p.n_tiles;  // 0 = last chunk in time
    const int tile = ticket - rchunk * p.n_tiles;
    const int chunk = p.n_chunks - 1 - rchunk;
    const int bidx = tile / p.n_dtiles;
    const int dtile = tile - bidx * p.n_dtiles;

    const int64_t d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    const bool lane_ok = d < p.D;
    const int64_t t0 = (int64_t)chunk * CHUNK + (int64_t)wave * L;
    const int64_t base = ((int64_t)bidx * p.T + t0) * p.D + d;
    const T *a = static_cast<const T *>(p.a) + base;
    const T *Ai = static_cast<const T *>(p.A) + base;
    const T *Bci = static_cast<const T *>(p.Bc) + base;
    const T *gA = static_cast<const T *>(p.gA) + base;
    const T *gB = static_cast<const T *>(p.gBc) + base;

    // 1. Loads.  Row r is time t = t0 + r.  c = a_{t+1}; Ap = A_{t-1}; Bp = Bc_{t-1}.
    raw_t rc[L], rgA[L], rgB[L], rAp[L], rBp[L];
#pragma unroll
    for (int r = 0; r < L; ++r) {
        const int64_t t = t0 + r;
        const bool ok = lane_ok && t < p.T;
        rc[r] = (ok && t + 1 < p.T) ? load_vec<T, VEC>(a + (r + 1) * p.D)
                                    : splat<T, VEC>(ok ? 0.f : 1.f);
        rgA[r] = ok ? load_vec<T, VEC>(gA + r * p.D) : splat<T, VEC>(0.f);
        rgB[r] = ok ? load_vec<T, VEC>(gB + r * p.D) : splat<T, VEC>(0.f);
        rAp[r] = (ok && t > 0) ? load_vec<T, VEC>(Ai + (r - 1) * p.D) : splat<T, VEC>(1.f);
        rBp[r] = (ok && t > 0) ? load_vec<T, VEC>(Bci + (r - 1) * p.D) : splat<T, VEC>(0.f);
    }

    // 2. Reverse serial scan of the wave's rows: the wave aggregate.
    float gP[VEC], gL[VEC], gM[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { gP[v] = 1.f; gL[v] = 0.f; gM[v] = 0.f; }
#pragma unroll
    for (int r = L - 1; r >= 0; --r) {
        float fc[VEC], fgA[VEC], fgB[VEC];
        PK::unpack(rc[r], fc);
        PK::unpack(rgA[r], fgA);
        PK::unpack(rgB[r], fgB);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            gL[v] = fmaf(fc[v], gL[v], fgB[v]);
            gM[v] = fmaf(fc[v], gM[v], fgA[v]);
            gP[v] = fc[v] * gP[v];
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        s_P[wave][lane * VEC + v] = gP[v];
        s_L[wave][lane * VEC + v] = gL[v];
        s_M[wave][lane * VEC + v] = gM[v];
    }
    __syncthreads();

    // 3. Wave 0: chunk aggregate (waves NW-1 .. 0), publish, look back over
    //    later chunks, publish the inclusive suffix.
    if (wave == 0) {
        float c[NV];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { c[v] = 1.f; c[VEC + v] = 0.f; c[2 * VEC + v] = 0.f; }
        for (int w = NW - 1; w >= 0; --w) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int i = lane * VEC + v;
                const float xP = s_P[w][i], xL = s_L[w][i], xM = s_M[w][i];
                c[VEC + v] = fmaf(xP, c[VEC + v], xL);
                c[2 * VEC + v] = fmaf(xP, c[2 * VEC + v], xM);
                c[v] = xP * c[v];
            }
        }
        float in[NV];
#pragma unroll
        for (int v = 0; v < VEC; ++v) { in[v] = 1.f; in[VEC + v] = 0.f; in[2 * VEC + v] = 0.f; }
        const int64_t slot = (int64_t)tile * p.n_chunks + chunk;
        const int64_t lane_off = (int64_t)lane * NV;
        if (chunk < p.n_chunks - 1) {
            store_floats<NV>(p.ws.agg + slot * (64 * NV) + lane_off, c);
            publish_flag(p.ws.flags + slot, FLAG_AGG);
            for (int j = chunk + 1; j < p.n_chunks; ++j) {
                const int64_t sj = (int64_t)tile * p.n_chunks + j;
                const uint32_t f = wait_flag(p.ws.flags + sj, p.ws.hdr + 1);
                const float *src = (f == FLAG_INC ? p.ws.inc : p.ws.agg) + sj * (64 * NV) + lane_off;
                float x[NV];
                load_floats<NV>(x, src);
                // slot j is applied before everything folded so far
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    in[VEC + v] = fmaf(in[v], x[VEC + v], in[VEC + v]);
                    in[2 * VEC + v] = fmaf(in[v], x[2 * VEC + v], in[2 * VEC + v]);
                    in[v] = in[v] * x[v];
                }
                if (f == FLAG_INC) break;
            }
        }
        float inc[NV];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            inc[v] = c[v] * in[v];
            inc[VEC + v] = fmaf(c[v], in[VEC + v], c[VEC + v]);
            inc[2 * VEC + v] = fmaf(c[v], in[2 * VEC + v], c[2 * VEC + v]);
        }
        store_floats<NV>(p.ws.inc + slot * (64 * NV) + lane_off, inc);
        publish_flag(p.ws.flags + slot, FLAG_INC);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            s_cP[lane * VEC + v] = in[v];
            s_cL[lane * VEC + v] = in[VEC + v];
            s_cM[lane * VEC + v] = in[2 * VEC + v];
        }
    }
    __syncthreads();

    // 4. Carry into this wave: chunk carry-in, then waves NW-1 .. wave+1.
    float lam[VEC], mu[VEC];
    {
        float cP[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            cP[v] = s_cP[lane * VEC + v];
            lam[v] = s_cL[lane * VEC + v];
            mu[v] = s_cM[lane * VEC + v];
        }
        for (int w = NW - 1; w > wave; --w) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int i = lane * VEC + v;
                const float xP = s_P[w][i];
                lam[v] = fmaf(xP, lam[v], s_L[w][i]);
                mu[v] = fmaf(xP, mu[v], s_M[w][i]);
                cP[v] = xP * cP[v];
            }
        }
    }

    // 5. Reverse rescan from registers; store da_t, db_t.
    if (!lane_ok) return;
    T *dao = static_cast<T *>(p.da) + base;
    T *dbo = static_cast<T *>(p.db) + base;
#pragma unroll
    for (int r = L - 1; r >= 0; --r) {
        float fc[VEC], fgA[VEC], fgB[VEC];
        PK::unpack(rc[r], fc);
        PK::unpack(rgA[r], fgA);
        PK::unpack(rgB[r], fgB);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            lam[v] = fmaf(fc[v], lam[v], fgB[v]);
            mu[v] = fmaf(fc[v], mu[v], fgA[v]);
        }
        if (t0 + r < p.T) {
            float fAp[VEC], fBp[VEC], da[VEC];
            PK::unpack(rAp[r], fAp);
            PK::unpack(rBp[r], fBp);
#pragma unroll
            for (int v = 0; v < VEC; ++v) da[v] = fmaf(lam[v], fBp[v], mu[v] * fAp[v]);
            store_vec<T, VEC>(dao + r * p.D, PK::pack(da));
            store_vec<T, VEC>(dbo + r * p.D, PK::pack(lam));
        }
    }
}

// ---------------------------------------------------------------------------
// Tile shapes.  VEC elements per lane (16-byte accesses when VEC*sizeof(T) is
// 16), L rows per wave held in registers, NW waves per workgroup.
// ---------------------------------------------------------------------------
template <typename T, int VEC> struct FwdShape { static constexpr int L = 8, NW = 8; };
template <typename T, int VEC> struct BwdShape { static constexpr int L = 4, NW = 8; };

struct Grid {
    int n_dtiles, n_tiles, n_chunks;
    size_t n_slots;
    bool ok;  // the work-item count fits the int32 ticket space
};

inline Grid make_grid(int64_t B, int64_t T, int64_t D, int tile, int chunk) {
    const int64_t nd = (D + tile - 1) / tile, nt = B * nd, nc = (T + chunk - 1) / chunk;
    Grid g;
    g.ok = nt <= INT32_MAX && nc <= INT32_MAX && nt * nc <= (int64_t)INT32_MAX;
    g.n_dtiles = (int)nd;
    g.n_tiles = (int)nt;
    g.n_chunks = (int)nc;
    g.n_slots = g.ok ? (size_t)nt * (size_t)nc : 0;
    return g;
}

template <typename E, int VEC>
size_t fwd_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = FwdShape<E, VEC>::L, NW = FwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW);
    return WsLayout(g.n_slots, 64 * 2 * VEC).total;
}

template <typename E, int VEC>
size_t bwd_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = BwdShape<E, VEC>::L, NW = BwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW);
    return WsLayout(g.n_slots, 64 * 3 * VEC).total;
}

template <typename E, int VEC>
mi_status run_fwd(const void *a, const void *b, void *A, void *Bc, int64_t B, int64_t T,
                  int64_t D, void *ws, size_t ws_bytes, hipStream_t s) {
    constexpr int L = FwdShape<E, VEC>::L, NW = FwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW);
    if (!g.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(g.n_slots, 64 * 2 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    FwdArgs p;
    p.a = a; p.b = b; p.A = A; p.Bc = Bc; p.T = T; p.D = D;
    p.n_dtiles = g.n_dtiles; p.n_tiles = g.n_tiles; p.n_chunks = g.n_chunks;
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, g.n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((linear_fwd_kernel<E, VEC, L, NW>), dim3((unsigned)g.n_slots),
                       dim3(NW * 64), 0, s, p);
    return launch_status();
}

template <typename E, int VEC>
mi_status run_bwd(const void *a, const void *A, const void *Bc, const void *gA,
                  const void *gBc, void *da, void *db, int64_t B, int64_t T, int64_t D,
                  void *ws, size_t ws_bytes, hipStream_t s) {
    constexpr int L = BwdShape<E, VEC>::L, NW = BwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW);
    if (!g.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(g.n_slots, 64 * 3 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    BwdArgs p;
    p.a = a; p.A = A; p.Bc = Bc; p.gA = gA; p.gBc = gBc; p.da = da; p.db = db;
    p.T = T; p.D = D;
    p.n_dtiles = g.n_dtiles; p.n_tiles = g.n_tiles; p.n_chunks = g.n_chunks;
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, g.n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((linear_bwd_kernel<E, VEC, L, NW>), dim3((unsigned)g.n_slots),
                       dim3(NW * 64), 0, s, p);
    return launch_status();
}

}  // namespace

size_t linear_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt) {
    // The vector width is chosen per call from pointer alignment, so size for
    // the largest requirement over every width the dtype may use.
    size_t m = 0;
    auto upd = [&](size_t x) { m = x > m ? x : m; };
    if (dt == MI_F32) {
        upd(fwd_ws<float, 4>(B, T, D)); upd(fwd_ws<float, 2>(B, T, D)); upd(fwd_ws<float, 1>(B, T, D));
        upd(bwd_ws<float, 4>(B, T, D)); upd(bwd_ws<float, 2>(B, T, D)); upd(bwd_ws<float, 1>(B, T, D));
    } else {
        upd(fwd_ws<bf16_t, 8>(B, T, D)); upd(fwd_ws<bf16_t, 4>(B, T, D));
        upd(fwd_ws<bf16_t, 2>(B, T, D)); upd(fwd_ws<bf16_t, 1>(B, T, D));
        upd(bwd_ws<bf16_t, 8>(B, T, D)); upd(bwd_ws<bf16_t, 4>(B, T, D));
        upd(bwd_ws<bf16_t, 2>(B, T, D)); upd(bwd_ws<bf16_t, 1>(B, T, D));
    }
    return m;
}

mi_status launch_linear_fwd(const void *a, const void *b, void *A, void *Bc, int64_t B,
                            int64_t T, int64_t D, mi_dtype dt, int vec, void *ws,
                            size_t ws_bytes, hipStream_t s) {
    if (dt == MI_F32) {
        switch (vec) {
            case 4: return run_fwd<float, 4>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
            case 2: return run_fwd<float, 2>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
            default: return run_fwd<float, 1>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
        }
    }
    switch (vec) {
        case 8: return run_fwd<bf16_t, 8>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
        case 4: return run_fwd<bf16_t, 4>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
        case 2: return run_fwd<bf16_t, 2>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
        default: return run_fwd<bf16_t, 1>(a, b, A, Bc, B, T, D, ws, ws_bytes, s);
    }
}

mi_status launch_linear_bwd(const void *a, const void *A, const void *Bc, const void *gA,
                            const void *gBc, void *da, void *db, int64_t B, int64_t T,
                            int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                            hipStream_t s) {
    if (dt == MI_F32) {
        switch (vec) {
            case 4: return run_bwd<float, 4>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
            case 2: return run_bwd<float, 2>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
            default: return run_bwd<float, 1>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
        }
    }
    switch (vec) {
        case 8: return run_bwd<bf16_t, 8>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
        case 4: return run_bwd<bf16_t, 4>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
        case 2: return run_bwd<bf16_t, 2>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
        default: return run_bwd<bf16_t, 1>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s);
    }
}

}  // namespace miscan
