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
    const void *h0;  // initial state (B, D), used by the H0 kernels; NULL = zero
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

struct BwdArgs {
    const void *a, *A, *Bc, *gA, *gBc;
    void *da, *db;
    const void *h0;  // initial state (B, D) for the H0 kernels; NULL = zero
    void *dh0;       // its gradient (B, D), written by the H0 kernels
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

// Carry algebra of the forward scan per channel: (A, h) maps a state h_in to
// A*h_in + h.  then(x, y) = x followed by y = (y.A*x.A, y.A*x.h + y.h).
struct FwdOp {
    static constexpr int NC = 2;
    static __device__ __forceinline__ void then(float (&r)[2], const float (&x)[2], const float (&y)[2]) {
        r[0] = y[0] * x[0];
        r[1] = fmaf(y[0], x[1], y[1]);
    }
};

// Carry algebra of the reverse scan per channel: (P, l, m) maps the adjoint
// state (lam, mu) entering from later time to (P*lam + l, P*mu + m).
// then(x, y) = x (later in time, applied first) followed by y.
struct BwdOp {
    static constexpr int NC = 3;
    static __device__ __forceinline__ void then(float (&r)[3], const float (&x)[3], const float (&y)[3]) {
        r[0] = y[0] * x[0];
        r[1] = fmaf(y[0], x[1], y[1]);
        r[2] = fmaf(y[0], x[2], y[2]);
    }
};

struct Item {
    int chunk, tile, bidx;
    int64_t row0;  // first row of the workgroup's chunk
    uint32_t wrow; // first row of this wave, relative to row0 (wave-uniform)
    int64_t t0;    // first row of this wave
    int64_t d;     // first channel of this lane
    bool lane_ok;  // this lane's channels exist
};

// Work item of a ticket.  Tickets run chunk-major in scan order: every tile's
// first chunk (in time for the forward, the last one for the reverse scan)
// before any tile's second.
template <int VEC, int L, int NW>
__device__ __forceinline__ Item decode_item(uint32_t ticket, int n_tiles, int n_dtiles, int64_t D, int lane,
                                            int wave, bool reverse, int n_chunks) {
    constexpr int TILE = 64 * VEC;
    Item it;
    const int ord = (int)ticket / n_tiles;
    it.tile = (int)ticket - ord * n_tiles;
    it.chunk = reverse ? n_chunks - 1 - ord : ord;
    it.bidx = it.tile / n_dtiles;
    const int dtile = it.tile - it.bidx * n_dtiles;
    it.d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    it.lane_ok = it.d < D;
    it.row0 = (int64_t)it.chunk * (NW * L);
    it.wrow = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * L;
    it.t0 = it.row0 + it.wrow;
    return it;
}

// ---------------------------------------------------------------------------
// Forward.  One workgroup = one work item (a tile x a time chunk): each wave
// scans its L rows in registers, the wave aggregates meet in LDS, the whole
// workgroup runs the look-back (wg_lookback), and each wave rescans its rows
// from its carry-in and stores A_t, Bc_t.
// ---------------------------------------------------------------------------
// LDS slot of channel ch of a tile whose lanes each hold VEC consecutive
// channels.  With VEC = 8 a lane's two 16-byte halves lie 32 bytes apart, so
// lanes l and l + 4 would hit the same four banks; swapping the halves of
// every other group of four lanes (bit 2 of the slot flips when bit 5 of the
// channel is set) spreads 8 consecutive lanes over all 32 banks and keeps the
// per-channel accesses of consecutive threads conflict-free.
template <int VEC>
__device__ __forceinline__ int lds_ch(int ch) {
    return VEC == 8 ? ch ^ ((ch >> 3) & 4) : ch;
}
// The lane's VEC channels of one LDS row, at their lds_ch slots (16-byte
// accesses: rows are 16-byte aligned).
template <int VEC>
__device__ __forceinline__ void lds_put_lane(float *row, int lane, const float (&x)[VEC]) {
    if constexpr (VEC == 8) {
        const int s = lane & 4;
        const f32x4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
        *reinterpret_cast<f32x4 *>(row + lane * 8 + s) = lo;
        *reinterpret_cast<f32x4 *>(row + lane * 8 + (s ^ 4)) = hi;
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) row[lane * VEC + v] = x[v];
    }
}
template <int VEC>
__device__ __forceinline__ void lds_get_lane(float (&x)[VEC], const float *row, int lane) {
    if constexpr (VEC == 8) {
        const int s = lane & 4;
        const f32x4 lo = *reinterpret_cast<const f32x4 *>(row + lane * 8 + s);
        const f32x4 hi = *reinterpret_cast<const f32x4 *>(row + lane * 8 + (s ^ 4));
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) x[v] = row[lane * VEC + v];
    }
}

// Both k=1 kernels are built for at least 4 waves per SIMD (the second launch
// bound), i.e. at most 128 VGPRs: two 8-wave workgroups then share a CU and
// overlap one's look-back and barriers with the other's streaming.
// H0: the scan starts from the state p.h0 instead of 0 (Bc then holds the
// states from h0): the carry entering chunk 0 is (1, h0).
template <typename T, int VEC, int L, int NW, bool H0 = false>
__global__ __launch_bounds__(NW * 64, 4) void linear_fwd_kernel(FwdArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC, NT = NW * 64, CPT = (TILE + NT - 1) / NT;

    __shared__ __align__(16) float s_A[NW][TILE];  // wave aggregates (lds_ch slots)
    __shared__ __align__(16) float s_H[NW][TILE];
    __shared__ __align__(16) float s_cA[TILE];     // chunk carry-in
    __shared__ __align__(16) float s_cH[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const Item it = decode_item<VEC, L, NW>(__builtin_amdgcn_readfirstlane(s_ticket), p.n_tiles, p.n_dtiles,
                                            p.D, lane, wave, false,
                                            p.n_chunks);
    // Offsets of rows or lanes outside the tensor are replaced by 0 (a valid
    // element) before the access, and the loaded value by the identity after
    // it, so no access leaves the tensor whatever the descriptor's range.
    const uint32_t voff = it.lane_ok ? (uint32_t)(it.d * (int64_t)sizeof(T)) : 0u;
    const uint32_t rowb = (uint32_t)(p.D * (int64_t)sizeof(T));  // bytes per row

    // 1. Load this wave's rows (identity step (1, 0) past T or D).
    raw_t ra[L], rb[L];
    {
        const rsrc_t sa = batch_rows<T>(p.a, it.bidx, it.row0, p.T, p.D);
        const rsrc_t sb = batch_rows<T>(p.b, it.bidx, it.row0, p.T, p.D);
        const raw_t one = splat<T, VEC>(1.f), zero = splat<T, VEC>(0.f);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const bool row_ok = it.t0 + r < p.T;  // wave-uniform
            const bool ok = it.lane_ok && row_ok;
            const uint32_t so = row_ok ? (it.wrow + r) * rowb : 0u;
            const raw_t xa = buf_load<T, VEC>(sa, voff, so);
            const raw_t xb = buf_load<T, VEC>(sb, voff, so);
            ra[r] = ok ? xa : one;
            rb[r] = ok ? xb : zero;
        }
    }

    // 2. Serial scan of the wave's rows from (1, 0): the wave aggregate.  Each
    //    row is widened only when its step runs (opaque): widening rows ahead
    //    of their step kept fp32 copies of several rows live at once and
    //    spilled 9 VGPRs of the bf16 kernel to scratch.
    float gA[VEC], gH[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { gA[v] = 1.f; gH[v] = 0.f; }
#pragma unroll
    for (int r = 0; r < L; ++r) {
        float fa[VEC], fb[VEC];
        opaque(ra[r]); opaque(rb[r]);
        PK::unpack(ra[r], fa);
        PK::unpack(rb[r], fb);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            gH[v] = fmaf(fa[v], gH[v], fb[v]);
            gA[v] = fa[v] * gA[v];
        }
    }
    lds_put_lane<VEC>(s_A[wave], lane, gA);
    lds_put_lane<VEC>(s_H[wave], lane, gH);
    lds_barrier();

    // 3. Chunk aggregate per channel (waves in time order), look-back, carry.
    const int64_t slot = (int64_t)it.tile * p.n_chunks + it.chunk;
    const LbPos lq = lb_pos(it.chunk, p.lb_window);
    {
        float c[CPT][2], in[CPT][2];
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            c[q][0] = 1.f; c[q][1] = 0.f;
            in[q][0] = 1.f; in[q][1] = 0.f;
            if (ch < TILE)
                for (int w = 0; w < NW; ++w) {
                    const float x[2] = {s_A[w][lds_ch<VEC>(ch)], s_H[w][lds_ch<VEC>(ch)]};
                    float r[2];
                    FwdOp::then(r, c[q], x);
                    c[q][0] = r[0]; c[q][1] = r[1];
                }
            if constexpr (H0) {  // the initial state (1, h0) of the first group's fold
                const int64_t dch = (int64_t)(it.tile - it.bidx * p.n_dtiles) * TILE + ch;
                if (!lq.has_inc && ch < TILE && dch < p.D && p.h0 != nullptr) {
                    float f0[1];
                    Pack<T, 1>::unpack(load_vec<T, 1>(static_cast<const T *>(p.h0) + (int64_t)it.bidx * p.D + dch), f0);
                    in[q][1] = f0[0];
                }
            }
        }
        wg_lookback<FwdOp, TILE, NT>(p.ws, slot, -1, lq, c, in);
        wg_store_inclusive<FwdOp, TILE, NT>(p.ws, slot, c, in);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            if (ch < TILE) { s_cA[lds_ch<VEC>(ch)] = in[q][0]; s_cH[lds_ch<VEC>(ch)] = in[q][1]; }
        }
        wg_publish(p.ws, slot);
    }

    // 4. Carry into this wave: chunk carry-in, then waves 0..wave-1.
    float hA[VEC], hH[VEC];
    lds_get_lane<VEC>(hA, s_cA, lane);
    lds_get_lane<VEC>(hH, s_cH, lane);
    for (int w = 0; w < wave; ++w) {
        float xA[VEC], xH[VEC];
        lds_get_lane<VEC>(xA, s_A[w], lane);
        lds_get_lane<VEC>(xH, s_H[w], lane);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            hH[v] = fmaf(xA[v], hH[v], xH[v]);
            hA[v] = xA[v] * hA[v];
        }
    }

    // 5. Rescan the rows from registers and store A_t, Bc_t.
    if (!it.lane_ok) return;
#pragma unroll
    for (int r = 0; r < L; ++r) { opaque(ra[r]); opaque(rb[r]); }
    char *const Ao = row_ptr<T>(p.A, it.bidx, it.row0, p.T, p.D);
    char *const Bo = row_ptr<T>(p.Bc, it.bidx, it.row0, p.T, p.D);
#pragma unroll
    for (int r = 0; r < L; ++r) {
        if (it.t0 + r < p.T) {
            float fa[VEC], fb[VEC];
            PK::unpack(ra[r], fa);
            PK::unpack(rb[r], fb);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                hA[v] = fa[v] * hA[v];
                hH[v] = fmaf(fa[v], hH[v], fb[v]);
            }
            const uint32_t so = (it.wrow + r) * rowb;
            row_store<T, VEC>(PK::pack(hA), Ao + so, voff);
            row_store<T, VEC>(PK::pack(hH), Bo + so, voff);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward.  Reverse time with c_t = a_{t+1} (c_T = 0):
//     lam_t = gBc_t + c_t lam_{t+1},  mu_t = gA_t + c_t mu_{t+1},
//     db_t = lam_t,  da_t = lam_t Bc_{t-1} + mu_t A_{t-1}  (A_0 = 1, Bc_0 = 0).
// Same work-item structure as the forward, with chunks taken from the end of
// time backwards and each wave scanning its rows from the last one.
// ---------------------------------------------------------------------------
// H0: the forward started from p.h0 (Bc holds those states): Bc_{-1} is h0
// in da at the first step, and dh0 = a_1 lam_1 is written as well.
template <typename T, int VEC, int L, int NW, bool H0 = false>
__global__ __launch_bounds__(NW * 64, 4) void linear_bwd_kernel(BwdArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC, NT = NW * 64, CPT = (TILE + NT - 1) / NT;

    __shared__ __align__(16) float s_P[NW][TILE];  // wave aggregates (lds_ch slots)
    __shared__ __align__(16) float s_L[NW][TILE];
    __shared__ __align__(16) float s_M[NW][TILE];
    __shared__ __align__(16) float s_cL[TILE];     // chunk carry-in
    __shared__ __align__(16) float s_cM[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const Item it = decode_item<VEC, L, NW>(__builtin_amdgcn_readfirstlane(s_ticket), p.n_tiles, p.n_dtiles,
                                            p.D, lane, wave, true,
                                            p.n_chunks);
    // Rows or lanes outside the tensor load from offset 0 (a valid element)
    // and are replaced by the identity; see the forward kernel.
    const uint32_t voff = it.lane_ok ? (uint32_t)(it.d * (int64_t)sizeof(T)) : 0u;
    const uint32_t rowb = (uint32_t)(p.D * (int64_t)sizeof(T));
    // Descriptors start one row before the chunk (the A_{t-1}, Bc_{t-1} halo),
    // except for the first chunk, which has no row before it.
    const int64_t first = it.row0 > 0 ? it.row0 - 1 : 0;
    const uint32_t sh = (uint32_t)(it.row0 - first);  // 1, or 0 for the first chunk

    // 1. Loads.  Row r is time t = t0 + r.  c = a_{t+1}; Ap = A_{t-1}; Bp = Bc_{t-1}.
    raw_t rc[L], rgA[L], rgB[L], rAp[L], rBp[L];
    {
        const rsrc_t sa = batch_rows<T>(p.a, it.bidx, first, p.T, p.D);
        const rsrc_t sgA = batch_rows<T>(p.gA, it.bidx, first, p.T, p.D);
        const rsrc_t sgB = batch_rows<T>(p.gBc, it.bidx, first, p.T, p.D);
        const raw_t one = splat<T, VEC>(1.f), zero = splat<T, VEC>(0.f);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const int64_t t = it.t0 + r;
            const bool ok = it.lane_ok && t < p.T;
            const uint32_t so = t < p.T ? (it.wrow + r + sh) * rowb : 0u;
            const uint32_t so_next = t + 1 < p.T ? (it.wrow + r + sh + 1) * rowb : 0u;
            const raw_t xc = buf_load<T, VEC>(sa, voff, so_next);
            const raw_t xgA = buf_load<T, VEC>(sgA, voff, so);
            const raw_t xgB = buf_load<T, VEC>(sgB, voff, so);
            rc[r] = (ok && t + 1 < p.T) ? xc : (ok ? zero : one);
            rgA[r] = ok ? xgA : zero;
            rgB[r] = ok ? xgB : zero;
        }
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
    lds_put_lane<VEC>(s_P[wave], lane, gP);
    lds_put_lane<VEC>(s_L[wave], lane, gL);
    lds_put_lane<VEC>(s_M[wave], lane, gM);
    lds_barrier();
    // A_{t-1}, Bc_{t-1} are needed only by the rescan: loaded after the
    // barrier (which the compiler cannot hoist them over), they overlap the
    // look-back instead of occupying registers during the first scan.
    {
        const rsrc_t sA = batch_rows<T>(p.A, it.bidx, first, p.T, p.D);
        const rsrc_t sB = batch_rows<T>(p.Bc, it.bidx, first, p.T, p.D);
        const raw_t one = splat<T, VEC>(1.f), zero = splat<T, VEC>(0.f);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const int64_t t = it.t0 + r;
            const bool row_ok = t < p.T && t > 0;  // wave-uniform
            const bool ok = it.lane_ok && row_ok;
            const uint32_t so = row_ok ? (it.wrow + r + sh - 1) * rowb : 0u;
            const raw_t xA = buf_load<T, VEC>(sA, voff, so);
            const raw_t xB = buf_load<T, VEC>(sB, voff, so);
            rAp[r] = ok ? xA : one;
            rBp[r] = ok ? xB : zero;
        }
    }
    raw_t ra0 = splat<T, VEC>(0.f);  // a at time row 0 (H0: dh0 = a_1 lam_1)
    if constexpr (H0) {
        if (it.t0 == 0 && it.lane_ok) {  // the wave holding time row 0
            const T *rowa = static_cast<const T *>(p.a) + (int64_t)it.bidx * p.T * p.D + it.d;
            ra0 = load_vec<T, VEC>(rowa);
            if (p.h0 != nullptr) rBp[0] = load_vec<T, VEC>(static_cast<const T *>(p.h0) + (int64_t)it.bidx * p.D + it.d);
        }
    }

    // 3. Chunk aggregate per channel (waves NW-1 .. 0), look-back over later
    //    chunks, carry.
    const int64_t slot = (int64_t)it.tile * p.n_chunks + it.chunk;
    const LbPos lq = lb_pos(p.n_chunks - 1 - it.chunk, p.lb_window);
    {
        float c[CPT][3], in[CPT][3];
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            c[q][0] = 1.f; c[q][1] = 0.f; c[q][2] = 0.f;
            in[q][0] = 1.f; in[q][1] = 0.f; in[q][2] = 0.f;
            if (ch < TILE)
                for (int w = NW - 1; w >= 0; --w) {
                    const int sl = lds_ch<VEC>(ch);
                    const float x[3] = {s_P[w][sl], s_L[w][sl], s_M[w][sl]};
                    float r[3];
                    BwdOp::then(r, c[q], x);
                    c[q][0] = r[0]; c[q][1] = r[1]; c[q][2] = r[2];
                }
        }
        wg_lookback<BwdOp, TILE, NT, 4>(p.ws, slot, +1, lq, c, in);
        wg_store_inclusive<BwdOp, TILE, NT>(p.ws, slot, c, in);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            if (ch < TILE) { s_cL[lds_ch<VEC>(ch)] = in[q][1]; s_cM[lds_ch<VEC>(ch)] = in[q][2]; }
        }
        wg_publish(p.ws, slot);
    }

    // 4. Adjoint state entering this wave: chunk carry-in, then waves NW-1 .. wave+1.
    float lam[VEC], mu[VEC];
    lds_get_lane<VEC>(lam, s_cL, lane);
    lds_get_lane<VEC>(mu, s_cM, lane);
    for (int w = NW - 1; w > wave; --w) {
        float xP[VEC], xL[VEC], xM[VEC];
        lds_get_lane<VEC>(xP, s_P[w], lane);
        lds_get_lane<VEC>(xL, s_L[w], lane);
        lds_get_lane<VEC>(xM, s_M[w], lane);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            lam[v] = fmaf(xP[v], lam[v], xL[v]);
            mu[v] = fmaf(xP[v], mu[v], xM[v]);
        }
    }

    // 5. Reverse rescan from registers; store da_t, db_t.
    if (!it.lane_ok) return;
#pragma unroll
    for (int r = 0; r < L; ++r) { opaque(rc[r]); opaque(rgA[r]); opaque(rgB[r]); }
    char *const dao = row_ptr<T>(p.da, it.bidx, it.row0, p.T, p.D);
    char *const dbo = row_ptr<T>(p.db, it.bidx, it.row0, p.T, p.D);
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
        if (it.t0 + r < p.T) {
            float fAp[VEC], fBp[VEC], da[VEC];
            PK::unpack(rAp[r], fAp);
            PK::unpack(rBp[r], fBp);
#pragma unroll
            for (int v = 0; v < VEC; ++v) da[v] = fmaf(lam[v], fBp[v], mu[v] * fAp[v]);
            const uint32_t so = (it.wrow + r) * rowb;
            row_store<T, VEC>(PK::pack(da), dao + so, voff);
            row_store<T, VEC>(PK::pack(lam), dbo + so, voff);
        }
    }
    if constexpr (H0) {
        if (it.t0 == 0) {  // lam now holds lam_1
            float fa0[VEC], g0[VEC];
            PK::unpack(ra0, fa0);
#pragma unroll
            for (int v = 0; v < VEC; ++v) g0[v] = fa0[v] * lam[v];
            row_store<T, VEC>(PK::pack(g0), row_ptr<T>(p.dh0, it.bidx, 0, 1, p.D), voff);
        }
    }
}

// ---------------------------------------------------------------------------
// Tile shapes.  VEC elements per lane (16-byte accesses when VEC*sizeof(T) is
// 16), L rows per wave held in registers, NW waves per workgroup.
// ---------------------------------------------------------------------------
#ifndef MISCAN_LIN_FWD_L
#define MISCAN_LIN_FWD_L 8
#endif
#ifndef MISCAN_LIN_FWD_NW
#define MISCAN_LIN_FWD_NW 8
#endif
// The backward reads five streams: with 8 rows a wave it needs about 204
// VGPRs and one workgroup fills a CU; with 4 rows (32-row chunks) about 120,
// so two workgroups share a CU and overlap each other's look-back and
// barriers (measured 656 -> 630 us on B=8, T=8192, D=4096, bf16), more than
// paying for the doubled look-back payload.
#ifndef MISCAN_LIN_BWD_L
#define MISCAN_LIN_BWD_L 4
#endif
#ifndef MISCAN_LIN_BWD_NW
#define MISCAN_LIN_BWD_NW 8
#endif
// Widest bf16 vector (elements per lane) each direction uses.
#ifndef MISCAN_LIN_FWD_BF16_VMAX
#define MISCAN_LIN_FWD_BF16_VMAX 8
#endif
#ifndef MISCAN_LIN_BWD_BF16_VMAX
#define MISCAN_LIN_BWD_BF16_VMAX 8
#endif
template <typename T, int VEC> struct FwdShape {
    static constexpr int L = MISCAN_LIN_FWD_L, NW = MISCAN_LIN_FWD_NW;
};
template <typename T, int VEC> struct BwdShape {
    static constexpr int L = MISCAN_LIN_BWD_L, NW = MISCAN_LIN_BWD_NW;
};

struct Grid {
    int n_dtiles, n_tiles, n_chunks;
    size_t n_slots;
    bool ok;  // the work-item count fits the int32 ticket space
};

inline Grid make_grid(int64_t B, int64_t T, int64_t D, int tile, int chunk, int esz) {
    const int64_t nd = (D + tile - 1) / tile, nt = B * nd, nc = (T + chunk - 1) / chunk;
    Grid g;
    // work items fit the int32 ticket space; a chunk's rows (plus the halo)
    // fit the 32-bit byte offsets of the row descriptors
    g.ok = nt <= INT32_MAX && nc <= INT32_MAX && nt * nc <= (int64_t)INT32_MAX &&
           (int64_t)(chunk + 2) * D * esz < ((int64_t)1 << 32);
    g.n_dtiles = (int)nd;
    g.n_tiles = (int)nt;
    g.n_chunks = (int)nc;
    g.n_slots = g.ok ? (size_t)nt * (size_t)nc : 0;
    return g;
}

// Look-back window.  One link of the chain of inclusive states (a flag round
// trip, the fold, the publish: about two microseconds) advances W chunks of a
// tile, while the chip streams one chunk of every tile in
// tiles * item_bytes / bandwidth.  The chain keeps pace when
// W >= link time * bandwidth / (tiles * item_bytes), and a smaller window
// folds fewer payloads per chunk: W = 2 measured 1.7 % faster than W = 4 on
// B=8, T=8192, D=4096 bf16, while thin, long inputs (one tile) still get the
// widest window.  LINK_BYTES is link time * bandwidth.
#ifndef MISCAN_LIN_LINK_BYTES
#define MISCAN_LIN_LINK_BYTES (8 << 20)
#endif
inline int lin_window(const Grid &g, int64_t D, int chunk, int tile, int esz, int streams) {
    const int64_t cols = D < tile ? D : tile;
    const int64_t row_bytes = (int64_t)g.n_tiles * chunk * cols * esz * streams;
    const int64_t want = row_bytes > 0 ? (MISCAN_LIN_LINK_BYTES + row_bytes - 1) / row_bytes : 1;
    return lb_window(1, want);  // the smallest power of two >= want in [2, MISCAN_LB_WMAX]
}

template <typename E, int VEC>
size_t fwd_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = FwdShape<E, VEC>::L, NW = FwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW, (int)sizeof(E));
    return WsLayout(g.n_slots, 64 * 2 * VEC).total;
}

template <typename E, int VEC>
size_t bwd_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = BwdShape<E, VEC>::L, NW = BwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW, (int)sizeof(E));
    return WsLayout(g.n_slots, 64 * 3 * VEC).total;
}

template <typename E, int VEC, bool H0 = false>
mi_status run_fwd(const void *a, const void *b, void *A, void *Bc, int64_t B, int64_t T,
                  int64_t D, void *ws, size_t ws_bytes, hipStream_t s, const void *h0 = nullptr) {
    constexpr int L = FwdShape<E, VEC>::L, NW = FwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW, (int)sizeof(E));
    if (!g.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(g.n_slots, 64 * 2 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    FwdArgs p;
    p.a = a; p.b = b; p.A = A; p.Bc = Bc; p.h0 = h0; p.T = T; p.D = D;
    p.n_dtiles = g.n_dtiles; p.n_tiles = g.n_tiles; p.n_chunks = g.n_chunks;
    p.lb_window = lin_window(g, D, L * NW, 64 * VEC, (int)sizeof(E), 4);  // a, b in; A, Bc out
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, g.n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((linear_fwd_kernel<E, VEC, L, NW, H0>), dim3((unsigned)g.n_slots), dim3(NW * 64), 0, s, p);
    return launch_status();
}

template <typename E, int VEC, bool H0 = false>
mi_status run_bwd(const void *a, const void *A, const void *Bc, const void *gA,
                  const void *gBc, void *da, void *db, int64_t B, int64_t T, int64_t D,
                  void *ws, size_t ws_bytes, hipStream_t s, const void *h0 = nullptr, void *dh0 = nullptr) {
    constexpr int L = BwdShape<E, VEC>::L, NW = BwdShape<E, VEC>::NW;
    Grid g = make_grid(B, T, D, 64 * VEC, L * NW, (int)sizeof(E));
    if (!g.ok) return MI_ERR_UNSUPPORTED;
    WsLayout lay(g.n_slots, 64 * 3 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    BwdArgs p;
    p.a = a; p.A = A; p.Bc = Bc; p.gA = gA; p.gBc = gBc; p.da = da; p.db = db; p.h0 = h0; p.dh0 = dh0;
    p.T = T; p.D = D;
    p.n_dtiles = g.n_dtiles; p.n_tiles = g.n_tiles; p.n_chunks = g.n_chunks;
    p.lb_window = lin_window(g, D, L * NW, 64 * VEC, (int)sizeof(E), 7);  // five streams in, two out
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, g.n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((linear_bwd_kernel<E, VEC, L, NW, H0>), dim3((unsigned)g.n_slots),
                       dim3(NW * 64), 0, s, p);
    return launch_status();
}

}  // namespace

// Workspace of the forward alone at one vector width (the width the call
// picks from D and the pointer alignment).  The 2-byte storage types (bf16,
// fp16) share their tilings.
size_t linear_fwd_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec) {
    if (dt == MI_F32) {
        switch (vec) {
            case 4: return fwd_ws<float, 4>(B, T, D);
            case 2: return fwd_ws<float, 2>(B, T, D);
            default: return fwd_ws<float, 1>(B, T, D);
        }
    }
    if (vec > MISCAN_LIN_FWD_BF16_VMAX) vec = MISCAN_LIN_FWD_BF16_VMAX;
    switch (vec) {
        case 8: return fwd_ws<bf16_t, 8>(B, T, D);
        case 4: return fwd_ws<bf16_t, 4>(B, T, D);
        case 2: return fwd_ws<bf16_t, 2>(B, T, D);
        default: return fwd_ws<bf16_t, 1>(B, T, D);
    }
}

size_t linear_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt) {
    // The vector width is chosen per call from pointer alignment, so size for
    // the largest requirement over every width the dtype may use.
    size_t m = 0;
    auto upd = [&](size_t x) { m = x > m ? x : m; };
    if (dt == MI_F32) {
        upd(fwd_ws<float, 4>(B, T, D)); upd(fwd_ws<float, 2>(B, T, D)); upd(fwd_ws<float, 1>(B, T, D));
        upd(bwd_ws<float, 4>(B, T, D)); upd(bwd_ws<float, 2>(B, T, D)); upd(bwd_ws<float, 1>(B, T, D));
    } else {  // bf16 and fp16
        upd(fwd_ws<bf16_t, 8>(B, T, D)); upd(fwd_ws<bf16_t, 4>(B, T, D));
        upd(fwd_ws<bf16_t, 2>(B, T, D)); upd(fwd_ws<bf16_t, 1>(B, T, D));
        upd(bwd_ws<bf16_t, 8>(B, T, D)); upd(bwd_ws<bf16_t, 4>(B, T, D));
        upd(bwd_ws<bf16_t, 2>(B, T, D)); upd(bwd_ws<bf16_t, 1>(B, T, D));
    }
    return m;
}

namespace {

// 2-byte storage (bf16 or fp16): the widest vector each direction uses.
template <typename E>
mi_status fwd_2byte(const void *a, const void *b, void *A, void *Bc, int64_t B, int64_t T, int64_t D, int vec,
                    void *ws, size_t ws_bytes, hipStream_t s, bool h0_kernels, const void *h0) {
#define MISCAN_LIN_FWD(V)                                                                        \
    (h0_kernels ? run_fwd<E, V, true>(a, b, A, Bc, B, T, D, ws, ws_bytes, s, h0)                 \
                : run_fwd<E, V, false>(a, b, A, Bc, B, T, D, ws, ws_bytes, s))
    if (vec > MISCAN_LIN_FWD_BF16_VMAX) vec = MISCAN_LIN_FWD_BF16_VMAX;
    switch (vec) {
        case 8: return MISCAN_LIN_FWD(8);
        case 4: return MISCAN_LIN_FWD(4);
        case 2: return MISCAN_LIN_FWD(2);
        default: return MISCAN_LIN_FWD(1);
    }
#undef MISCAN_LIN_FWD
}

template <typename E>
mi_status bwd_2byte(const void *a, const void *A, const void *Bc, const void *gA, const void *gBc, void *da,
                    void *db, int64_t B, int64_t T, int64_t D, int vec, void *ws, size_t ws_bytes, hipStream_t s,
                    bool h0_kernels, const void *h0, void *dh0) {
#define MISCAN_LIN_BWD(V)                                                                                  \
    (h0_kernels ? run_bwd<E, V, true>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s, h0, dh0)        \
                : run_bwd<E, V, false>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s))
    if (vec > MISCAN_LIN_BWD_BF16_VMAX) vec = MISCAN_LIN_BWD_BF16_VMAX;
    switch (vec) {
        case 8: return MISCAN_LIN_BWD(8);
        case 4: return MISCAN_LIN_BWD(4);
        case 2: return MISCAN_LIN_BWD(2);
        default: return MISCAN_LIN_BWD(1);
    }
#undef MISCAN_LIN_BWD
}

}  // namespace

// h0_kernels: the H0 instantiations (initial state in, dh0 out); h0 may be
// NULL (zero) there.
mi_status launch_linear_fwd(const void *a, const void *b, void *A, void *Bc, int64_t B,
                            int64_t T, int64_t D, mi_dtype dt, int vec, void *ws,
                            size_t ws_bytes, hipStream_t s, bool h0_kernels, const void *h0) {
    if (dt == MI_BF16) return fwd_2byte<bf16_t>(a, b, A, Bc, B, T, D, vec, ws, ws_bytes, s, h0_kernels, h0);
    if (dt == MI_F16) return fwd_2byte<f16_t>(a, b, A, Bc, B, T, D, vec, ws, ws_bytes, s, h0_kernels, h0);
#define MISCAN_LIN_FWD(V)                                                                        \
    (h0_kernels ? run_fwd<float, V, true>(a, b, A, Bc, B, T, D, ws, ws_bytes, s, h0)             \
                : run_fwd<float, V, false>(a, b, A, Bc, B, T, D, ws, ws_bytes, s))
    switch (vec) {
        case 4: return MISCAN_LIN_FWD(4);
        case 2: return MISCAN_LIN_FWD(2);
        default: return MISCAN_LIN_FWD(1);
    }
#undef MISCAN_LIN_FWD
}

mi_status launch_linear_bwd(const void *a, const void *A, const void *Bc, const void *gA,
                            const void *gBc, void *da, void *db, int64_t B, int64_t T,
                            int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                            hipStream_t s, bool h0_kernels, const void *h0, void *dh0) {
    if (dt == MI_BF16)
        return bwd_2byte<bf16_t>(a, A, Bc, gA, gBc, da, db, B, T, D, vec, ws, ws_bytes, s, h0_kernels, h0, dh0);
    if (dt == MI_F16)
        return bwd_2byte<f16_t>(a, A, Bc, gA, gBc, da, db, B, T, D, vec, ws, ws_bytes, s, h0_kernels, h0, dh0);
#define MISCAN_LIN_BWD(V)                                                                                  \
    (h0_kernels ? run_bwd<float, V, true>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s, h0, dh0)    \
                : run_bwd<float, V, false>(a, A, Bc, gA, gBc, da, db, B, T, D, ws, ws_bytes, s))
    switch (vec) {
        case 4: return MISCAN_LIN_BWD(4);
        case 2: return MISCAN_LIN_BWD(2);
        default: return MISCAN_LIN_BWD(1);
    }
#undef MISCAN_LIN_BWD
}

}  // namespace miscan
