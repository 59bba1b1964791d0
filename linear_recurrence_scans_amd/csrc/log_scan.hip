// log_scan.hip -- log-space scan: h_t = a_t h_{t-1} + b_t with the state kept
// as log h.
//
// Operation: minGRU docs, "Triton kernels" page, Kernel entry points,
// parallel_scan_log_fwd.  log_coeffs (B,T,D) holds log a_t; log_values
// (B,T+1,D) holds log h_0 in slot 0 and log b_t in slots 1..T; the result is
// h_1..h_T as one (B,T,D) tensor.
//
// Everything runs in base 2 (x2 = x * log2(e)), so the per-step work is the
// hardware's v_exp_f32 / v_log_f32:
//     lh_t = lae(lc_t + lh_{t-1}, lv_t),  lae(x, y) = log2(2^x + 2^y)
//          = max + log2(1 + 2^(min - max)),
// and only the stored states are exponentiated (h_t = 2^lh_t).  A segment
// transform is (la, lh) with la = sum of lc over the segment and lh the
// segment's state started from log 0 = -inf; composition of an earlier
// segment 1 and a later segment 2 is
//     (la1 + la2, lae(la2 + lh1, lh2)),
// a running max plus log-sum-exp.  Prefix sums of lc over the whole sequence
// are never formed, so no large cancelling sums appear.
//
// The mapping (lanes along D, waves along time, LDS combine, decoupled
// look-back, rescan from registers) is the one of linear_scan.hip.
#include "common.hpp"
#include "internal.hpp"

namespace miscan {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

// log2(2^x + 2^y) with log2(0 + 0) = -inf, +inf absorbing, NaN propagating.
__device__ __forceinline__ float lae2(float x, float y) {
    const float m = fmaxf(x, y);
    const float lo = fminf(x, y);
    float r = m + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(lo - m));
    r = __builtin_isinf(m) ? m : r;
    r = (x != x || y != y) ? (x + y) : r;
    return r;
}

struct LogArgs {
    const void *lc, *lv;
    void *h;
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

// Carry algebra per channel: (la, lh) maps a log-state x to lae(la + x, lh).
// then(x, y) = x followed by y = (x.la + y.la, lae(y.la + x.lh, y.lh)).
struct LogOp {
    static constexpr int NC = 2;
    static __device__ __forceinline__ void then(float (&r)[2], const float (&x)[2], const float (&y)[2]) {
        r[0] = x[0] + y[0];
        r[1] = lae2(y[0] + x[1], y[1]);
    }
};

// Predecessors whose payload loads one look-back round trip issues, and the
// largest look-back window.  The log scans' workloads have few channel tiles
// and few chunks, all running at once: a window that reaches the first chunk
// lets every chunk fold straight from the initial state, with no chain of
// inclusive states to wait for.
#ifndef MISCAN_LOG_BATCH
#define MISCAN_LOG_BATCH 16
#endif
#ifndef MISCAN_LOG_WMAX
#define MISCAN_LOG_WMAX 32
#endif

template <typename T, int VEC, int L, int NW>
__global__ __launch_bounds__(NW * 64) void log_fwd_kernel(LogArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC, NT = NW * 64, CPT = (TILE + NT - 1) / NT;
    constexpr int CHUNK = NW * L;
    const float NEG_INF = -__builtin_inff();

    __shared__ float s_la[NW][TILE];
    __shared__ float s_lh[NW][TILE];
    __shared__ float s_c[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)__builtin_amdgcn_readfirstlane(s_ticket);
    const int chunk = ticket / p.n_tiles;
    const int tile = ticket - chunk * p.n_tiles;
    const int bidx = tile / p.n_dtiles;
    const int dtile = tile - bidx * p.n_dtiles;

    const int64_t d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    const bool lane_ok = d < p.D;
    const int64_t row0 = (int64_t)chunk * CHUNK;
    const uint32_t wrow = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * L;
    const int64_t t0 = row0 + wrow;
    // Rows or lanes outside the tensor load from offset 0 and are replaced.
    const uint32_t voff = lane_ok ? (uint32_t)(d * (int64_t)sizeof(T)) : 0u;
    const uint32_t rowb = (uint32_t)(p.D * (int64_t)sizeof(T));

    // 1. Loads; identity step past T or D is (lc, lv) = (0, -inf).
    //    log_coeffs row t pairs with log_values row t + 1.
    raw_t rlc[L], rlv[L];
    {
        const rsrc_t slc = batch_rows<T>(p.lc, bidx, row0, p.T, p.D);
        const rsrc_t slv = make_rows(static_cast<const T *>(p.lv) + ((int64_t)bidx * (p.T + 1) + row0 + 1) * p.D,
                                     (p.T - row0) * p.D * (int64_t)sizeof(T));
        const raw_t zero = splat<T, VEC>(0.f), ninf = splat<T, VEC>(NEG_INF);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const bool row_ok = t0 + r < p.T;  // wave-uniform
            const bool ok = lane_ok && row_ok;
            const uint32_t so = row_ok ? (wrow + r) * rowb : 0u;
            const raw_t xc = buf_load<T, VEC>(slc, voff, so);
            const raw_t xv = buf_load<T, VEC>(slv, voff, so);
            rlc[r] = ok ? xc : zero;
            rlv[r] = ok ? xv : ninf;
        }
    }

    // 2. Wave aggregate from (0, -inf).
    float ga[VEC], gh[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { ga[v] = 0.f; gh[v] = NEG_INF; }
#pragma unroll
    for (int r = 0; r < L; ++r) {
        float fc[VEC], fv[VEC];
        PK::unpack(rlc[r], fc);
        PK::unpack(rlv[r], fv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const float c2 = fc[v] * LOG2E;
            gh[v] = lae2(c2 + gh[v], fv[v] * LOG2E);
            ga[v] += c2;
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        s_la[wave][lane * VEC + v] = ga[v];
        s_lh[wave][lane * VEC + v] = gh[v];
    }
    lds_barrier();

    // 3. Chunk aggregate per channel, look-back, carry.  The scan's initial
    //    state is log h_0 (log_values slot 0): the first look-back group folds
    //    from it.
    const int64_t slot = (int64_t)tile * p.n_chunks + chunk;
    const LbPos lq = lb_pos(chunk, p.lb_window);
    {
        float c[CPT][2], in[CPT][2];
        const int64_t d_tile = (int64_t)dtile * TILE;
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            c[q][0] = 0.f; c[q][1] = NEG_INF;
            in[q][0] = 0.f; in[q][1] = NEG_INF;
            if (ch < TILE) {
                for (int w = 0; w < NW; ++w) {
                    const float x[2] = {s_la[w][ch], s_lh[w][ch]};
                    float r[2];
                    LogOp::then(r, c[q], x);
                    c[q][0] = r[0]; c[q][1] = r[1];
                }
                if (!lq.has_inc && d_tile + ch < p.D) {
                    const T *lv0 = static_cast<const T *>(p.lv) + (int64_t)bidx * (p.T + 1) * p.D + d_tile + ch;
                    float f0[1];
                    Pack<T, 1>::unpack(load_vec<T, 1>(lv0), f0);
                    in[q][1] = f0[0] * LOG2E;
                }
            }
        }
        wg_lookback<LogOp, TILE, NT, MISCAN_LOG_BATCH>(p.ws, slot, -1, lq, c, in);
        wg_store_inclusive<LogOp, TILE, NT>(p.ws, slot, c, in);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            if (ch < TILE) s_c[ch] = in[q][1];
        }
        wg_publish(p.ws, slot);
    }

    // 4. State entering this wave: chunk carry-in, then waves 0..wave-1.
    float lh[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) lh[v] = s_c[lane * VEC + v];
    for (int w = 0; w < wave; ++w) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            lh[v] = lae2(s_la[w][lane * VEC + v] + lh[v], s_lh[w][lane * VEC + v]);
    }

    // 5. Rescan and store h_t = 2^lh_t.
    if (!lane_ok) return;
#pragma unroll
    for (int r = 0; r < L; ++r) { opaque(rlc[r]); opaque(rlv[r]); }
    char *const ho = row_ptr<T>(p.h, bidx, row0, p.T, p.D);
#pragma unroll
    for (int r = 0; r < L; ++r) {
        if (t0 + r < p.T) {
            float fc[VEC], fv[VEC], out[VEC];
            PK::unpack(rlc[r], fc);
            PK::unpack(rlv[r], fv);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                lh[v] = lae2(fc[v] * LOG2E + lh[v], fv[v] * LOG2E);
                out[v] = exp2f(lh[v]);
            }
            row_store<T, VEC>(PK::pack(out), ho + (wrow + r) * rowb, voff);
        }
    }
}

// ---------------------------------------------------------------------------
// Backward of the log-space scan.  With a_t = e^{lc_t}, b_t = e^{lv_t},
// h_0 = e^{lv_0} and g_t = dL/dh_t, the adjoint of the forward recurrence is
//     lam_t = g_t + a_{t+1} lam_{t+1}   (a_{T+1} = 0),
//     d lc_t = lam_t a_t h_{t-1},  d lv_t = lam_t b_t,  d lv_0 = a_1 lam_1 h_0,
// with h_{t-1} read from the forward output (h_0 from log_values slot 0).
// lam is a plain linear recurrence (g is signed, so it stays in linear
// space); the work-item structure is the channel backward's: chunks from the
// end of time, each wave scanning its rows from the last one.
// In rows (0-based, row r is time r + 1): c_r = e^{lc[r+1]} (0 on the last
// row), lam_r = g[r] + c_r lam_{r+1}; dlc[r] = lam_r e^{lc[r]} h[r-1]
// (h_0 for r = 0); dlv[r+1] = lam_r e^{lv[r+1]}; dlv[0] = lam_0 e^{lc[0]} h_0.
// ---------------------------------------------------------------------------
struct LogBwdArgs {
    const void *lc, *lv, *h, *g;
    void *dlc, *dlv;
    int64_t T, D;
    int n_dtiles, n_tiles, n_chunks;
    int lb_window;  // look-back window W (a power of two)
    WsPtrs ws;
};

// (P, l) maps lam entering from later time to P lam + l; then(x, y) = x
// (later, applied first) followed by y.
struct LogBwdOp {
    static constexpr int NC = 2;
    static __device__ __forceinline__ void then(float (&r)[2], const float (&x)[2], const float (&y)[2]) {
        r[0] = y[0] * x[0];
        r[1] = fmaf(y[0], x[1], y[1]);
    }
};

template <typename T, int VEC, int L, int NW>
__global__ __launch_bounds__(NW * 64) void log_bwd_kernel(LogBwdArgs p) {
    using PK = Pack<T, VEC>;
    using raw_t = typename PK::raw_t;
    constexpr int TILE = 64 * VEC, NT = NW * 64, CPT = (TILE + NT - 1) / NT;
    constexpr int CHUNK = NW * L;

    __shared__ float s_P[NW][TILE];
    __shared__ float s_L[NW][TILE];
    __shared__ float s_cL[TILE];
    __shared__ uint32_t s_ticket;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) s_ticket = take_ticket(p.ws.hdr);
    __syncthreads();
    const int ticket = (int)__builtin_amdgcn_readfirstlane(s_ticket);
    const int ord = ticket / p.n_tiles;
    const int tile = ticket - ord * p.n_tiles;
    const int chunk = p.n_chunks - 1 - ord;
    const int bidx = tile / p.n_dtiles;
    const int dtile = tile - bidx * p.n_dtiles;
    const int64_t d = (int64_t)dtile * TILE + (int64_t)lane * VEC;
    const bool lane_ok = d < p.D;
    const int64_t row0 = (int64_t)chunk * CHUNK;
    const uint32_t wrow = (uint32_t)__builtin_amdgcn_readfirstlane(wave) * L;
    const int64_t t0 = row0 + wrow;
    // Rows or lanes outside a tensor load from offset 0 and are replaced.
    const uint32_t voff = lane_ok ? (uint32_t)(d * (int64_t)sizeof(T)) : 0u;
    const uint32_t rowb = (uint32_t)(p.D * (int64_t)sizeof(T));

    // 1. Scan inputs: lc of the next row (for c) and g.
    raw_t rc[L], rg[L];
    {
        const rsrc_t slc = batch_rows<T>(p.lc, bidx, row0, p.T, p.D);
        const rsrc_t sg = batch_rows<T>(p.g, bidx, row0, p.T, p.D);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const int64_t t = t0 + r;
            const uint32_t so = t < p.T ? (wrow + r) * rowb : 0u;
            const uint32_t so_next = t + 1 < p.T ? (wrow + r + 1) * rowb : 0u;
            rc[r] = buf_load<T, VEC>(slc, voff, so_next);
            rg[r] = buf_load<T, VEC>(sg, voff, so);
        }
    }
    // c_r and g_r as fp32: identity (1, 0) past T or D, c = 0 on the last row.
    auto coef = [&](int r, float (&c)[VEC], float (&gv)[VEC]) {
        const int64_t t = t0 + r;
        PK::unpack(rc[r], c);
        PK::unpack(rg[r], gv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            c[v] = !(lane_ok && t < p.T) ? 1.f : (t + 1 < p.T ? expf(c[v]) : 0.f);
            gv[v] = (lane_ok && t < p.T) ? gv[v] : 0.f;
        }
    };

    // 2. Reverse scan of the wave's rows: the wave aggregate.
    float gP[VEC], gL[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) { gP[v] = 1.f; gL[v] = 0.f; }
#pragma unroll
    for (int r = L - 1; r >= 0; --r) {
        float c[VEC], gv[VEC];
        coef(r, c, gv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            gL[v] = fmaf(c[v], gL[v], gv[v]);
            gP[v] = c[v] * gP[v];
        }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        s_P[wave][lane * VEC + v] = gP[v];
        s_L[wave][lane * VEC + v] = gL[v];
    }
    lds_barrier();

    // Rescan inputs, loaded after the barrier so that they overlap the
    // look-back: lc of the wave's first row, lv of rows + 1, h of rows - 1.
    raw_t rlc0, rlv[L], rh[L];
    {
        const rsrc_t slc = batch_rows<T>(p.lc, bidx, row0, p.T, p.D);
        rlc0 = buf_load<T, VEC>(slc, voff, t0 < p.T ? wrow * rowb : 0u);
        const rsrc_t slv = make_rows(static_cast<const T *>(p.lv) + ((int64_t)bidx * (p.T + 1) + row0 + 1) * p.D,
                                     (p.T - row0) * p.D * (int64_t)sizeof(T));
        const int64_t first = row0 > 0 ? row0 - 1 : 0;  // h halo row
        const uint32_t sh = (uint32_t)(row0 - first);
        const rsrc_t shh = batch_rows<T>(p.h, bidx, first, p.T, p.D);
#pragma unroll
        for (int r = 0; r < L; ++r) {
            const int64_t t = t0 + r;
            rlv[r] = buf_load<T, VEC>(slv, voff, t < p.T ? (wrow + r) * rowb : 0u);
            rh[r] = buf_load<T, VEC>(shh, voff, (t < p.T && t > 0) ? (wrow + r + sh - 1) * rowb : 0u);
        }
    }

    // 3. Chunk aggregate (waves NW-1 .. 0), look-back over later chunks, carry.
    const int64_t slot = (int64_t)tile * p.n_chunks + chunk;
    const LbPos lq = lb_pos(ord, p.lb_window);
    {
        float c[CPT][2], in[CPT][2];
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            c[q][0] = 1.f; c[q][1] = 0.f;
            in[q][0] = 1.f; in[q][1] = 0.f;
            if (ch < TILE)
                for (int w = NW - 1; w >= 0; --w) {
                    const float x[2] = {s_P[w][ch], s_L[w][ch]};
                    float r[2];
                    LogBwdOp::then(r, c[q], x);
                    c[q][0] = r[0]; c[q][1] = r[1];
                }
        }
        wg_lookback<LogBwdOp, TILE, NT, MISCAN_LOG_BATCH>(p.ws, slot, +1, lq, c, in);
        wg_store_inclusive<LogBwdOp, TILE, NT>(p.ws, slot, c, in);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            if (ch < TILE) s_cL[ch] = in[q][1];
        }
        wg_publish(p.ws, slot);
    }

    // 4. lam entering this wave: chunk carry-in, then waves NW-1 .. wave+1.
    float lam[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) lam[v] = s_cL[lane * VEC + v];
    for (int w = NW - 1; w > wave; --w) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) lam[v] = fmaf(s_P[w][lane * VEC + v], lam[v], s_L[w][lane * VEC + v]);
    }

    // 5. Reverse rescan; store dlc[r], dlv[r+1], and dlv[0] on row 0.
    if (!lane_ok) return;
#pragma unroll
    for (int r = 0; r < L; ++r) { opaque(rc[r]); opaque(rg[r]); }
    float h0[VEC];
    if (t0 == 0) {  // wave-uniform: the wave that holds time row 0
        const T *lv0 = static_cast<const T *>(p.lv) + (int64_t)bidx * (p.T + 1) * p.D + d;
        PK::unpack(load_vec<T, VEC>(lv0), h0);
#pragma unroll
        for (int v = 0; v < VEC; ++v) h0[v] = expf(h0[v]);
    }
    char *const dlco = row_ptr<T>(p.dlc, bidx, row0, p.T, p.D);
    char *const dlvo = reinterpret_cast<char *>(static_cast<T *>(p.dlv) + ((int64_t)bidx * (p.T + 1) + row0 + 1) * p.D);
#pragma unroll
    for (int r = L - 1; r >= 0; --r) {
        float c[VEC], gv[VEC];
        coef(r, c, gv);
#pragma unroll
        for (int v = 0; v < VEC; ++v) lam[v] = fmaf(c[v], lam[v], gv[v]);
        const int64_t t = t0 + r;
        if (t < p.T) {
            float e[VEC], hp[VEC], fv[VEC], dc[VEC], dv[VEC];
            // e^{lc[t]}: the next-row coefficient of row r - 1, or the extra row
            PK::unpack(r > 0 ? rc[r - 1] : rlc0, e);
            PK::unpack(rh[r], hp);
            PK::unpack(rlv[r], fv);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                e[v] = expf(e[v]);
                if (t == 0) hp[v] = h0[v];
                dc[v] = lam[v] * e[v] * hp[v];
                dv[v] = lam[v] * expf(fv[v]);
            }
            const uint32_t so = (wrow + r) * rowb;
            row_store<T, VEC>(PK::pack(dc), dlco + so, voff);
            row_store<T, VEC>(PK::pack(dv), dlvo + so, voff);
            if (t == 0) {
                float d0[VEC];
#pragma unroll
                for (int v = 0; v < VEC; ++v) d0[v] = lam[v] * e[v] * h0[v];
                row_store<T, VEC>(PK::pack(d0), dlvo - (int64_t)p.D * (int64_t)sizeof(T), voff);
            }
        }
    }
}

#ifndef MISCAN_LOG_L
#define MISCAN_LOG_L 16
#endif
#ifndef MISCAN_LOG_NW
#define MISCAN_LOG_NW 8
#endif
// Widest fp32 vector (elements per lane); narrower tiles mean more work items.
#ifndef MISCAN_LOG_F32_VMAX
#define MISCAN_LOG_F32_VMAX 4
#endif
template <typename T, int VEC> struct LogShape {
    static constexpr int L = MISCAN_LOG_L, NW = MISCAN_LOG_NW;
};

#ifndef MISCAN_LOGB_L
#define MISCAN_LOGB_L 8
#endif
#ifndef MISCAN_LOGB_NW
#define MISCAN_LOGB_NW 8
#endif
template <typename T, int VEC> struct LogBwdShape {
    static constexpr int L = MISCAN_LOGB_L, NW = MISCAN_LOGB_NW;
};

template <typename E, int VEC>
size_t log_bwd_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = LogBwdShape<E, VEC>::L, NW = LogBwdShape<E, VEC>::NW;
    const int64_t tile = 64 * VEC, chunk = L * NW;
    const size_t n_slots = (size_t)(B * ((D + tile - 1) / tile)) * (size_t)((T + chunk - 1) / chunk);
    return WsLayout(n_slots, 64 * 2 * VEC).total;
}

template <typename E, int VEC>
mi_status run_log_bwd(const void *lc, const void *lv, const void *h, const void *g, void *dlc, void *dlv,
                      int64_t B, int64_t T, int64_t D, void *ws, size_t ws_bytes, hipStream_t s) {
    constexpr int L = LogBwdShape<E, VEC>::L, NW = LogBwdShape<E, VEC>::NW;
    const int64_t tile = 64 * VEC, chunk = L * NW;
    const int64_t nd = (D + tile - 1) / tile, nc = (T + chunk - 1) / chunk;
    if (B * nd > INT32_MAX || nc > INT32_MAX || B * nd * nc > (int64_t)INT32_MAX) return MI_ERR_UNSUPPORTED;
    if ((chunk + 2) * D * (int64_t)sizeof(E) >= ((int64_t)1 << 32)) return MI_ERR_UNSUPPORTED;
    LogBwdArgs p;
    p.n_dtiles = (int)nd;
    p.n_tiles = (int)(B * nd);
    p.n_chunks = (int)nc;
    const size_t n_slots = (size_t)p.n_tiles * (size_t)p.n_chunks;
    WsLayout lay(n_slots, 64 * 2 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    p.lc = lc; p.lv = lv; p.h = h; p.g = g; p.dlc = dlc; p.dlv = dlv; p.T = T; p.D = D;
    p.lb_window = lb_window(p.n_tiles, MISCAN_LB_RESIDENT, MISCAN_LOG_WMAX);
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((log_bwd_kernel<E, VEC, L, NW>), dim3((unsigned)n_slots), dim3(NW * 64), 0, s, p);
    return launch_status();
}

template <typename E, int VEC>
size_t log_ws(int64_t B, int64_t T, int64_t D) {
    constexpr int L = LogShape<E, VEC>::L, NW = LogShape<E, VEC>::NW;
    const int64_t tile = 64 * VEC, chunk = L * NW;
    const size_t n_slots = (size_t)(B * ((D + tile - 1) / tile)) * (size_t)((T + chunk - 1) / chunk);
    return WsLayout(n_slots, 64 * 2 * VEC).total;
}

template <typename E, int VEC>
mi_status run_log(const void *lc, const void *lv, void *h, int64_t B, int64_t T, int64_t D,
                  void *ws, size_t ws_bytes, hipStream_t s) {
    constexpr int L = LogShape<E, VEC>::L, NW = LogShape<E, VEC>::NW;
    const int64_t tile = 64 * VEC, chunk = L * NW;
    const int64_t nd = (D + tile - 1) / tile, nc = (T + chunk - 1) / chunk;
    if (B * nd > INT32_MAX || nc > INT32_MAX || B * nd * nc > (int64_t)INT32_MAX) return MI_ERR_UNSUPPORTED;
    if ((chunk + 2) * D * (int64_t)sizeof(E) >= ((int64_t)1 << 32)) return MI_ERR_UNSUPPORTED;
    LogArgs p;
    p.n_dtiles = (int)((D + tile - 1) / tile);
    p.n_tiles = (int)(B * p.n_dtiles);
    p.n_chunks = (int)((T + chunk - 1) / chunk);
    const size_t n_slots = (size_t)p.n_tiles * (size_t)p.n_chunks;
    WsLayout lay(n_slots, 64 * 2 * VEC);
    if (ws == nullptr || ws_bytes < lay.total) return MI_ERR_WORKSPACE;
    p.lc = lc; p.lv = lv; p.h = h; p.T = T; p.D = D;
    p.lb_window = lb_window(p.n_tiles, MISCAN_LB_RESIDENT, MISCAN_LOG_WMAX);
    p.ws = ws_ptrs(ws, lay);
    mi_status st = clear_workspace(p.ws, n_slots, s);
    if (st != MI_OK) return st;
    hipLaunchKernelGGL((log_fwd_kernel<E, VEC, L, NW>), dim3((unsigned)n_slots), dim3(NW * 64),
                       0, s, p);
    return launch_status();
}

}  // namespace

size_t log_workspace_bytes(int64_t B, int64_t T, int64_t D, mi_dtype dt) {
    size_t m = 0;
    auto upd = [&](size_t x) { m = x > m ? x : m; };
    // one workspace serves the forward and the backward
    if (dt == MI_F32) {
        upd(log_ws<float, 4>(B, T, D)); upd(log_ws<float, 2>(B, T, D)); upd(log_ws<float, 1>(B, T, D));
        upd(log_bwd_ws<float, 4>(B, T, D)); upd(log_bwd_ws<float, 2>(B, T, D)); upd(log_bwd_ws<float, 1>(B, T, D));
    } else {  // bf16 and fp16 share their tilings
        upd(log_ws<bf16_t, 8>(B, T, D)); upd(log_ws<bf16_t, 4>(B, T, D));
        upd(log_ws<bf16_t, 2>(B, T, D)); upd(log_ws<bf16_t, 1>(B, T, D));
        upd(log_bwd_ws<bf16_t, 8>(B, T, D)); upd(log_bwd_ws<bf16_t, 4>(B, T, D));
        upd(log_bwd_ws<bf16_t, 2>(B, T, D)); upd(log_bwd_ws<bf16_t, 1>(B, T, D));
    }
    return m;
}

namespace {

template <typename E>
mi_status log_fwd_2byte(const void *lc, const void *lv, void *h, int64_t B, int64_t T, int64_t D, int vec,
                        void *ws, size_t ws_bytes, hipStream_t s) {
    switch (vec) {
        case 8: return run_log<E, 8>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        case 4: return run_log<E, 4>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        case 2: return run_log<E, 2>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        default: return run_log<E, 1>(lc, lv, h, B, T, D, ws, ws_bytes, s);
    }
}

template <typename E>
mi_status log_bwd_2byte(const void *lc, const void *lv, const void *h, const void *g, void *dlc, void *dlv,
                        int64_t B, int64_t T, int64_t D, int vec, void *ws, size_t ws_bytes, hipStream_t s) {
    switch (vec) {
        case 8: return run_log_bwd<E, 8>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
        case 4: return run_log_bwd<E, 4>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
        case 2: return run_log_bwd<E, 2>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
        default: return run_log_bwd<E, 1>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
    }
}

}  // namespace

mi_status launch_log_fwd(const void *lc, const void *lv, void *h, int64_t B, int64_t T,
                         int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                         hipStream_t s) {
    if (dt == MI_BF16) return log_fwd_2byte<bf16_t>(lc, lv, h, B, T, D, vec, ws, ws_bytes, s);
    if (dt == MI_F16) return log_fwd_2byte<f16_t>(lc, lv, h, B, T, D, vec, ws, ws_bytes, s);
    if (vec > MISCAN_LOG_F32_VMAX) vec = MISCAN_LOG_F32_VMAX;
    switch (vec) {
        case 4: return run_log<float, 4>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        case 2: return run_log<float, 2>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        default: return run_log<float, 1>(lc, lv, h, B, T, D, ws, ws_bytes, s);
    }
}

mi_status launch_log_bwd(const void *lc, const void *lv, const void *h, const void *g, void *dlc, void *dlv,
                         int64_t B, int64_t T, int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                         hipStream_t s) {
    if (dt == MI_BF16) return log_bwd_2byte<bf16_t>(lc, lv, h, g, dlc, dlv, B, T, D, vec, ws, ws_bytes, s);
    if (dt == MI_F16) return log_bwd_2byte<f16_t>(lc, lv, h, g, dlc, dlv, B, T, D, vec, ws, ws_bytes, s);
    if (vec > MISCAN_LOG_F32_VMAX) vec = MISCAN_LOG_F32_VMAX;
    switch (vec) {
        case 4: return run_log_bwd<float, 4>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
        case 2: return run_log_bwd<float, 2>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
        default: return run_log_bwd<float, 1>(lc, lv, h, g, dlc, dlv, B, T, D, ws, ws_bytes, s);
    }
}

}  // namespace miscan
