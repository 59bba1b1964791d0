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

// Predecessors whose payload loads one look-back round trip issues.
#ifndef MISCAN_LOG_BATCH
#define MISCAN_LOG_BATCH 8
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
    __shared__ int s_k;

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

    // 3. Chunk aggregate per channel, look-back, carry.  Before the first
    //    chunk the state is log h_0 (log_values slot 0).
    const int64_t slot = (int64_t)tile * p.n_chunks + chunk;
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
                if (chunk == 0 && d_tile + ch < p.D) {
                    const T *lv0 = static_cast<const T *>(p.lv) + (int64_t)bidx * (p.T + 1) * p.D + d_tile + ch;
                    float f0[1];
                    Pack<T, 1>::unpack(load_vec<T, 1>(lv0), f0);
                    in[q][1] = f0[0] * LOG2E;
                }
            }
        }
        wg_lookback<LogOp, TILE, NT, MISCAN_LOG_BATCH>(p.ws, slot, -1, chunk, c, in, &s_k);
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int ch = threadIdx.x + q * NT;
            if (ch < TILE) s_c[ch] = in[q][1];
        }
        wg_publish_inc(p.ws, slot);
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
    if (dt == MI_F32) {
        upd(log_ws<float, 4>(B, T, D)); upd(log_ws<float, 2>(B, T, D)); upd(log_ws<float, 1>(B, T, D));
    } else {
        upd(log_ws<bf16_t, 8>(B, T, D)); upd(log_ws<bf16_t, 4>(B, T, D));
        upd(log_ws<bf16_t, 2>(B, T, D)); upd(log_ws<bf16_t, 1>(B, T, D));
    }
    return m;
}

mi_status launch_log_fwd(const void *lc, const void *lv, void *h, int64_t B, int64_t T,
                         int64_t D, mi_dtype dt, int vec, void *ws, size_t ws_bytes,
                         hipStream_t s) {
    if (dt == MI_F32) {
        if (vec > MISCAN_LOG_F32_VMAX) vec = MISCAN_LOG_F32_VMAX;
        switch (vec) {
            case 4: return run_log<float, 4>(lc, lv, h, B, T, D, ws, ws_bytes, s);
            case 2: return run_log<float, 2>(lc, lv, h, B, T, D, ws, ws_bytes, s);
            default: return run_log<float, 1>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        }
    }
    switch (vec) {
        case 8: return run_log<bf16_t, 8>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        case 4: return run_log<bf16_t, 4>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        case 2: return run_log<bf16_t, 2>(lc, lv, h, B, T, D, ws, ws_bytes, s);
        default: return run_log<bf16_t, 1>(lc, lv, h, B, T, D, ws, ws_bytes, s);
    }
}

}  // namespace miscan
