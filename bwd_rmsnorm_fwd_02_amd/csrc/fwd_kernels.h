// RMSNorm forward for gfx950: one pass per row (kernel templates).
//
// Computes, per row (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a
// dw-accuracy backward routes", opening description): rstd = 1/sqrt(mean(x^2)
// + eps) and y = BF16(x * rstd * w); in the residual form ("Key" paragraph)
// h = BF16(x + r) is written first and the row statistics are taken on h.
//
// Layout: a row group of `tpr` lanes owns a row; lane l holds the 16-byte
// vectors l, l + tpr, ... (NV of them), so every access is a coalesced
// 16-byte load or store and each row is read from HBM exactly once. A block
// holds `rpb` row groups; each iteration a row group holds U rows at once,
// and the block walks the rows grid-stride (persistent). With U <= 2 the
// next iteration's rows are loaded before the current ones are reduced and
// written (software pipelining); with larger U the block already holds
// enough rows at once, and other blocks on the CU cover its compute phase.
//
// Sum of squares: exact BF16 squares summed per vector in FP32, vectors
// accumulated in FP64, then a butterfly over the row group (plus an LDS
// exchange, behind an LDS-only barrier, when a row spans several waves).
// rstd is formed in FP64 and rounded once to FP32, within ~1e-7 relative of
// the exact value. The weights a lane needs stay in registers.
#pragma once

#include "rmsn_device.h"

namespace rmsn {

template <int NV, int U, bool RES>
struct FwdTile {
    uint4 x[U][NV];
    uint4 r[U][NV];  // residual input (RES only)
};

// Every lane issues the same loads: rows past the end and vectors past the
// row end are clamped to the last valid ones and their values ignored, so
// there are no branches around memory operations (branches there make the
// compiler's wait counting fall back to waiting for everything).
template <int NV, int U, bool RES, bool NTX>
__device__ __forceinline__ void fwd_load(const FwdParams& p, int64_t r0, int slot, int lr,
                                         FwdTile<NV, U, RES>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
        int64_t r = r0 + slot + (int64_t)k * p.rpb;
        if (r > p.rows - 1) r = p.rows - 1;
        const int64_t ox = row_offset(r, p.heads, p.ax);
        int64_t orr = 0;
        if constexpr (RES) orr = row_offset(r, p.heads, p.ar);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            int vi = lr + v * p.tpr;
            if (vi > p.nvec - 1) vi = p.nvec - 1;
            const int64_t c = (int64_t)vi * kVec;
            t.x[k][v] = ld16p<NTX>(p.x + ox + c);
            if constexpr (RES) t.r[k][v] = ld16p<NTX>(p.r + orr + c);
        }
    }
}

template <int NV, int U, bool RES>
__device__ __forceinline__ void fwd_ready(const FwdTile<NV, U, RES>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            use_now(t.x[k][v]);
            if constexpr (RES) use_now(t.r[k][v]);
        }
}

// NTX: stream (non-temporal) the loads of x and r.
template <int NV, int U, typename WT, bool RES, bool WIDE, bool NTX>
__global__ void __launch_bounds__(WIDE ? (NV * U >= 4 ? 512 : 1024) : 256) k_fwd(FwdParams p) {
    constexpr bool PF = U <= 2;  // software-pipeline the next iteration's rows
    extern __shared__ double lds_fwd[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    const int wpr = WIDE ? p.tpr / 64 : 1;  // waves per row
    double* red = lds_fwd;                  // [2][rpb][U][wpr]

    float wv[NV][8];
    bool vok[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int vi = lr + v * p.tpr;
        vok[v] = (slot < p.rpb) && (vi < p.nvec);
        if (vok[v]) {
            load_w8<WT>(p.w, vi, wv[v]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[v][e] = 0.f;
        }
    }

    const int64_t per_iter = (int64_t)p.rpb * U;
    const int64_t stride = (int64_t)gridDim.x * per_iter;
    int64_t r0 = (int64_t)blockIdx.x * per_iter;
    if (r0 >= p.rows) return;  // whole block idle (uniform)
    FwdTile<NV, U, RES> cur;
    FwdTile<NV, PF ? U : 1, RES> nxt;
    fwd_load<NV, U, RES, NTX>(p, r0, slot, lr, cur);
    fwd_ready<NV, U, RES>(cur);
    int buf = 0;
#pragma unroll 1
    for (; r0 < p.rows; r0 += stride) {
        if constexpr (PF) fwd_load<NV, U, RES, NTX>(p, r0 + stride, slot, lr, nxt);

        // compute: h (residual), sum of squares, row sums, outputs in registers
        double acc[U];
        float xf[U][NV][8];
        uint4 hout[U][NV];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            acc[k] = 0.0;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                uint4 xv = cur.x[k][v];
                if constexpr (RES) {
                    float a[8], b[8];
                    unpack8(xv, a);
                    unpack8(cur.r[k][v], b);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
                    xv = pack8(a);  // h = BF16(x + r)
                    hout[k][v] = xv;
                }
                unpack8(xv, xf[k][v]);
                float s = xf[k][v][0] * xf[k][v][0];
#pragma unroll
                for (int e = 1; e < 8; ++e) s = __builtin_fmaf(xf[k][v][e], xf[k][v][e], s);
                if (vok[v]) acc[k] += (double)s;
            }
        }
        double tot[U];
        if constexpr (WIDE) {
            const int wave = lr >> 6;
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const double a = group_sum<64>(acc[k]);
                if ((lr & 63) == 0 && slot < p.rpb) red[((buf * p.rpb + slot) * U + k) * wpr + wave] = a;
            }
            lds_barrier();
#pragma unroll
            for (int k = 0; k < U; ++k) {
                double t = 0.0;
                if (slot < p.rpb)
                    for (int i = 0; i < wpr; ++i) t += red[((buf * p.rpb + slot) * U + k) * wpr + i];
                tot[k] = t;
            }
            buf ^= 1;
        } else {
#pragma unroll
            for (int k = 0; k < U; ++k) tot[k] = group_sum_rt(acc[k], p.tpr);
        }
        float rs[U];
        uint4 yout[U][NV];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const double ms = tot[k] / (double)p.H;
            rs[k] = (float)(1.0 / __builtin_sqrt(ms + (double)p.eps));
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (xf[k][v][e] * rs[k]) * wv[v][e];
                yout[k][v] = pack8(o);
            }
        }
        // The next tile must be complete before its registers take over. The
        // wait lands here, before this iteration's stores are issued, so it
        // covers only that tile and the previous iteration's stores.
        if constexpr (PF) {
            fwd_ready<NV, U, RES>(nxt);
            cur = nxt;
        }
        // stores
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = r0 + slot + (int64_t)k * p.rpb;
            if (slot >= p.rpb || r >= p.rows) continue;
            if (lr == 0) p.rstd[r] = rs[k];
            const int64_t oy = row_offset(r, p.heads, p.ay);
            int64_t oh = 0;
            if constexpr (RES) oh = row_offset(r, p.heads, p.ah);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (!vok[v]) continue;
                const int64_t c = (int64_t)(lr + v * p.tpr) * kVec;
                if constexpr (RES) st16_stream(p.h + oh + c, hout[k][v]);
                st16_stream(p.y + oy + c, yout[k][v]);
            }
        }
        if constexpr (!PF) {
            if (r0 + stride < p.rows) fwd_load<NV, U, RES, NTX>(p, r0 + stride, slot, lr, cur);
        }
    }
}

// LDS bytes the forward kernel needs for a route.
inline size_t fwd_lds_bytes(const rmsn_route_t& r) {
    if (r.lanes_per_row <= 64) return 0;
    return sizeof(double) * 2 * (size_t)r.rows_per_block * r.unroll * (r.lanes_per_row / 64);
}

template <int NV, int U, typename WT, bool RES>
static int launch_fwd_t(const FwdParams& p, const Route& rt, hipStream_t s) {
    const rmsn_route_t& r = rt.r;
    const size_t lds = fwd_lds_bytes(r);
    dim3 grid((unsigned)r.grid), block((unsigned)r.block_threads);
    const bool ntx = r.stream_loads >= 2;
    if (r.lanes_per_row > 64) {
        if (ntx) launch_kernel((k_fwd<NV, U, WT, RES, true, true>), grid, block, lds, s, p);
        else launch_kernel((k_fwd<NV, U, WT, RES, true, false>), grid, block, lds, s, p);
    } else {
        if (ntx) launch_kernel((k_fwd<NV, U, WT, RES, false, true>), grid, block, lds, s, p);
        else launch_kernel((k_fwd<NV, U, WT, RES, false, false>), grid, block, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

// (NV, U) pairs compiled: NV * U <= 8.
template <typename WT, bool RES>
static int launch_fwd_shape(const FwdParams& p, const Route& rt, hipStream_t s) {
    const int nv = rt.r.vec_per_lane, u = rt.r.unroll;
    if (nv == 1) {
        switch (u) {
            case 1: return launch_fwd_t<1, 1, WT, RES>(p, rt, s);
            case 2: return launch_fwd_t<1, 2, WT, RES>(p, rt, s);
            case 4: return launch_fwd_t<1, 4, WT, RES>(p, rt, s);
            case 8: return launch_fwd_t<1, 8, WT, RES>(p, rt, s);
        }
    } else if (nv == 2) {
        switch (u) {
            case 1: return launch_fwd_t<2, 1, WT, RES>(p, rt, s);
            case 2: return launch_fwd_t<2, 2, WT, RES>(p, rt, s);
            case 4: return launch_fwd_t<2, 4, WT, RES>(p, rt, s);
        }
    } else if (nv == 4) {
        switch (u) {
            case 1: return launch_fwd_t<4, 1, WT, RES>(p, rt, s);
            case 2: return launch_fwd_t<4, 2, WT, RES>(p, rt, s);
        }
    }
    return RMSN_ERR_SHAPE;
}

template <typename WT>
static int launch_fwd_wt(const FwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return residual ? launch_fwd_shape<WT, true>(p, rt, s) : launch_fwd_shape<WT, false>(p, rt, s);
}

}  // namespace rmsn
