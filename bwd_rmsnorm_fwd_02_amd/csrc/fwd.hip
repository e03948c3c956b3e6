// RMSNorm forward for gfx950: one pass per row.
//
// Computes, per row (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a
// dw-accuracy backward routes", opening description): rstd = 1/sqrt(mean(x^2)
// + eps) and y = BF16(x * rstd * w); in the residual form ("Key" paragraph)
// h = BF16(x + r) is written first and the row statistics are taken on h.
//
// Layout: a row group of `tpr` lanes owns one row; lane l holds the 16-byte
// vectors l, l + tpr, ... (NV of them), so every load and store is a
// coalesced 16-byte access and the row is read from HBM exactly once. A
// block holds `rpb` row groups and walks the rows grid-stride (persistent).
// Sum of squares: exact BF16 squares summed per vector in FP32, vectors
// accumulated in FP64, then a butterfly over the row group (plus an LDS
// exchange when a row spans several waves). rstd is formed in FP64 and
// rounded once to FP32, so it is within about 1e-7 relative of the exact
// value. The weights a lane needs stay in registers for all its rows.
#include "rmsn_device.h"

namespace rmsn {

template <int NV, typename WT, bool RES, bool WIDE>
__global__ void __launch_bounds__(1024) k_fwd(FwdParams p) {
    extern __shared__ double lds_fwd[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    const int wpr = WIDE ? p.tpr / 64 : 1;  // waves per row
    double* red = lds_fwd;                  // [2][rpb][wpr]

    float wv[NV][8];
    bool vok[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int v = lr + k * p.tpr;
        vok[k] = (slot < p.rpb) && (v < p.nvec);
        if (vok[k]) {
            load_w8<WT>(p.w, v, wv[k]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[k][e] = 0.f;
        }
    }

    const int64_t step = (int64_t)gridDim.x * p.rpb;
    int buf = 0;
#pragma unroll 1
    for (int64_t r0 = (int64_t)blockIdx.x * p.rpb; r0 < p.rows; r0 += step) {
        const int64_t r = r0 + slot;
        const bool active = (slot < p.rpb) && (r < p.rows);
        float xf[NV][8];
        double acc = 0.0;
        if (active) {
            const int64_t ox = row_offset(r, p.heads, p.ax);
            uint4 xv[NV];
#pragma unroll
            for (int k = 0; k < NV; ++k)
                if (vok[k]) xv[k] = ld16(p.x + ox + (int64_t)(lr + k * p.tpr) * kVec);
            if constexpr (RES) {
                const int64_t orr = row_offset(r, p.heads, p.ar);
                const int64_t oh = row_offset(r, p.heads, p.ah);
                uint4 rv[NV];
#pragma unroll
                for (int k = 0; k < NV; ++k)
                    if (vok[k]) rv[k] = ld16(p.r + orr + (int64_t)(lr + k * p.tpr) * kVec);
#pragma unroll
                for (int k = 0; k < NV; ++k) {
                    if (!vok[k]) continue;
                    float a[8], b[8];
                    unpack8(xv[k], a);
                    unpack8(rv[k], b);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
                    xv[k] = pack8(a);  // h = BF16(x + r)
                    st16(p.h + oh + (int64_t)(lr + k * p.tpr) * kVec, xv[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                unpack8(xv[k], xf[k]);
                float s = xf[k][0] * xf[k][0];
#pragma unroll
                for (int e = 1; e < 8; ++e) s = __builtin_fmaf(xf[k][e], xf[k][e], s);
                acc += (double)s;
            }
        }
        double tot;
        if constexpr (WIDE) {
            acc = group_sum<64>(acc);
            const int wave = lr >> 6;
            if ((lr & 63) == 0 && slot < p.rpb) red[(buf * p.rpb + slot) * wpr + wave] = acc;
            __syncthreads();
            tot = 0.0;
            if (slot < p.rpb)
                for (int i = 0; i < wpr; ++i) tot += red[(buf * p.rpb + slot) * wpr + i];
            buf ^= 1;
        } else {
            tot = group_sum_rt(acc, p.tpr);
        }
        if (active) {
            const double ms = tot / (double)p.H;
            const float rs = (float)(1.0 / __builtin_sqrt(ms + (double)p.eps));
            if (lr == 0) p.rstd[r] = rs;
            const int64_t oy = row_offset(r, p.heads, p.ay);
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (xf[k][e] * rs) * wv[k][e];
                st16(p.y + oy + (int64_t)(lr + k * p.tpr) * kVec, pack8(o));
            }
        }
    }
}

template <int NV, typename WT, bool RES>
static int launch_fwd_t(const FwdParams& p, const Route& rt, hipStream_t s) {
    const rmsn_route_t& r = rt.r;
    const bool wide = r.lanes_per_row > 64;
    const size_t lds = wide ? sizeof(double) * 2 * r.rows_per_block * (r.lanes_per_row / 64) : 0;
    dim3 grid((unsigned)r.grid), block((unsigned)r.block_threads);
    if (wide)
        hipLaunchKernelGGL((k_fwd<NV, WT, RES, true>), grid, block, lds, s, p);
    else
        hipLaunchKernelGGL((k_fwd<NV, WT, RES, false>), grid, block, lds, s, p);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <typename WT, bool RES>
static int launch_fwd_nv(const FwdParams& p, const Route& rt, hipStream_t s) {
    switch (rt.r.vec_per_lane) {
        case 1: return launch_fwd_t<1, WT, RES>(p, rt, s);
        case 2: return launch_fwd_t<2, WT, RES>(p, rt, s);
        default: return RMSN_ERR_SHAPE;
    }
}

int launch_fwd(const FwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
               hipStream_t s) {
    if (wdt == RMSN_BF16)
        return residual ? launch_fwd_nv<uint16_t, true>(p, rt, s)
                        : launch_fwd_nv<uint16_t, false>(p, rt, s);
    return residual ? launch_fwd_nv<float, true>(p, rt, s) : launch_fwd_nv<float, false>(p, rt, s);
}

}  // namespace rmsn
