// LayerNorm for gfx950 (kernel templates): the adjacent normalisation of
// the same training stacks (ROCm TransformerEngine PR "Microbenchmarking
// and CI performance regression test", benchmark_normalization table:
// RMSNorm and LayerNorm forward and backward on MI355).
//
// Per row, with the usual definition:
//   forward   mu = mean(x), var = mean((x - mu)^2), rstd = 1/sqrt(var + eps),
//             y = BF16((x - mu) * rstd * gamma + beta)
//   backward  xhat = (x - mu) * rstd, g = dy * gamma,
//             dx = BF16(rstd * (g - mean(g) - xhat * mean(g * xhat))),
//             dgamma_j = sum_t dy * xhat, dbeta_j = sum_t dy
//
// The row layout, pipelining and partition are those of the RMSNorm
// kernels: a row group of `tpr` lanes owns a row, each lane NV 16-byte
// vectors of it; U rows per iteration, the next iteration's rows loaded
// before the current ones are reduced (U <= 2); blocks take the row tiles
// b, b + P, b + 2P, ... with P fixed by the shape.
//
// Forward statistics are two passes over the row held in registers: the
// mean (FP32 sums per 16-byte vector, added in FP64), then the sum of
// squared deviations from the FP32-rounded mean (same scheme), so rows with
// a large offset keep their variance. rstd is formed in FP64 and rounded
// once. The backward's two row sums, sum(g) and sum(g * xhat), travel in one
// exchange. dgamma is accumulated per lane in FP64 (dy * (x - mu) is formed
// in FP32 and scaled by rstd in the FP64 fused multiply-add), dbeta in FP32
// (a lane adds at most rows/P BF16 values: even a million same-sign rows
// over 512 blocks stay within ~1e-6 relative of the exact partial, four
// orders below the budget, and it leaves the wide-row shapes registers to
// spare); both are combined per block in slot order and written as one
// partial row of 2H values; the column reduce then sums the P partials in
// FP64 in a fixed order. Both modes run this path, so dx and, in the
// deterministic mode, dgamma and dbeta are bit-reproducible.
#pragma once

#include "rmsn_device.h"

namespace rmsn {

template <int NV, int U>
struct LnFwdTile {
    uint4 x[U][NV];
};

template <int NV, int U, bool NTX>
__device__ __forceinline__ void ln_fwd_load(const LnFwdParams& p, int64_t r0, int slot, int lr,
                                            LnFwdTile<NV, U>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
        int64_t r = r0 + slot + (int64_t)k * p.rpb;
        if (r > p.rows - 1) r = p.rows - 1;  // clamped: no branch around the loads
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            int vi = lr + v * p.tpr;
            if (vi > p.nvec - 1) vi = p.nvec - 1;
            t.x[k][v] = ld16p<NTX>(p.x + r * p.H + (int64_t)vi * kVec);
        }
    }
}

template <int NV, int U>
__device__ __forceinline__ void ln_fwd_ready(const LnFwdTile<NV, U>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
        for (int v = 0; v < NV; ++v) use_now(t.x[k][v]);
}

// Row-group sums of U FP64 per-lane values; WIDE rows exchange wave sums
// through LDS (double-buffered by `buf`, one LDS-only barrier per call).
template <int U, bool WIDE>
__device__ __forceinline__ void ln_row_sums_d(double (&v)[U], int tpr, int rpb, int slot, int lr,
                                              double* red, int& buf) {
    if constexpr (WIDE) {
        const int wpr = tpr >> 6;
        const int wave = lr >> 6;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const double a = group_sum<64>(v[k]);
            if ((lr & 63) == 0 && slot < rpb) red[((buf * rpb + slot) * U + k) * wpr + wave] = a;
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < U; ++k) {
            double t = 0.0;
            if (slot < rpb)
                for (int i = 0; i < wpr; ++i) t += red[((buf * rpb + slot) * U + k) * wpr + i];
            v[k] = t;
        }
        buf ^= 1;
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) v[k] = group_sum_rt(v[k], tpr);
    }
}

// NTX: stream (non-temporal) the loads of x.
template <int NV, int U, typename WT, bool WIDE, bool NTX>
__global__ void __launch_bounds__(WIDE ? (NV * U >= 4 ? 512 : 1024) : 256) k_ln_fwd(LnFwdParams p) {
    constexpr bool PF = U <= 2;
    extern __shared__ double lds_lnf[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    double* red = lds_lnf;  // [2][rpb][U][wpr]

    float gv[NV][8], bv[NV][8];
    bool vok[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int vi = lr + v * p.tpr;
        vok[v] = (slot < p.rpb) && (vi < p.nvec);
        if (vok[v]) {
            load_w8<WT>(p.gamma, vi, gv[v]);
            if (p.beta) {
                load_w8<WT>(p.beta, vi, bv[v]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) bv[v][e] = 0.f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[v][e] = bv[v][e] = 0.f;
        }
    }

    const int64_t per_iter = (int64_t)p.rpb * U;
    const int64_t stride = (int64_t)gridDim.x * per_iter;
    int64_t r0 = (int64_t)blockIdx.x * per_iter;
    if (r0 >= p.rows) return;  // whole block idle (uniform)
    LnFwdTile<NV, U> cur;
    LnFwdTile<NV, PF ? U : 1> nxt;
    ln_fwd_load<NV, U, NTX>(p, r0, slot, lr, cur);
    ln_fwd_ready<NV, U>(cur);
    int buf = 0;
#pragma unroll 1
    for (; r0 < p.rows; r0 += stride) {
        if constexpr (PF) ln_fwd_load<NV, U, NTX>(p, r0 + stride, slot, lr, nxt);

        // pass 1: mean
        double s1[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            s1[k] = 0.0;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float xf[8];
                unpack8(cur.x[k][v], xf);
                float s = xf[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) s += xf[e];
                if (vok[v]) s1[k] += (double)s;
            }
        }
        ln_row_sums_d<U, WIDE>(s1, p.tpr, p.rpb, slot, lr, red, buf);
        float muf[U];
#pragma unroll
        for (int k = 0; k < U; ++k) muf[k] = (float)(s1[k] / (double)p.H);

        // pass 2: squared deviations from the (FP32) mean
        double s2[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            s2[k] = 0.0;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float xf[8];
                unpack8(cur.x[k][v], xf);
                float d = xf[0] - muf[k];
                float q = d * d;
#pragma unroll
                for (int e = 1; e < 8; ++e) {
                    d = xf[e] - muf[k];
                    q = __builtin_fmaf(d, d, q);
                }
                if (vok[v]) s2[k] += (double)q;
            }
        }
        ln_row_sums_d<U, WIDE>(s2, p.tpr, p.rpb, slot, lr, red, buf);
        float rs[U];
        uint4 yout[U][NV];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const double var = s2[k] / (double)p.H;
            rs[k] = (float)(1.0 / __builtin_sqrt(var + (double)p.eps));
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float xf[8], o[8];
                unpack8(cur.x[k][v], xf);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = __builtin_fmaf((xf[e] - muf[k]) * rs[k], gv[v][e], bv[v][e]);
                yout[k][v] = pack8(o);
            }
        }
        if constexpr (PF) {
            ln_fwd_ready<NV, U>(nxt);
            cur = nxt;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = r0 + slot + (int64_t)k * p.rpb;
            if (slot >= p.rpb || r >= p.rows) continue;
            if (lr == 0) {
                p.mean[r] = muf[k];
                p.rstd[r] = rs[k];
            }
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (!vok[v]) continue;
                st16_stream(p.y + r * p.H + (int64_t)(lr + v * p.tpr) * kVec, yout[k][v]);
            }
        }
        if constexpr (!PF) {
            if (r0 + stride < p.rows) ln_fwd_load<NV, U, NTX>(p, r0 + stride, slot, lr, cur);
        }
    }
}

// ------------------------------------------------------------------ backward

template <int NV, int U>
struct LnBwdTile {
    uint4 x[U][NV];
    uint4 dy[U][NV];
    float mu[U];
    float rs[U];
};

// NT: 0 plain loads, 1 stream dy, 2 stream x too.
template <int NV, int U, int NT>
__device__ __forceinline__ void ln_bwd_load(const LnBwdParams& p, int64_t r0, int slot, int lr,
                                            LnBwdTile<NV, U>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
        int64_t r = r0 + slot + (int64_t)k * p.rpb;
        if (r > p.rows - 1) r = p.rows - 1;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            int vi = lr + v * p.tpr;
            if (vi > p.nvec - 1) vi = p.nvec - 1;
            const int64_t o = r * p.H + (int64_t)vi * kVec;
            t.x[k][v] = ld16p<(NT >= 2)>(p.x + o);
            t.dy[k][v] = ld16p<(NT >= 1)>(p.dy + o);
        }
        t.mu[k] = p.mean[r];
        t.rs[k] = p.rstd[r];
    }
}

template <int NV, int U>
__device__ __forceinline__ void ln_bwd_ready(const LnBwdTile<NV, U>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            use_now(t.x[k][v]);
            use_now(t.dy[k][v]);
        }
        use_now(t.mu[k]);
        use_now(t.rs[k]);
    }
}

// Floats of the LDS row-sum exchange area of the backward: two sums per
// wave of each row group, double-buffered (none for rows within one wave).
__host__ __device__ inline int ln_bwd_exch_floats(int tpr, int rpb, int U, bool wide) {
    return wide ? 2 * 2 * rpb * U * (tpr >> 6) : 0;
}

// Row-group sums of the two per-lane FP32 sums (sum g, sum g * xhat) of U
// rows, one exchange for both.
template <int U, bool WIDE>
__device__ __forceinline__ void ln_row_sums2(float (&a)[U], float (&b)[U], int tpr, int rpb,
                                             int slot, int lr, float* red, int& buf) {
    if constexpr (WIDE) {
        const int wpr = tpr >> 6;
        const int wave = lr >> 6;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const float sa = group_sum<64>(a[k]);
            const float sb = group_sum<64>(b[k]);
            if ((lr & 63) == 0 && slot < rpb) {
                const int i = (((buf * rpb + slot) * U + k) * wpr + wave) * 2;
                red[i] = sa;
                red[i + 1] = sb;
            }
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float ta = 0.f, tb = 0.f;
            if (slot < rpb) {
                const int i0 = ((buf * rpb + slot) * U + k) * wpr * 2;
                for (int i = 0; i < wpr; ++i) {
                    ta += red[i0 + 2 * i];
                    tb += red[i0 + 2 * i + 1];
                }
            }
            a[k] = ta;
            b[k] = tb;
        }
        buf ^= 1;
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            a[k] = group_sum_rt(a[k], tpr);
            b[k] = group_sum_rt(b[k], tpr);
        }
    }
}

template <int NV, int U, typename WT, bool WIDE, bool F64, int NT>
__global__ void __launch_bounds__(WIDE ? (NV * U >= 2 ? 512 : 1024) : 256)
    k_ln_bwd_row(LnBwdParams p) {
    // Rows of more than 8192 elements take 512 lanes with four vectors each
    // (a 1024-lane group would leave 128 registers per lane, too few for the
    // accumulators of both column sums); with those accumulators a second
    // tile does not fit either, so that shape does not prefetch.
    constexpr bool PF = U <= 2 && !(WIDE && NV == 2 && U == 1);
    // With four vectors per lane the registers go to the FP64 dgamma sums
    // and the two tiles: the FP32 dbeta sums live in LDS (each lane its own
    // slots, same additions in the same order) and BF16 gamma stays packed,
    // unpacked at each use.
    constexpr bool BL = NV >= 4;
    constexpr bool GPK = BL && sizeof(WT) == 2;
    extern __shared__ double lds_lnb[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    // LDS: [2H] doubles for the slot combine, then the row-sum exchange
    // area, then (BL) the dbeta sums, [2 NV][blockDim] float4
    double* comb = lds_lnb;
    float* red = reinterpret_cast<float*>(lds_lnb + (p.rpb > 1 ? 2 * p.H : 0));
    float4* abl = reinterpret_cast<float4*>(red + ln_bwd_exch_floats(p.tpr, p.rpb, U, WIDE));

    float gv[GPK ? 1 : NV][8];
    uint4 gq[GPK ? NV : 1];
    bool vok[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int vi = lr + v * p.tpr;
        vok[v] = (slot < p.rpb) && (vi < p.nvec);
        if constexpr (GPK) {
            gq[v] = vok[v] ? ld16(static_cast<const uint16_t*>(p.gamma) + (int64_t)vi * kVec)
                           : make_uint4(0, 0, 0, 0);
        } else if (vok[v]) {
            load_w8<WT>(p.gamma, vi, gv[v]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gv[v][e] = 0.f;
        }
    }
    auto gamma8 = [&](int v, float (&f)[8]) {
        if constexpr (GPK) {
            unpack8(opaque(gq[v]), f);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = gv[v][e];
        }
    };
    double ag[NV][8];
    float ab[NV][8];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ag[v][e] = 0.0;
            ab[v][e] = 0.f;
        }
    if constexpr (BL) {
#pragma unroll
        for (int i = 0; i < 2 * NV; ++i) abl[i * blockDim.x + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
    }

    const int64_t P = gridDim.x;
    const int64_t b = blockIdx.x;
    const int64_t per_iter = (int64_t)p.rpb * U;
    const int64_t stride = P * per_iter;
    int buf = 0;
    int64_t r0 = b * per_iter;
    if (r0 < p.rows) {
        LnBwdTile<NV, U> cur;
        LnBwdTile<NV, PF ? U : 1> nxt;
        ln_bwd_load<NV, U, NT>(p, r0, slot, lr, cur);
        ln_bwd_ready<NV, U>(cur);
#pragma unroll 1
        for (; r0 < p.rows; r0 += stride) {
            if constexpr (PF) ln_bwd_load<NV, U, NT>(p, r0 + stride, slot, lr, nxt);
            float s1[U], s2[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                s1[k] = 0.f;
                s2[k] = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float xf[8], dyf[8], gf[8];
                    unpack8(cur.x[k][v], xf);
                    unpack8(cur.dy[k][v], dyf);
                    gamma8(v, gf);
                    float a = 0.f, c = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float g = dyf[e] * gf[e];
                        const float xh = (xf[e] - cur.mu[k]) * cur.rs[k];
                        a += g;
                        c = __builtin_fmaf(g, xh, c);
                    }
                    if (vok[v]) {
                        s1[k] += a;
                        s2[k] += c;
                    }
                }
            }
            ln_row_sums2<U, WIDE>(s1, s2, p.tpr, p.rpb, slot, lr, red, buf);
            uint4 out[U][NV];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int64_t r = r0 + slot + (int64_t)k * p.rpb;
                const bool live = (slot < p.rpb) && (r < p.rows);
                const float c1 = s1[k] / (float)p.H;
                const float c2 = s2[k] / (float)p.H;
                const float rs = cur.rs[k];
                const double rs64 = (double)rs;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    float xf[8], dyf[8], o[8], gf[8];
                    // With two or more vectors per lane, holding the first
                    // loop's unpacked values across the exchange would crowd
                    // out the accumulators: recompute them (opaque copies).
                    if constexpr (NV >= 2) {
                        unpack8(opaque(cur.x[k][v]), xf);
                        unpack8(opaque(cur.dy[k][v]), dyf);
                    } else {
                        unpack8(cur.x[k][v], xf);
                        unpack8(cur.dy[k][v], dyf);
                    }
                    gamma8(v, gf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float g = dyf[e] * gf[e];
                        const float d = xf[e] - cur.mu[k];
                        const float xh = d * rs;
                        o[e] = (g - __builtin_fmaf(xh, c2, c1)) * rs;
                        if (live && vok[v]) {
                            ag[v][e] = __builtin_fma((double)(dyf[e] * d), rs64, ag[v][e]);
                            if constexpr (!BL) ab[v][e] += dyf[e];
                        }
                    }
                    if constexpr (BL) {
                        if (live && vok[v]) {
                            float4* q = abl + (2 * v) * blockDim.x + tid;
                            float4 lo = q[0], hi = q[blockDim.x];
                            lo.x += dyf[0]; lo.y += dyf[1]; lo.z += dyf[2]; lo.w += dyf[3];
                            hi.x += dyf[4]; hi.y += dyf[5]; hi.z += dyf[6]; hi.w += dyf[7];
                            q[0] = lo;
                            q[blockDim.x] = hi;
                        }
                    }
                    out[k][v] = pack8(o);
                }
            }
            if constexpr (PF) {
                ln_bwd_ready<NV, U>(nxt);
                cur = nxt;
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int64_t r = r0 + slot + (int64_t)k * p.rpb;
                if (slot >= p.rpb || r >= p.rows) continue;
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    if (!vok[v]) continue;
                    st16_stream(p.dx + r * p.H + (int64_t)(lr + v * p.tpr) * kVec, out[k][v]);
                }
            }
            if constexpr (!PF) {
                if (r0 + stride < p.rows) ln_bwd_load<NV, U, NT>(p, r0 + stride, slot, lr, cur);
            }
        }
    }

    if constexpr (BL) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const float4 lo = abl[(2 * v) * blockDim.x + tid], hi = abl[(2 * v + 1) * blockDim.x + tid];
            ab[v][0] = lo.x; ab[v][1] = lo.y; ab[v][2] = lo.z; ab[v][3] = lo.w;
            ab[v][4] = hi.x; ab[v][5] = hi.y; ab[v][6] = hi.z; ab[v][7] = hi.w;
        }
    }

    // Combine the row slots in slot order (fixed).
    if (p.rpb > 1) {
        for (int s = 1; s < p.rpb; ++s) {
            __syncthreads();
            if (slot == s) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    if (vok[v])
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = (lr + v * p.tpr) * kVec + e;
                            comb[c] = ag[v][e];
                            comb[p.H + c] = (double)ab[v][e];
                        }
            }
            __syncthreads();
            if (slot == 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    if (vok[v])
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int c = (lr + v * p.tpr) * kVec + e;
                            ag[v][e] += comb[c];
                            ab[v][e] += (float)comb[p.H + c];
                        }
            }
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (!vok[v]) continue;
            const int64_t col = (int64_t)(lr + v * p.tpr) * kVec;
            if constexpr (F64) {
                double* row = static_cast<double*>(p.partial) + b * 2 * (int64_t)p.H;
                double2* dg = reinterpret_cast<double2*>(row + col);
                double2* db = reinterpret_cast<double2*>(row + p.H + col);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dg[e] = make_double2(ag[v][2 * e], ag[v][2 * e + 1]);
                    db[e] = make_double2((double)ab[v][2 * e], (double)ab[v][2 * e + 1]);
                }
            } else {
                float* row = static_cast<float*>(p.partial) + b * 2 * (int64_t)p.H;
                float4* dg = reinterpret_cast<float4*>(row + col);
                float4* db = reinterpret_cast<float4*>(row + p.H + col);
                dg[0] = make_float4((float)ag[v][0], (float)ag[v][1], (float)ag[v][2], (float)ag[v][3]);
                dg[1] = make_float4((float)ag[v][4], (float)ag[v][5], (float)ag[v][6], (float)ag[v][7]);
                db[0] = make_float4(ab[v][0], ab[v][1], ab[v][2], ab[v][3]);
                db[1] = make_float4(ab[v][4], ab[v][5], ab[v][6], ab[v][7]);
            }
        }
    }
}

// ----------------------------------------------------------------- launchers

inline size_t ln_fwd_lds_bytes(const rmsn_route_t& r) {
    if (r.lanes_per_row <= 64) return 0;
    return sizeof(double) * 2 * (size_t)r.rows_per_block * r.unroll * (r.lanes_per_row / 64);
}

inline size_t ln_bwd_lds_bytes(const rmsn_route_t& r, int H) {
    size_t lds = r.rows_per_block > 1 ? sizeof(double) * 2 * (size_t)H : 0;
    lds += sizeof(float) *
           (size_t)ln_bwd_exch_floats(r.lanes_per_row, r.rows_per_block, r.unroll, r.lanes_per_row > 64);
    if (r.vec_per_lane >= 4) lds += 16 * 2 * (size_t)r.vec_per_lane * r.block_threads;  // dbeta sums
    return lds;
}

template <int NV, int U, typename WT>
static int launch_ln_fwd_t(const LnFwdParams& p, const Route& rt, hipStream_t s) {
    const size_t lds = ln_fwd_lds_bytes(rt.r);
    dim3 grid((unsigned)rt.r.grid), block((unsigned)rt.r.block_threads);
    const bool ntx = rt.r.stream_loads >= 2;
    if (rt.r.lanes_per_row > 64) {
        if (ntx) launch_kernel((k_ln_fwd<NV, U, WT, true, true>), grid, block, lds, s, p);
        else launch_kernel((k_ln_fwd<NV, U, WT, true, false>), grid, block, lds, s, p);
    } else {
        if (ntx) launch_kernel((k_ln_fwd<NV, U, WT, false, true>), grid, block, lds, s, p);
        else launch_kernel((k_ln_fwd<NV, U, WT, false, false>), grid, block, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

// (NV, U) pairs compiled for the LayerNorm forward.
template <typename WT>
static int launch_ln_fwd_wt(const LnFwdParams& p, const Route& rt, hipStream_t s) {
    const int nv = rt.r.vec_per_lane, u = rt.r.unroll;
    if (nv == 1 && u == 1) return launch_ln_fwd_t<1, 1, WT>(p, rt, s);
    if (nv == 1 && u == 2) return launch_ln_fwd_t<1, 2, WT>(p, rt, s);
    if (nv == 2 && u == 1) return launch_ln_fwd_t<2, 1, WT>(p, rt, s);
    if (nv == 2 && u == 2) return launch_ln_fwd_t<2, 2, WT>(p, rt, s);
    if (nv == 2 && u == 4) return launch_ln_fwd_t<2, 4, WT>(p, rt, s);
    if (nv == 4 && u == 1) return launch_ln_fwd_t<4, 1, WT>(p, rt, s);
    return RMSN_ERR_SHAPE;
}

template <int NV, int U, typename WT, bool WIDE, int NT>
static int launch_ln_bwd_nt(const LnBwdParams& p, const Route& rt, size_t lds, hipStream_t s) {
    dim3 grid((unsigned)rt.r.grid), block((unsigned)rt.r.block_threads);
    if (rt.r.partial_f64)
        launch_kernel((k_ln_bwd_row<NV, U, WT, WIDE, true, NT>), grid, block, lds, s, p);
    else
        launch_kernel((k_ln_bwd_row<NV, U, WT, WIDE, false, NT>), grid, block, lds, s, p);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <int NV, int U, typename WT, bool WIDE>
static int launch_ln_bwd_mode(const LnBwdParams& p, const Route& rt, size_t lds, hipStream_t s) {
    switch (rt.r.stream_loads) {
        case 0: return launch_ln_bwd_nt<NV, U, WT, WIDE, 0>(p, rt, lds, s);
        case 1: return launch_ln_bwd_nt<NV, U, WT, WIDE, 1>(p, rt, lds, s);
        case 2: return launch_ln_bwd_nt<NV, U, WT, WIDE, 2>(p, rt, lds, s);
        default: return RMSN_ERR_SHAPE;
    }
}

template <int NV, int U, typename WT>
static int launch_ln_bwd_t(const LnBwdParams& p, const Route& rt, hipStream_t s) {
    const size_t lds = ln_bwd_lds_bytes(rt.r, p.H);
    if (rt.r.lanes_per_row > 64) return launch_ln_bwd_mode<NV, U, WT, true>(p, rt, lds, s);
    return launch_ln_bwd_mode<NV, U, WT, false>(p, rt, lds, s);
}

// (NV, U) pairs compiled for the LayerNorm backward.
template <typename WT>
static int launch_ln_bwd_wt(const LnBwdParams& p, const Route& rt, hipStream_t s) {
    const int nv = rt.r.vec_per_lane, u = rt.r.unroll;
    if (nv == 1 && u == 1) return launch_ln_bwd_t<1, 1, WT>(p, rt, s);
    if (nv == 1 && u == 2) return launch_ln_bwd_t<1, 2, WT>(p, rt, s);
    if (nv == 2 && u == 1) return launch_ln_bwd_t<2, 1, WT>(p, rt, s);
    if (nv == 2 && u == 2) return launch_ln_bwd_t<2, 2, WT>(p, rt, s);
    if (nv == 4 && u == 1) return launch_ln_bwd_t<4, 1, WT>(p, rt, s);
    return RMSN_ERR_SHAPE;
}

}  // namespace rmsn
