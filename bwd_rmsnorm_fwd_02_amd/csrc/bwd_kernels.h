// RMSNorm backward for gfx950 (kernel templates): dx per row, and dw as a
// column sum over rows.
//
// Per row (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
// backward routes", opening description): with xhat = x * rstd and
// g = dy * w, c = mean(g * xhat), dx = BF16(rstd * (g - xhat * c)); in the
// residual form ("Key": combined grad) dh = BF16(dres + that gradient). dx
// is computed by one function (bwd_compute) for every kernel and mode here; for
// a given launch shape it is bit-identical between deterministic and
// non-deterministic calls.
//
// dw_j = sum over rows of dy * xhat. Each lane owns fixed columns (the same
// 16-byte vectors it owns in every row) and accumulates dy*x*rstd in FP64
// registers: dy*x is exact in FP32 (two 8-bit significands), and the FP64
// fused multiply-add by the row's rstd loses nothing that matters. gfx950
// runs FP64 FMA at the rate of unpacked FP32, so this costs three vector
// operations per element and replaces the compensated FP32 sums (TwoSum
// plus periodic FP64 fold) that the pages use on hardware with slow FP64.
//
// How the per-block sums meet:
// * fixed order (both modes, as the route table has them): block b takes the
//   row tiles b, b + P, b + 2P, ..., where P (the grid) is a function of the
//   shape only; it adds them in that order, combines its row slots in slot
//   order and writes its partial row; k_dw_reduce then sums the P partials
//   in a fixed order. No step depends on scheduling or on the CU count.
// * atomic (the non-deterministic mode, only through a route override, as
//   it measured slower): the same blocks add their sums into an FP64
//   accumulator with hardware atomics; the last block to finish (a ticket
//   counter) converts it to FP32 dw.
// * small T: one launch of k_bwd_small — column tasks sum whole columns over
//   every row in a fixed row order while row tasks produce dx.
//
// Recompute form (RC): the row kernel takes no rstd input and forms each
// row's rstd from the x row it already holds, with the forward's arithmetic
// (FP32 sums of squares per 16-byte vector, added in FP64, one rounding of
// 1/sqrt(mean + eps) to FP32). For activation recompute, where a training
// step runs the forward, the forward again, then the backward (the pages'
// "2xfwd+bwd"), this serves callers that kept x but not rstd.
#pragma once

#include "rmsn_device.h"

namespace rmsn {

enum { kModePartF32 = 0, kModePartF64 = 1, kModeAtomic = 2 };

// Rows a row group holds at once: x, dy, (dres), rstd for U rows.
template <int NV, int U, bool RES>
struct BwdTile {
    uint4 x[U][NV];
    uint4 dy[U][NV];
    uint4 dres[U][NV];  // RES with a residual gradient only
    float rs[U];
};

// Issue the loads of rows r0 + slot + k*rpb (k < U). Every lane issues the
// same loads: rows at or past rend and vectors past the row end are clamped
// to the last valid ones and their values ignored, so there are no branches
// around memory operations (branches there make the compiler's wait counting
// fall back to waiting for everything). Without a residual gradient the dres
// slot reloads dy, which stays unused.
// NT: 0 plain loads, 1 stream dy (and dres), 2 stream x too.
template <int NV, int U, bool RES, bool RC = false, int NT = 0>
__device__ __forceinline__ void bwd_load(const BwdParams& p, int64_t r0, int64_t rend, int slot,
                                         int lr, BwdTile<NV, U, RES>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
        int64_t r = r0 + slot + (int64_t)k * p.rpb;
        if (r > rend - 1) r = rend - 1;
        const int64_t ox = row_offset(r, p.heads, p.ax);
        const int64_t ody = row_offset(r, p.heads, p.ady);
        int64_t ores = 0;
        const uint16_t* rsrc = p.dy;
        if constexpr (RES) {
            if (p.dres) {
                ores = row_offset(r, p.heads, p.ares);
                rsrc = p.dres;
            } else {
                ores = ody;
            }
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            int vi = lr + v * p.tpr;
            if (vi > p.nvec - 1) vi = p.nvec - 1;
            const int64_t c = (int64_t)vi * kVec;
            t.x[k][v] = ld16p<(NT >= 2)>(p.x + ox + c);
            t.dy[k][v] = ld16p<(NT >= 1)>(p.dy + ody + c);
            if constexpr (RES) t.dres[k][v] = ld16p<(NT >= 1)>(rsrc + ores + c);
        }
        if constexpr (!RC) t.rs[k] = p.rstd[r];
    }
}

template <int NV, int U, bool RES, bool RC = false>
__device__ __forceinline__ void bwd_ready(const BwdTile<NV, U, RES>& t) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            use_now(t.x[k][v]);
            use_now(t.dy[k][v]);
            if constexpr (RES) use_now(t.dres[k][v]);
        }
        if constexpr (!RC) use_now(t.rs[k]);
    }
}

// Row-group sums of U per-lane FP32 values (the dot products) and, in the
// recompute form, U FP64 values (the sums of squares). WIDE rows span
// several waves and exchange wave sums through LDS (FP32 area `red`, FP64
// area `redd`), double-buffered by `buf` so that one LDS-only barrier per
// iteration suffices. The order of every sum is fixed; the dot products are
// summed the same way in every form, so dx does not depend on the form. The
// sums of squares take the vector-ALU reduction (wave_sums): they are exact
// in FP64 in any order, and it keeps their exchange short.
template <int U, bool WIDE, bool RC>
__device__ __forceinline__ void row_sums(float (&dot)[U], double (&ss)[U], const BwdParams& p,
                                         int slot, int lr, float* red, double* redd, int& buf) {
    if constexpr (WIDE) {
        const int wpr = p.tpr >> 6;
        const int wave = lr >> 6;
        const int lane = lr & 63;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const float a = group_sum<64>(dot[k]);
            if (lane == 0 && slot < p.rpb) red[((buf * p.rpb + slot) * U + k) * wpr + wave] = a;
        }
        if constexpr (RC) {
            // lane q < U holds the sum of squares of row wave_row<U>(q)
            const double b = wave_sums<U>(ss, lane);
            if (lane < U && slot < p.rpb)
                redd[((buf * p.rpb + slot) * U + wave_row<U>(lane)) * wpr + wave] = b;
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float t = 0.f;
            double q = 0.0;
            if (slot < p.rpb) {
                const int i0 = ((buf * p.rpb + slot) * U + k) * wpr;
                for (int i = 0; i < wpr; ++i) {
                    t += red[i0 + i];
                    if constexpr (RC) q += redd[i0 + i];
                }
            }
            dot[k] = t;
            if constexpr (RC) ss[k] = q;
        }
        buf ^= 1;
    } else {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            dot[k] = group_sum_rt(dot[k], p.tpr);
            if constexpr (RC) ss[k] = group_sum_rt(ss[k], p.tpr);
        }
    }
}

// The backward of the rows held in a tile, up to the stores: dx (or dh)
// packed into `out`, and, if ACC, dy*x*rstd added into acc for rows below
// rend. No memory operation happens here except the LDS exchange of row
// sums (`red` FP32, `redd` FP64 for the recompute form's sums of squares).
template <int NV, int U, bool RES, bool WIDE, bool ACC, bool RC = false>
__device__ __forceinline__ void bwd_compute(const BwdParams& p, int64_t r0, int64_t rend,
                                            int slot, int lr, const float (&wv)[NV][8],
                                            const bool (&vok)[NV], const BwdTile<NV, U, RES>& t,
                                            double (&acc)[NV][8], uint4 (&out)[U][NV], float* red,
                                            double* redd, int& buf) {
    float dot[U];
    double ss[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        dot[k] = 0.f;
        ss[k] = 0.0;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float xf[8], dyf[8];
            unpack8(t.x[k][v], xf);
            unpack8(t.dy[k][v], dyf);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = __builtin_fmaf(dyf[e] * wv[v][e], xf[e], s);
            if (vok[v]) dot[k] += s;
            if constexpr (RC) {
                // the forward's per-vector sum of squares, added in FP64
                float q = xf[0] * xf[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) q = __builtin_fmaf(xf[e], xf[e], q);
                if (vok[v]) ss[k] += (double)q;
            }
        }
    }
    row_sums<U, WIDE, RC>(dot, ss, p, slot, lr, red, redd, buf);
    float rsc[U];
    if constexpr (RC) {
#pragma unroll
        for (int k = 0; k < U; ++k)
            rsc[k] = (float)(1.0 / __builtin_sqrt(ss[k] / (double)p.H + (double)p.eps));
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t r = r0 + slot + (int64_t)k * p.rpb;
        const bool live = (slot < p.rpb) && (r < rend);
        float rs;
        if constexpr (RC) rs = rsc[k];
        else rs = t.rs[k];
        // c = (1/H) sum_j g_j * xhat_j = rstd * sum_j g_j x_j / H
        const float c = (dot[k] * rs) / (float)p.H;
        const double rs64 = (double)rs;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float xf[8], dyf[8], o[8];
            if constexpr (NV >= 4) {
                // four vectors per lane: recompute the unpacked row rather
                // than hold the first loop's copy across the exchange
                unpack8(opaque(t.x[k][v]), xf);
                unpack8(opaque(t.dy[k][v]), dyf);
            } else {
                unpack8(t.x[k][v], xf);
                unpack8(t.dy[k][v], dyf);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = dyf[e] * wv[v][e];
                const float xh = xf[e] * rs;
                o[e] = __builtin_fmaf(-xh, c, g) * rs;
            }
            if constexpr (RES) {
                if (p.dres) {
                    float d[8];
                    unpack8(t.dres[k][v], d);
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] += d[e];
                }
            }
            out[k][v] = pack8(o);
            if constexpr (ACC) {
                if (live && vok[v]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[v][e] = __builtin_fma((double)(dyf[e] * xf[e]), rs64, acc[v][e]);
                }
            }
        }
    }
}

// Store the dx (or dh) rows of a tile that lie below rend.
template <int NV, int U>
__device__ __forceinline__ void bwd_store(const BwdParams& p, int64_t r0, int64_t rend, int slot,
                                          int lr, const bool (&vok)[NV], const uint4 (&out)[U][NV]) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int64_t r = r0 + slot + (int64_t)k * p.rpb;
        if (slot >= p.rpb || r >= rend) continue;
        const int64_t odx = row_offset(r, p.heads, p.adx);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (!vok[v]) continue;
            st16_stream(p.dx + odx + (int64_t)(lr + v * p.tpr) * kVec, out[k][v]);
        }
    }
}

template <int NV, typename WT>
__device__ __forceinline__ void load_weights(const BwdParams& p, int slot, int lr,
                                             float (&wv)[NV][8], bool (&vok)[NV]) {
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
}

// Large-T row kernel: dx for the block's rows plus the block's dw sums.
// Each iteration a row group takes U rows; with U <= 2 the next iteration's
// rows are loaded before the current ones are processed.
// Blocks of rows wider than a wave hold at most 512 threads once a lane
// holds more than one 16-byte vector per tensor (NV * U >= 2): with 1024
// the 128 registers a lane may use are too few and the tile spills.
template <int NV, int U, typename WT, bool RES, bool WIDE, int MODE, bool RC = false, int NT = 0,
          bool CA = false>
__global__ void __launch_bounds__(WIDE ? (NV * U >= 2 ? 512 : 1024) : 256) k_bwd_row(BwdParams p) {
    // Rows above 8192 elements take four vectors per lane on 512 lanes (a
    // 1024-lane group leaves 128 registers per lane); with the row unpacked
    // again after the exchange, the prefetched tile still fits (about 235
    // registers).
    constexpr bool PF = U <= 2;
    extern __shared__ double lds_bwd[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    // LDS: [H] doubles for the serial slot combine, then (recompute form)
    // the FP64 exchange area, then the FP32 row-sum exchange area. The
    // one-step combine (CA) takes [rpb, H] doubles from the start, over the
    // exchange areas, once the loop is done with them.
    double* comb = lds_bwd;
    double* redd = lds_bwd + (p.rpb > 1 ? p.H : 0);
    const int nexch = WIDE ? 2 * p.rpb * U * (p.tpr >> 6) : 0;
    float* red = reinterpret_cast<float*>(redd + (RC ? nexch : 0));

    float wv[NV][8];
    bool vok[NV];
    load_weights<NV, WT>(p, slot, lr, wv, vok);

    double acc[NV][8];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[v][e] = 0.0;

    // Block b takes iterations b, b + P, b + 2P, ... of per_iter rows each:
    // a fixed partition (a function of the shape and the route only) in which
    // all blocks sweep one compact window of rows together, which keeps the
    // HBM access stream local.
    const int64_t P = gridDim.x;
    const int64_t b = blockIdx.x;
    const int64_t per_iter = (int64_t)p.rpb * U;
    const int64_t stride = P * per_iter;
    const int64_t rend = p.rows;
    int buf = 0;
    int64_t r0 = b * per_iter;
    if (r0 < rend) {
        BwdTile<NV, U, RES> cur;
        BwdTile<NV, PF ? U : 1, RES> nxt;
        bwd_load<NV, U, RES, RC, NT>(p, r0, rend, slot, lr, cur);
        bwd_ready<NV, U, RES, RC>(cur);
#pragma unroll 1
        for (; r0 < rend; r0 += stride) {
            if constexpr (PF) bwd_load<NV, U, RES, RC, NT>(p, r0 + stride, rend, slot, lr, nxt);
            uint4 out[U][NV];
            bwd_compute<NV, U, RES, WIDE, true, RC>(p, r0, rend, slot, lr, wv, vok, cur, acc, out, red,
                                                    redd, buf);
            // The next tile must be complete before its registers take over;
            // the wait lands before this iteration's stores are issued.
            if constexpr (PF) {
                bwd_ready<NV, U, RES, RC>(nxt);
                cur = nxt;
            }
            bwd_store<NV, U>(p, r0, rend, slot, lr, vok, out);
            if constexpr (!PF) {
                if (r0 + stride < rend) bwd_load<NV, U, RES, RC, NT>(p, r0 + stride, rend, slot, lr, cur);
            }
        }
    }

    // Combine the row slots in slot order: acc(0) + acc(1) + ... (fixed).
    if constexpr (CA && (MODE == kModePartF64 || MODE == kModePartF32)) {
        // Every slot stores its sums at once; then each thread folds
        // whole columns in slot order (the same additions as the serial
        // form below) and writes them to the block's partial row.
        __syncthreads();
        if (slot < p.rpb) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
                if (vok[v])
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        comb[(int64_t)slot * p.H + (lr + v * p.tpr) * kVec + e] = acc[v][e];
        }
        __syncthreads();
        // a thread takes column pairs; the reads of four slots are issued
        // before their sums
        const int npair = p.H >> 1;
        for (int i = tid; i < npair; i += (int)blockDim.x) {
            const double2* cp = reinterpret_cast<const double2*>(comb) + i;
            double2 sum = cp[0];
            int q = 1;
            for (; q + 4 <= p.rpb; q += 4) {
                const double2 a0 = cp[(int64_t)q * npair], a1 = cp[(int64_t)(q + 1) * npair];
                const double2 a2 = cp[(int64_t)(q + 2) * npair], a3 = cp[(int64_t)(q + 3) * npair];
                sum.x += a0.x; sum.y += a0.y;
                sum.x += a1.x; sum.y += a1.y;
                sum.x += a2.x; sum.y += a2.y;
                sum.x += a3.x; sum.y += a3.y;
            }
            for (; q < p.rpb; ++q) {
                const double2 a = cp[(int64_t)q * npair];
                sum.x += a.x; sum.y += a.y;
            }
            if constexpr (MODE == kModePartF64)
                reinterpret_cast<double2*>(static_cast<double*>(p.partial) + b * p.H)[i] = sum;
            else
                reinterpret_cast<float2*>(static_cast<float*>(p.partial) + b * p.H)[i] =
                    make_float2((float)sum.x, (float)sum.y);
        }
        return;
    }
    if (p.rpb > 1) {
        for (int s = 1; s < p.rpb; ++s) {
            __syncthreads();
            if (slot == s) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    if (vok[v])
#pragma unroll
                        for (int e = 0; e < 8; ++e) comb[(lr + v * p.tpr) * kVec + e] = acc[v][e];
            }
            __syncthreads();
            if (slot == 0) {
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    if (vok[v])
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[v][e] += comb[(lr + v * p.tpr) * kVec + e];
            }
        }
    }

    if constexpr (MODE == kModePartF64 || MODE == kModePartF32) {
        if (slot == 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (!vok[v]) continue;
                const int64_t col = (int64_t)(lr + v * p.tpr) * kVec;
                if constexpr (MODE == kModePartF64) {
                    double2* dst = reinterpret_cast<double2*>(static_cast<double*>(p.partial) + b * p.H + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = make_double2(acc[v][2 * e], acc[v][2 * e + 1]);
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.partial) + b * p.H + col);
                    dst[0] = make_float4((float)acc[v][0], (float)acc[v][1], (float)acc[v][2], (float)acc[v][3]);
                    dst[1] = make_float4((float)acc[v][4], (float)acc[v][5], (float)acc[v][6], (float)acc[v][7]);
                }
            }
        }
    } else if constexpr (MODE == kModeAtomic) {
        if (slot == 0) {
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (!vok[v]) continue;
                const int64_t col = (int64_t)(lr + v * p.tpr) * kVec;
#pragma unroll
                for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p.acc + col + e, acc[v][e]);
            }
        }
        __threadfence();
        __syncthreads();
        __shared__ unsigned int last;
        if (tid == 0) last = (atomicAdd(p.ticket, 1u) == (unsigned int)(P - 1)) ? 1u : 0u;
        __syncthreads();
        if (last) {
            __threadfence();
            for (int j = tid; j < p.H; j += blockDim.x) {
                unsigned long long old =
                    atomicExch(reinterpret_cast<unsigned long long*>(p.acc + j), 0ull);
                p.dw[j] = (float)__longlong_as_double((long long)old);
            }
            if (tid == 0) atomicExch(p.ticket, 0u);
        }
    }
}

// Small-T backward, one launch. Blocks [0, ncol_blocks) are column tasks:
// thread (vector column v, split s) sums rows [s*T/S, (s+1)*T/S) in order,
// and the S split sums are added in split order. The other blocks are row
// tasks computing dx with the shared row code.
template <int NV, typename WT, bool RES>
__global__ void __launch_bounds__(256) k_bwd_small(BwdParams p) {
    extern __shared__ double lds_small[];
    const int tid = threadIdx.x;
    if ((int)blockIdx.x < p.ncol_blocks) {
        const int S = p.col_splits;
        const int vb = blockDim.x / S;  // vector columns per block
        const int lv = tid % vb;
        const int s = tid / vb;
        const int v = blockIdx.x * vb + lv;
        double a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0.0;
        if (v < p.nvec) {
            const int64_t r0 = ((int64_t)s * p.rows) / S;
            const int64_t r1 = ((int64_t)(s + 1) * p.rows) / S;
            for (int64_t r = r0; r < r1; ++r) {
                const int64_t ox = row_offset(r, p.heads, p.ax) + (int64_t)v * kVec;
                const int64_t ody = row_offset(r, p.heads, p.ady) + (int64_t)v * kVec;
                float xf[8], dyf[8];
                unpack8(ld16(p.x + ox), xf);
                unpack8(ld16(p.dy + ody), dyf);
                const double rs = (double)p.rstd[r];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = __builtin_fma((double)(dyf[e] * xf[e]), rs, a[e]);
            }
        }
        double* sm = lds_small;  // [S][vb*8]
#pragma unroll
        for (int e = 0; e < 8; ++e) sm[(s * vb + lv) * 8 + e] = a[e];
        __syncthreads();
        if (s == 0 && v < p.nvec) {
            for (int q = 1; q < S; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] += sm[(q * vb + lv) * 8 + e];
#pragma unroll
            for (int e = 0; e < 8; ++e) p.dw[(int64_t)v * kVec + e] = (float)a[e];
        }
        return;
    }
    // Row task: rows [rb, rb + rpb), one per row group.
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    float wv[NV][8];
    bool vok[NV];
    load_weights<NV, WT>(p, slot, lr, wv, vok);
    double acc[NV][8];
    float* red = reinterpret_cast<float*>(lds_small);
    int buf = 0;
    const int64_t rb = (int64_t)(blockIdx.x - p.ncol_blocks) * p.rpb;
    BwdTile<NV, 1, RES> t;
    uint4 out[1][NV];
    bwd_load<NV, 1, RES>(p, rb, p.rows, slot, lr, t);
    if (p.tpr > 64)
        bwd_compute<NV, 1, RES, true, false>(p, rb, p.rows, slot, lr, wv, vok, t, acc, out, red,
                                             nullptr, buf);
    else
        bwd_compute<NV, 1, RES, false, false>(p, rb, p.rows, slot, lr, wv, vok, t, acc, out, red,
                                              nullptr, buf);
    bwd_store<NV, 1>(p, rb, p.rows, slot, lr, vok, out);
}

// ----------------------------------------------------------------- launchers

// LDS of the row kernel: the serial combine's [H] doubles (several slots)
// and the loop's row-sum exchange after them; the one-step combine reuses
// the whole area and extends it to [rpb, H] doubles.
inline size_t bwd_row_lds_bytes(const rmsn_route_t& r, int H, bool rc) {
    size_t lds = r.rows_per_block > 1 ? sizeof(double) * (size_t)H : 0;
    if (r.lanes_per_row > 64) {
        const size_t n = 2 * (size_t)r.rows_per_block * r.unroll * (r.lanes_per_row / 64);
        lds += sizeof(float) * n;
        if (rc) lds += sizeof(double) * n;
    }
    if (bwd_row_comb_all(r, H)) {
        const size_t all = sizeof(double) * (size_t)r.rows_per_block * (size_t)H;
        if (all > lds) lds = all;
    }
    return lds;
}

// CA: the one-step slot combine (bwd_row_comb_all), compiled as its own
// kernels so that the serial-combine kernels keep their code unchanged.
template <int NV, int U, typename WT, bool RES, bool WIDE, bool RC, int NT, bool CA>
static int launch_row_nt(const BwdParams& p, const Route& rt, size_t lds, hipStream_t s) {
    dim3 grid((unsigned)rt.r.grid), block((unsigned)rt.r.block_threads);
    if (rt.r.kind == RMSN_KIND_BWD_ROW_ATOMIC) {
        if constexpr (NV == 1 && U <= 2 && !CA)
            launch_kernel((k_bwd_row<NV, U, WT, RES, WIDE, kModeAtomic, RC, NT>), grid, block, lds, s, p);
        else
            return RMSN_ERR_SHAPE;
    } else if (rt.r.partial_f64) {
        launch_kernel((k_bwd_row<NV, U, WT, RES, WIDE, kModePartF64, RC, NT, CA>), grid, block, lds, s, p);
    } else {
        launch_kernel((k_bwd_row<NV, U, WT, RES, WIDE, kModePartF32, RC, NT, CA>), grid, block, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <int NV, int U, typename WT, bool RES, bool WIDE, bool RC, bool CA>
static int launch_row_mode(const BwdParams& p, const Route& rt, size_t lds, hipStream_t s) {
    switch (rt.r.stream_loads) {
        case 0: return launch_row_nt<NV, U, WT, RES, WIDE, RC, 0, CA>(p, rt, lds, s);
        case 1: return launch_row_nt<NV, U, WT, RES, WIDE, RC, 1, CA>(p, rt, lds, s);
        case 2: return launch_row_nt<NV, U, WT, RES, WIDE, RC, 2, CA>(p, rt, lds, s);
        default: return RMSN_ERR_SHAPE;
    }
}

template <int NV, int U, typename WT, bool RES, bool RC, bool CA>
static int launch_row_t(const BwdParams& p, const Route& rt, hipStream_t s) {
    if (bwd_row_comb_all(rt.r, p.H) != CA) return RMSN_ERR_SHAPE;
    const size_t lds = bwd_row_lds_bytes(rt.r, p.H, RC);
    if (rt.r.lanes_per_row > 64) return launch_row_mode<NV, U, WT, RES, true, RC, CA>(p, rt, lds, s);
    return launch_row_mode<NV, U, WT, RES, false, RC, CA>(p, rt, lds, s);
}

// (NV, U) pairs compiled: NV * U <= 4 (eight vectors per lane and tensor
// spill at any block size).
template <typename WT, bool RES, bool RC, bool CA>
static int launch_row_shape(const BwdParams& p, const Route& rt, hipStream_t s) {
    const int nv = rt.r.vec_per_lane, u = rt.r.unroll;
    if (nv == 4) return u == 1 ? launch_row_t<4, 1, WT, RES, RC, CA>(p, rt, s) : RMSN_ERR_SHAPE;
    if (nv == 1) {
        switch (u) {
            case 1: return launch_row_t<1, 1, WT, RES, RC, CA>(p, rt, s);
            case 2: return launch_row_t<1, 2, WT, RES, RC, CA>(p, rt, s);
            case 4: return launch_row_t<1, 4, WT, RES, RC, CA>(p, rt, s);
        }
    } else if (nv == 2) {
        switch (u) {
            case 1: return launch_row_t<2, 1, WT, RES, RC, CA>(p, rt, s);
            case 2: return launch_row_t<2, 2, WT, RES, RC, CA>(p, rt, s);
        }
    }
    return RMSN_ERR_SHAPE;
}

template <int NV, typename WT, bool RES>
static int launch_small_t(const BwdParams& p, const Route& rt, hipStream_t s) {
    const rmsn_route_t& r = rt.r;
    const int vb = 256 / p.col_splits;
    size_t lds = sizeof(double) * (size_t)p.col_splits * vb * 8;
    const size_t lds_red =
        sizeof(float) * 2 * r.rows_per_block * (r.lanes_per_row > 64 ? r.lanes_per_row / 64 : 1);
    if (lds_red > lds) lds = lds_red;
    launch_kernel((k_bwd_small<NV, WT, RES>), dim3((unsigned)r.grid), dim3(256), lds, s, p);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <typename WT, bool RES>
static int launch_small_shape(const BwdParams& p, const Route& rt, hipStream_t s) {
    switch (rt.r.vec_per_lane) {
        case 1: return launch_small_t<1, WT, RES>(p, rt, s);
        case 2: return launch_small_t<2, WT, RES>(p, rt, s);
        case 4: return launch_small_t<4, WT, RES>(p, rt, s);
        case 8: return launch_small_t<8, WT, RES>(p, rt, s);
        default: return RMSN_ERR_SHAPE;
    }
}

// form: kFormPlain, kFormResidual or kFormRecompute.
template <typename WT, bool CA>
static int launch_bwd_row_wt(const BwdParams& p, const Route& rt, int form, hipStream_t s) {
    switch (form) {
        case kFormPlain: return launch_row_shape<WT, false, false, CA>(p, rt, s);
        case kFormResidual: return launch_row_shape<WT, true, false, CA>(p, rt, s);
        case kFormRecompute: return launch_row_shape<WT, false, true, CA>(p, rt, s);
        default: return RMSN_ERR_SHAPE;
    }
}

template <typename WT>
static int launch_bwd_small_wt(const BwdParams& p, const Route& rt, bool residual, hipStream_t s) {
    return residual ? launch_small_shape<WT, true>(p, rt, s) : launch_small_shape<WT, false>(p, rt, s);
}

}  // namespace rmsn
