// RMSNorm backward for gfx950: dx per row, and dw as a column sum over rows.
//
// Per row (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
// backward routes", opening description): with xhat = x * rstd and
// g = dy * w, c = mean(g * xhat), dx = BF16(rstd * (g - xhat * c)); in the
// residual form ("Key": combined grad) dh = BF16(dres + that gradient). dx
// uses the same arithmetic in every mode and route of this file, so it is
// bit-identical between deterministic and non-deterministic calls.
//
// dw_j = sum over rows of dy * xhat. Each lane owns fixed columns (the same
// 16-byte vectors it owns in every row) and accumulates dy*x*rstd in FP64
// registers: dy*x is exact in FP32 (two 8-bit significands), and the FP64
// fused multiply-add by the row's rstd loses nothing that matters. gfx950
// runs FP64 FMA at the rate of unpacked FP32, so this costs three vector
// operations per element and replaces the compensated FP32 sums (TwoSum
// plus periodic FP64 fold) that the pages use on hardware with slow FP64.
//
// How the per-block sums meet (the only difference between the modes):
// * deterministic: block b owns the contiguous row range
//   [b*rows/P, (b+1)*rows/P), where P (the grid) is a function of the shape
//   only; row slots inside the block are combined in slot order; the block
//   writes its partial row; k_dw_reduce then sums the P partials in a fixed
//   order. No step depends on scheduling or on the CU count.
// * atomic (non-deterministic): the same blocks add their sums into an FP64
//   accumulator with hardware atomics; the last block to finish (a ticket
//   counter) converts it to FP32 dw and clears the accumulator and counter.
// * small T: one launch of k_bwd_small — column tasks sum whole columns over
//   every row in a fixed row order while row tasks produce dx.
#include "rmsn_device.h"

namespace rmsn {

enum { kModePartF32 = 0, kModePartF64 = 1, kModeAtomic = 2, kModeNoDw = 3 };

// Row-group sum of a per-lane FP32 value. WIDE rows span several waves and
// exchange wave sums through LDS (double-buffered by `buf`).
template <bool WIDE>
__device__ __forceinline__ float row_sum(float v, const BwdParams& p, int slot, int lr,
                                         float* red, int& buf) {
    if constexpr (WIDE) {
        const int wpr = p.tpr >> 6;
        v = group_sum<64>(v);
        if ((lr & 63) == 0 && slot < p.rpb) red[(buf * p.rpb + slot) * wpr + (lr >> 6)] = v;
        __syncthreads();
        float t = 0.f;
        if (slot < p.rpb)
            for (int i = 0; i < wpr; ++i) t += red[(buf * p.rpb + slot) * wpr + i];
        buf ^= 1;
        return t;
    } else {
        return group_sum_rt(v, p.tpr);
    }
}

// The per-row backward shared by every kernel here. Loads the row, computes
// and stores dx, and (if ACC) adds dy*x*rstd into acc.
template <int NV, typename WT, bool RES, bool WIDE, bool ACC>
__device__ __forceinline__ void bwd_one_row(const BwdParams& p, int64_t r, bool active,
                                            int slot, int lr, const float (&wv)[NV][8],
                                            const bool (&vok)[NV], double (&acc)[NV][8],
                                            float* red, int& buf) {
    float xf[NV][8], dyf[NV][8];
    float rs = 0.f;
    float dot = 0.f;
    if (active) {
        const int64_t ox = row_offset(r, p.heads, p.ax);
        const int64_t ody = row_offset(r, p.heads, p.ady);
        uint4 xv[NV], dv[NV];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (!vok[k]) continue;
            const int64_t c = (int64_t)(lr + k * p.tpr) * kVec;
            xv[k] = ld16(p.x + ox + c);
            dv[k] = ld16(p.dy + ody + c);
        }
        rs = p.rstd[r];
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            if (!vok[k]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[k][e] = dyf[k][e] = 0.f;
                continue;
            }
            unpack8(xv[k], xf[k]);
            unpack8(dv[k], dyf[k]);
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) s = __builtin_fmaf(dyf[k][e] * wv[k][e], xf[k][e], s);
            dot += s;
        }
    }
    const float sum_gx = row_sum<WIDE>(dot, p, slot, lr, red, buf);
    if (!active) return;
    // c = (1/H) sum_j g_j * xhat_j = rstd * sum_j g_j x_j / H
    const float c = (sum_gx * rs) / (float)p.H;
    const int64_t odx = row_offset(r, p.heads, p.adx);
    int64_t ores = 0;
    if constexpr (RES) {
        if (p.dres) ores = row_offset(r, p.heads, p.ares);
    }
    const double rs64 = (double)rs;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        if (!vok[k]) continue;
        const int64_t col = (int64_t)(lr + k * p.tpr) * kVec;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float g = dyf[k][e] * wv[k][e];
            const float xh = xf[k][e] * rs;
            o[e] = __builtin_fmaf(-xh, c, g) * rs;
        }
        if constexpr (RES) {
            if (p.dres) {
                float d[8];
                unpack8(ld16(p.dres + ores + col), d);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += d[e];
            }
        }
        st16(p.dx + odx + col, pack8(o));
        if constexpr (ACC) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[k][e] = __builtin_fma((double)(dyf[k][e] * xf[k][e]), rs64, acc[k][e]);
        }
    }
}

template <int NV, typename WT>
__device__ __forceinline__ void load_weights(const BwdParams& p, int slot, int lr,
                                             float (&wv)[NV][8], bool (&vok)[NV]) {
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
}

// Large-T row kernel: dx for the block's rows plus the block's dw sums.
template <int NV, typename WT, bool RES, bool WIDE, int MODE>
__global__ void __launch_bounds__(1024) k_bwd_row(BwdParams p) {
    extern __shared__ double lds_bwd[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    // LDS: [H] doubles for the slot combine, then the row-sum exchange area
    double* comb = lds_bwd;
    float* red = reinterpret_cast<float*>(lds_bwd + (p.rpb > 1 ? p.H : 0));

    float wv[NV][8];
    bool vok[NV];
    load_weights<NV, WT>(p, slot, lr, wv, vok);

    double acc[NV][8];
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.0;

    const int64_t P = gridDim.x;
    const int64_t b = blockIdx.x;
    const int64_t rbeg = (b * p.rows) / P;
    const int64_t rend = ((b + 1) * p.rows) / P;
    const int64_t nit = (rend - rbeg + p.rpb - 1) / p.rpb;
    int buf = 0;
#pragma unroll 1
    for (int64_t it = 0; it < nit; ++it) {
        const int64_t r = rbeg + it * p.rpb + slot;
        const bool active = (slot < p.rpb) && (r < rend);
        bwd_one_row<NV, WT, false, WIDE, true>(p, r, active, slot, lr, wv, vok, acc, red, buf);
    }

    // Combine the row slots in slot order: acc(0) + acc(1) + ... (fixed).
    if (p.rpb > 1) {
        for (int s = 1; s < p.rpb; ++s) {
            __syncthreads();
            if (slot == s) {
#pragma unroll
                for (int k = 0; k < NV; ++k)
                    if (vok[k])
#pragma unroll
                        for (int e = 0; e < 8; ++e) comb[(lr + k * p.tpr) * kVec + e] = acc[k][e];
            }
            __syncthreads();
            if (slot == 0) {
#pragma unroll
                for (int k = 0; k < NV; ++k)
                    if (vok[k])
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[k][e] += comb[(lr + k * p.tpr) * kVec + e];
            }
        }
    }

    if constexpr (MODE == kModePartF64 || MODE == kModePartF32) {
        if (slot == 0) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                const int64_t col = (int64_t)(lr + k * p.tpr) * kVec;
                if constexpr (MODE == kModePartF64) {
                    double2* dst = reinterpret_cast<double2*>(static_cast<double*>(p.partial) + b * p.H + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = make_double2(acc[k][2 * e], acc[k][2 * e + 1]);
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.partial) + b * p.H + col);
                    dst[0] = make_float4((float)acc[k][0], (float)acc[k][1], (float)acc[k][2], (float)acc[k][3]);
                    dst[1] = make_float4((float)acc[k][4], (float)acc[k][5], (float)acc[k][6], (float)acc[k][7]);
                }
            }
        }
    } else if constexpr (MODE == kModeAtomic) {
        if (slot == 0) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                const int64_t col = (int64_t)(lr + k * p.tpr) * kVec;
#pragma unroll
                for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p.acc + col + e, acc[k][e]);
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

// Residual variant: identical except the row work adds dres (kept separate
// so the plain kernel carries no residual branches).
template <int NV, typename WT, bool WIDE, int MODE>
__global__ void __launch_bounds__(1024) k_bwd_row_res(BwdParams p) {
    extern __shared__ double lds_bwd[];
    const int tid = threadIdx.x;
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    double* comb = lds_bwd;
    float* red = reinterpret_cast<float*>(lds_bwd + (p.rpb > 1 ? p.H : 0));

    float wv[NV][8];
    bool vok[NV];
    load_weights<NV, WT>(p, slot, lr, wv, vok);
    double acc[NV][8];
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.0;

    const int64_t P = gridDim.x;
    const int64_t b = blockIdx.x;
    const int64_t rbeg = (b * p.rows) / P;
    const int64_t rend = ((b + 1) * p.rows) / P;
    const int64_t nit = (rend - rbeg + p.rpb - 1) / p.rpb;
    int buf = 0;
#pragma unroll 1
    for (int64_t it = 0; it < nit; ++it) {
        const int64_t r = rbeg + it * p.rpb + slot;
        const bool active = (slot < p.rpb) && (r < rend);
        bwd_one_row<NV, WT, true, WIDE, true>(p, r, active, slot, lr, wv, vok, acc, red, buf);
    }
    if (p.rpb > 1) {
        for (int s = 1; s < p.rpb; ++s) {
            __syncthreads();
            if (slot == s) {
#pragma unroll
                for (int k = 0; k < NV; ++k)
                    if (vok[k])
#pragma unroll
                        for (int e = 0; e < 8; ++e) comb[(lr + k * p.tpr) * kVec + e] = acc[k][e];
            }
            __syncthreads();
            if (slot == 0) {
#pragma unroll
                for (int k = 0; k < NV; ++k)
                    if (vok[k])
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[k][e] += comb[(lr + k * p.tpr) * kVec + e];
            }
        }
    }
    if constexpr (MODE == kModePartF64 || MODE == kModePartF32) {
        if (slot == 0) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                const int64_t col = (int64_t)(lr + k * p.tpr) * kVec;
                if constexpr (MODE == kModePartF64) {
                    double2* dst = reinterpret_cast<double2*>(static_cast<double*>(p.partial) + b * p.H + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = make_double2(acc[k][2 * e], acc[k][2 * e + 1]);
                } else {
                    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.partial) + b * p.H + col);
                    dst[0] = make_float4((float)acc[k][0], (float)acc[k][1], (float)acc[k][2], (float)acc[k][3]);
                    dst[1] = make_float4((float)acc[k][4], (float)acc[k][5], (float)acc[k][6], (float)acc[k][7]);
                }
            }
        }
    } else if constexpr (MODE == kModeAtomic) {
        if (slot == 0) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                if (!vok[k]) continue;
                const int64_t col = (int64_t)(lr + k * p.tpr) * kVec;
#pragma unroll
                for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p.acc + col + e, acc[k][e]);
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

// Fixed-order reduction of P partial rows: thread (chunk cc, slice s) sums
// partial rows s, s + S, s + 2S, ... of a 16-byte column chunk in increasing
// order; the S slice sums are then added in a fixed pairwise tree.
template <typename PT>
__global__ void __launch_bounds__(256) k_dw_reduce(const PT* __restrict__ part, int64_t P,
                                                   int32_t H, float* __restrict__ dw) {
    constexpr int CPC = 16 / sizeof(PT);  // columns per 16-byte chunk
    constexpr int CC = 16;                // chunks per block
    constexpr int S = 16;                 // slices
    __shared__ double sm[S][CC * CPC];
    const int cc = threadIdx.x % CC;
    const int s = threadIdx.x / CC;
    const int64_t col0 = ((int64_t)blockIdx.x * CC + cc) * CPC;
    double a[CPC];
#pragma unroll
    for (int e = 0; e < CPC; ++e) a[e] = 0.0;
    if (col0 < H) {
        for (int64_t q = s; q < P; q += S) {
            const PT* src = part + q * H + col0;
            if constexpr (CPC == 2) {
                double2 v = *reinterpret_cast<const double2*>(src);
                a[0] += v.x;
                a[1] += v.y;
            } else {
                float4 v = *reinterpret_cast<const float4*>(src);
                a[0] += (double)v.x;
                a[1] += (double)v.y;
                a[2] += (double)v.z;
                a[3] += (double)v.w;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < CPC; ++e) sm[s][cc * CPC + e] = a[e];
    __syncthreads();
#pragma unroll
    for (int half = S / 2; half >= 1; half >>= 1) {
        if (s < half) {
#pragma unroll
            for (int e = 0; e < CPC; ++e) sm[s][cc * CPC + e] += sm[s + half][cc * CPC + e];
        }
        __syncthreads();
    }
    if (s == 0 && col0 < H) {
#pragma unroll
        for (int e = 0; e < CPC; ++e) dw[col0 + e] = (float)sm[0][cc * CPC + e];
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
    // Row task.
    const int slot = tid / p.tpr;
    const int lr = tid - slot * p.tpr;
    float wv[NV][8];
    bool vok[NV];
    load_weights<NV, WT>(p, slot, lr, wv, vok);
    double acc[NV][8];
    float* red = reinterpret_cast<float*>(lds_small);
    int buf = 0;
    const int64_t rb = (int64_t)(blockIdx.x - p.ncol_blocks) * p.rpb;
    const int64_t r = rb + slot;
    const bool active = (slot < p.rpb) && (r < p.rows);
    if (p.tpr > 64)
        bwd_one_row<NV, WT, RES, true, false>(p, r, active, slot, lr, wv, vok, acc, red, buf);
    else
        bwd_one_row<NV, WT, RES, false, false>(p, r, active, slot, lr, wv, vok, acc, red, buf);
}

// Zero fill with vector stores (used for workspace initialisation; a kernel
// rather than a memset so that it can sit inside captured graphs).
__global__ void __launch_bounds__(256) k_fill_zero(uint4* p, int64_t n16, uint8_t* tail,
                                                   int64_t ntail) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = i0; i < n16; i += step) p[i] = make_uint4(0, 0, 0, 0);
    if (i0 < ntail) tail[i0] = 0;
}

// ----------------------------------------------------------------- launchers

template <int NV, typename WT, bool RES, bool WIDE>
static void launch_row_mode(const BwdParams& p, const Route& rt, size_t lds, hipStream_t s) {
    dim3 grid((unsigned)rt.r.grid), block((unsigned)rt.r.block_threads);
    if (rt.r.kind == RMSN_KIND_BWD_ROW_ATOMIC) {
        if constexpr (RES)
            hipLaunchKernelGGL((k_bwd_row_res<NV, WT, WIDE, kModeAtomic>), grid, block, lds, s, p);
        else
            hipLaunchKernelGGL((k_bwd_row<NV, WT, false, WIDE, kModeAtomic>), grid, block, lds, s, p);
    } else if (rt.r.partial_f64) {
        if constexpr (RES)
            hipLaunchKernelGGL((k_bwd_row_res<NV, WT, WIDE, kModePartF64>), grid, block, lds, s, p);
        else
            hipLaunchKernelGGL((k_bwd_row<NV, WT, false, WIDE, kModePartF64>), grid, block, lds, s, p);
    } else {
        if constexpr (RES)
            hipLaunchKernelGGL((k_bwd_row_res<NV, WT, WIDE, kModePartF32>), grid, block, lds, s, p);
        else
            hipLaunchKernelGGL((k_bwd_row<NV, WT, false, WIDE, kModePartF32>), grid, block, lds, s, p);
    }
}

template <int NV, typename WT, bool RES>
static int launch_row_nv(const BwdParams& p, const Route& rt, hipStream_t s) {
    const rmsn_route_t& r = rt.r;
    const bool wide = r.lanes_per_row > 64;
    size_t lds = (r.rows_per_block > 1 ? sizeof(double) * (size_t)p.H : 0);
    if (wide) lds += sizeof(float) * 2 * r.rows_per_block * (r.lanes_per_row / 64);
    if (wide)
        launch_row_mode<NV, WT, RES, true>(p, rt, lds, s);
    else
        launch_row_mode<NV, WT, RES, false>(p, rt, lds, s);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <typename WT, bool RES>
static int launch_row_wt(const BwdParams& p, const Route& rt, hipStream_t s) {
    switch (rt.r.vec_per_lane) {
        case 1: return launch_row_nv<1, WT, RES>(p, rt, s);
        case 2: return launch_row_nv<2, WT, RES>(p, rt, s);
        default: return RMSN_ERR_SHAPE;
    }
}

int launch_bwd_row(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
                   hipStream_t s) {
    if (wdt == RMSN_BF16)
        return residual ? launch_row_wt<uint16_t, true>(p, rt, s) : launch_row_wt<uint16_t, false>(p, rt, s);
    return residual ? launch_row_wt<float, true>(p, rt, s) : launch_row_wt<float, false>(p, rt, s);
}

int launch_dw_reduce(const BwdParams& p, const Route& rt, hipStream_t s) {
    dim3 grid((unsigned)rt.r.reduce_grid), block(256);
    if (rt.r.partial_f64)
        hipLaunchKernelGGL(k_dw_reduce<double>, grid, block, 0, s,
                           static_cast<const double*>(p.partial), (int64_t)rt.r.partials, p.H, p.dw);
    else
        hipLaunchKernelGGL(k_dw_reduce<float>, grid, block, 0, s,
                           static_cast<const float*>(p.partial), (int64_t)rt.r.partials, p.H, p.dw);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <int NV, typename WT, bool RES>
static int launch_small_t(const BwdParams& p, const Route& rt, hipStream_t s) {
    const rmsn_route_t& r = rt.r;
    const int vb = 256 / p.col_splits;
    size_t lds = sizeof(double) * (size_t)p.col_splits * vb * 8;
    const size_t lds_red = sizeof(float) * 2 * r.rows_per_block * (r.lanes_per_row > 64 ? r.lanes_per_row / 64 : 1);
    if (lds_red > lds) lds = lds_red;
    hipLaunchKernelGGL((k_bwd_small<NV, WT, RES>), dim3((unsigned)r.grid), dim3(256), lds, s, p);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

template <typename WT, bool RES>
static int launch_small_wt(const BwdParams& p, const Route& rt, hipStream_t s) {
    switch (rt.r.vec_per_lane) {
        case 1: return launch_small_t<1, WT, RES>(p, rt, s);
        case 2: return launch_small_t<2, WT, RES>(p, rt, s);
        case 4: return launch_small_t<4, WT, RES>(p, rt, s);
        case 8: return launch_small_t<8, WT, RES>(p, rt, s);
        default: return RMSN_ERR_SHAPE;
    }
}

int launch_bwd_small(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
                     hipStream_t s) {
    if (wdt == RMSN_BF16)
        return residual ? launch_small_wt<uint16_t, true>(p, rt, s) : launch_small_wt<uint16_t, false>(p, rt, s);
    return residual ? launch_small_wt<float, true>(p, rt, s) : launch_small_wt<float, false>(p, rt, s);
}

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
    if (bytes == 0) return RMSN_OK;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t ntail = (int64_t)(bytes % 16);
    int64_t blocks = (n16 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint4*>(ptr), n16, static_cast<uint8_t*>(ptr) + n16 * 16, ntail);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

}  // namespace rmsn
