// dw reduce, zero fill, and the weight-dtype dispatch of the launchers.
#include "rmsn_device.h"

namespace rmsn {

// Fixed-order reduction of P partial rows of W columns. A block owns CC * 16
// contiguous bytes of columns (CC chunks of 16 bytes) and S = blockDim/CC
// slices: thread (chunk c, slice s) sums partial rows s, s + S, s + 2S, ...
// in increasing order, four loads in flight at a time. The slice sums are
// then added in a fixed order: a butterfly over the slices each wave holds,
// then the waves in index order (one thread per column). Nothing depends on
// timing, so the result is bit-reproducible. Columns below `split` go to out0, the others to out1
// (LayerNorm's dgamma and dbeta share one partial row); split is a multiple
// of the chunk width.
template <typename PT, int CC>
__device__ __forceinline__ void dw_reduce_block(const PT* __restrict__ part, int64_t P, int32_t H,
                                                float* __restrict__ dw, float* __restrict__ out1,
                                                int32_t split, int64_t blk, double* sm_red) {
    constexpr int CPC = 16 / sizeof(PT);  // columns per 16-byte chunk
    constexpr int NCOL = CC * CPC;        // columns per block
    constexpr int NW = kReduceThreads / 64;
    constexpr int S = kReduceThreads / CC;
    const int cc = threadIdx.x % CC;
    const int s = threadIdx.x / CC;
    const int64_t col0 = (blk * CC + cc) * CPC;
    const bool col_ok = col0 < H;
    double a[CPC];
#pragma unroll
    for (int e = 0; e < CPC; ++e) a[e] = 0.0;
    if (col_ok) {
#pragma unroll 1
        for (int64_t q = s; q < P; q += 4 * (int64_t)S) {
            PT v[4][CPC];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t row = q + (int64_t)u * S;
#pragma unroll
                for (int e = 0; e < CPC; ++e) v[u][e] = PT(0);
                if (row < P) {
                    const PT* src = part + row * H + col0;
                    if constexpr (CPC == 2) {
                        double2 t = *reinterpret_cast<const double2*>(src);
                        v[u][0] = t.x;
                        v[u][1] = t.y;
                    } else {
                        float4 t = *reinterpret_cast<const float4*>(src);
                        v[u][0] = t.x;
                        v[u][1] = t.y;
                        v[u][2] = t.z;
                        v[u][3] = t.w;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < CPC; ++e) a[e] += (double)v[u][e];
        }
    }
    // butterfly over the wave's 64 / CC slices (the lane bits above the
    // chunk index), fixed pairing
#pragma unroll
    for (int e = 0; e < CPC; ++e) {
#pragma unroll
        for (int m = CC; m < 64; m <<= 1) a[e] += __shfl_xor(a[e], m, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) < CC) {
#pragma unroll
        for (int e = 0; e < CPC; ++e) sm_red[wave * NCOL + cc * CPC + e] = a[e];
    }
    __syncthreads();
    // chunks are whole columns of one side of split (H and split are
    // multiples of 8 columns), so the per-column tests match the chunk's
    if (threadIdx.x < NCOL) {
        const int c = threadIdx.x;
        const int64_t col = blk * NCOL + c;
        if (col < H) {
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < NW; ++w) t += sm_red[w * NCOL + c];
            float* dst = col < split ? dw + col : out1 + (col - split);
            *dst = (float)t;
        }
    }
}

template <typename PT, int CC>
__global__ void __launch_bounds__(kReduceThreads) k_dw_reduce(const PT* __restrict__ part, int64_t P,
                                                              int32_t H, float* __restrict__ dw,
                                                              float* __restrict__ out1, int32_t split) {
    __shared__ double sm_red[(kReduceThreads / 64) * CC * (16 / sizeof(PT))];
    dw_reduce_block<PT, CC>(part, P, H, dw, out1, split, (int64_t)blockIdx.x, sm_red);
}

// Several deferred reductions in one launch, all with partial rows of type
// PT: job k owns the blocks [block0_k, block0_{k+1}), and each of its blocks
// does exactly what block (blockIdx - block0_k) of k_dw_reduce does for that
// job alone, so every job's dw has the bits of the separate reduce.
template <typename PT>
__global__ void __launch_bounds__(kReduceThreads) k_dw_reduce_batch(DwJobs jobs) {
    __shared__ double sm_red[(kReduceThreads / 64) * kReduceChunks * (16 / sizeof(PT))];
    const int64_t b = blockIdx.x;
    // the block's job, read field by field in a uniform loop (no dynamic
    // index into the argument table)
    const void* part = nullptr;
    int64_t P = 0, block0 = 0;
    int32_t H = 0;
    float* dw = nullptr;
#pragma unroll
    for (int i = 0; i < kMaxBatchJobs; ++i) {
        if (i < jobs.n && b >= jobs.j[i].block0) {
            part = jobs.j[i].part;
            P = jobs.j[i].P;
            H = jobs.j[i].H;
            dw = jobs.j[i].dw;
            block0 = jobs.j[i].block0;
        }
    }
    // the job's pointers are uniform across the block: passed through
    // readfirstlane they reach the inlined body as plain values (inlining it
    // on the argument table's own pointers crashes this compiler's inliner)
    const uint64_t pb = (uint64_t)part, db = (uint64_t)dw;
    const PT* part_u = reinterpret_cast<const PT*>(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(pb >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pb));
    float* dw_u = reinterpret_cast<float*>(
        ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(db >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)db));
    dw_reduce_block<PT, kReduceChunks>(part_u, P, H, dw_u, nullptr, H, b - block0, sm_red);
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

int launch_col_reduce(const void* partial, const Route& rt, int32_t W, float* out0, float* out1,
                      int32_t split, hipStream_t s) {
    if (rt.r.reduce_threads != kReduceThreads) return RMSN_ERR_SHAPE;
    dim3 grid((unsigned)rt.r.reduce_grid), block((unsigned)kReduceThreads);
    const size_t lds = 0;
    // the route sizes the grid for 16-byte chunks per block (kReduceChunks)
    if (rt.r.partial_f64)
        launch_kernel((k_dw_reduce<double, kReduceChunks>), grid, block, lds, s,
                      static_cast<const double*>(partial), (int64_t)rt.r.partials, W, out0, out1,
                      split);
    else
        launch_kernel((k_dw_reduce<float, kReduceChunks>), grid, block, lds, s,
                      static_cast<const float*>(partial), (int64_t)rt.r.partials, W, out0, out1,
                      split);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

int launch_dw_reduce_batch(const DwJobs& jobs, int64_t blocks, hipStream_t s) {
    if (jobs.n < 1 || blocks < 1) return RMSN_OK;
    if (jobs.j[0].f64)
        launch_kernel(k_dw_reduce_batch<double>, dim3((unsigned)blocks), dim3((unsigned)kReduceThreads),
                      0, s, jobs);
    else
        launch_kernel(k_dw_reduce_batch<float>, dim3((unsigned)blocks), dim3((unsigned)kReduceThreads),
                      0, s, jobs);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

int launch_dw_reduce(const BwdParams& p, const Route& rt, hipStream_t s) {
    return launch_col_reduce(p.partial, rt, p.H, p.dw, nullptr, p.H, s);
}

int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
    if (bytes == 0) return RMSN_OK;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t ntail = (int64_t)(bytes % 16);
    int64_t blocks = (n16 + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    launch_kernel(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint4*>(ptr), n16, static_cast<uint8_t*>(ptr) + n16 * 16, ntail);
    return hipGetLastError() == hipSuccess ? RMSN_OK : RMSN_ERR_LAUNCH;
}

int launch_fwd(const FwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
               hipStream_t s) {
    return wdt == RMSN_BF16 ? launch_fwd_bf16w(p, rt, residual, s) : launch_fwd_f32w(p, rt, residual, s);
}

int launch_bwd_row(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, int form,
                   hipStream_t s) {
    if (bwd_row_comb_all(rt.r, p.H))
        return wdt == RMSN_BF16 ? launch_bwd_row_bf16w_ca(p, rt, form, s)
                                : launch_bwd_row_f32w_ca(p, rt, form, s);
    return wdt == RMSN_BF16 ? launch_bwd_row_bf16w(p, rt, form, s)
                            : launch_bwd_row_f32w(p, rt, form, s);
}

int launch_bwd_small(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
                     hipStream_t s) {
    return wdt == RMSN_BF16 ? launch_bwd_small_bf16w(p, rt, residual, s)
                            : launch_bwd_small_f32w(p, rt, residual, s);
}

int launch_ln_fwd(const LnFwdParams& p, const Route& rt, rmsn_dtype_t wdt, hipStream_t s) {
    return wdt == RMSN_BF16 ? launch_ln_fwd_bf16w(p, rt, s) : launch_ln_fwd_f32w(p, rt, s);
}

int launch_ln_bwd_row(const LnBwdParams& p, const Route& rt, rmsn_dtype_t wdt, hipStream_t s) {
    return wdt == RMSN_BF16 ? launch_ln_bwd_row_bf16w(p, rt, s) : launch_ln_bwd_row_f32w(p, rt, s);
}

}  // namespace rmsn
