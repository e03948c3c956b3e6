// Internal declarations shared by the C-ABI layer and the kernel launchers.
// Host-visible only: parameter blocks passed by value to the kernels, and
// the launcher entry points each kernel file provides.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rmsnorm.h"

namespace rmsn {

// Widths the kernels are compiled for: vectors of 8 BF16 (16 bytes) per lane.
constexpr int kVec = 8;
constexpr int64_t kMaxH = 16384;
// The partition of rows into dw partials is derived from this fixed CU count,
// never from the device, so deterministic dw bits do not depend on the part.
constexpr int kPartitionCUs = 256;
// 16-byte column chunks per block of the dw column reduce (128 bytes of
// columns per block; 4 and 16 chunks measured slower at 4096 x 4096 and
// 32768 x 4 x 256).
constexpr int kReduceChunks = 8;
// Threads per block of the dw reduce (16 waves: 128 slices of the partial
// rows, one round of loads up to P = 512).
constexpr int kReduceThreads = 1024;

// Backward forms: plain rows, fused residual (h, optional dres), or plain
// rows with rstd recomputed from x inside the backward.
enum { kFormPlain = 0, kFormResidual = 1, kFormRecompute = 2 };

// Addressing of one tensor: row r = (t, head) starts at t*st_t + head*st_h.
struct RowAddr {
    int64_t st_t;
    int64_t st_h;
};

struct FwdParams {
    const uint16_t* x;
    const uint16_t* r;      // residual input (residual form) or null
    uint16_t* h;            // residual output h = BF16(x + r) or null
    uint16_t* y;
    float* rstd;
    const void* w;
    RowAddr ax, ar, ah, ay;
    int64_t rows;
    int32_t heads;
    int32_t H;
    int32_t nvec;           // H / 8
    int32_t tpr;            // lanes per row
    int32_t rpb;            // row slots per block
    float eps;
};

struct BwdParams {
    const uint16_t* dy;
    const uint16_t* x;      // x, or h in the residual form
    const uint16_t* dres;   // residual-stream gradient or null
    const float* rstd;
    const void* w;
    uint16_t* dx;
    float* dw;              // written by the finalising kernel/block
    void* partial;          // [P, H] FP32 or FP64 partials (deterministic route)
    double* acc;            // [H] FP64 accumulator (atomic route)
    unsigned int* ticket;   // block counter (atomic route)
    RowAddr ady, ax, ares, adx;
    int64_t rows;
    int32_t heads;
    int32_t H;
    int32_t nvec;
    int32_t tpr;
    int32_t rpb;
    int32_t ncol_blocks;    // column-task blocks (small-T kernel)
    int32_t col_splits;     // row splits per column task (small-T kernel)
    float eps;              // recompute form only
};

// One deferred dw reduction of a batch: the partial rows an earlier
// backward left (P rows of H, FP64 if f64 else FP32), its dw, and the first
// block of the batched launch that works on it.
struct DwJob {
    const void* part;
    int64_t P;
    int32_t H;
    int32_t f64;
    float* dw;
    int64_t block0;
};
// Jobs per batched launch (the table travels in the kernel arguments).
constexpr int kMaxBatchJobs = 32;
struct DwJobs {
    int32_t n;
    DwJob j[kMaxBatchJobs];
};

// LayerNorm (contiguous [rows, H]).
struct LnFwdParams {
    const uint16_t* x;
    uint16_t* y;
    float* mean;
    float* rstd;
    const void* gamma;
    const void* beta;       // may be null: zero bias
    int64_t rows;
    int32_t H;
    int32_t nvec;
    int32_t tpr;
    int32_t rpb;
    float eps;
};

struct LnBwdParams {
    const uint16_t* dy;
    const uint16_t* x;
    const float* mean;
    const float* rstd;
    const void* gamma;
    uint16_t* dx;
    void* partial;          // [P, 2H] FP32 or FP64: dgamma sums, then dbeta sums
    int64_t rows;
    int32_t H;
    int32_t nvec;
    int32_t tpr;
    int32_t rpb;
};

struct Route {
    rmsn_route_t r;
    size_t workspace;       // bytes needed
};

// Route table (route.cpp). op 0 fwd, 1 bwd, 2 LayerNorm fwd, 3 LayerNorm
// bwd; form kForm* (RMSNorm backward).
int route(int op, int64_t rows, int64_t H, rmsn_dtype_t wdt, int det, int form, Route* out);
// Tuning override of the route table (NULL clears).
int set_route_knobs(int op, const rmsn_route_knobs_t* knobs);

// Launchers (one per kernel file). They launch on `s` and return
// hipGetLastError() mapped to an RMSN status.
int launch_fwd(const FwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
               hipStream_t s);
int launch_bwd_row(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, int form,
                   hipStream_t s);
int launch_dw_reduce(const BwdParams& p, const Route& rt, hipStream_t s);
int launch_dw_reduce_batch(const DwJobs& jobs, int64_t blocks, hipStream_t s);
// Column reduce of rt.partials partial rows of W columns: columns < split go
// to out0, the rest to out1.
int launch_col_reduce(const void* partial, const Route& rt, int32_t W, float* out0, float* out1,
                      int32_t split, hipStream_t s);
int launch_ln_fwd(const LnFwdParams& p, const Route& rt, rmsn_dtype_t wdt, hipStream_t s);
int launch_ln_bwd_row(const LnBwdParams& p, const Route& rt, rmsn_dtype_t wdt, hipStream_t s);
int launch_ln_fwd_bf16w(const LnFwdParams& p, const Route& rt, hipStream_t s);
int launch_ln_fwd_f32w(const LnFwdParams& p, const Route& rt, hipStream_t s);
int launch_ln_bwd_row_bf16w(const LnBwdParams& p, const Route& rt, hipStream_t s);
int launch_ln_bwd_row_f32w(const LnBwdParams& p, const Route& rt, hipStream_t s);
int launch_bwd_small(const BwdParams& p, const Route& rt, rmsn_dtype_t wdt, bool residual,
                     hipStream_t s);
int launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
// Per weight dtype (one translation unit each, compiled in parallel).
int launch_fwd_bf16w(const FwdParams& p, const Route& rt, bool residual, hipStream_t s);
int launch_fwd_f32w(const FwdParams& p, const Route& rt, bool residual, hipStream_t s);
int launch_bwd_row_bf16w(const BwdParams& p, const Route& rt, int form, hipStream_t s);
int launch_bwd_row_f32w(const BwdParams& p, const Route& rt, int form, hipStream_t s);
// The same with the one-step slot combine (bwd_row_comb_all true).
int launch_bwd_row_bf16w_ca(const BwdParams& p, const Route& rt, int form, hipStream_t s);
int launch_bwd_row_f32w_ca(const BwdParams& p, const Route& rt, int form, hipStream_t s);
int launch_bwd_small_bf16w(const BwdParams& p, const Route& rt, bool residual, hipStream_t s);
int launch_bwd_small_f32w(const BwdParams& p, const Route& rt, bool residual, hipStream_t s);

// The backward row kernel combines its row slots' dw sums in one step
// (every slot's sums in LDS at once, [rpb, H] doubles, then every thread
// folds whole columns in slot order) when there are at least four slots and
// the sums fit in kCombAllLds; otherwise slot by slot through an [H] area.
// Both add in the same order. With two slots the serial form is one round
// and measured faster (4096 x 4096: 35.9 against 36.2 us per step); with
// eight it is seven rounds (32768 x 4 x 256: the one-step form -2.6 %).
constexpr size_t kCombAllLds = 64 * 1024;

inline bool bwd_row_comb_all(const rmsn_route_t& r, int H) {
    return r.rows_per_block >= 4 && r.kind == RMSN_KIND_BWD_ROW_DET &&
           sizeof(double) * (size_t)r.rows_per_block * (size_t)H <= kCombAllLds;
}

// Kernel timing hooks (api.cpp). timer_begin names the kernel kind the API
// is about to launch; when timing is enabled, the next launch takes a pair
// of events that the dispatch itself records (no separate marker packets).
void timer_begin(int kind, hipStream_t s);
void timer_end(int kind, hipStream_t s);
bool timer_take(hipEvent_t* start, hipEvent_t* stop);

template <typename K, typename... Args>
inline void launch_kernel(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (timer_take(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

}  // namespace rmsn
