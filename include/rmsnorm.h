/*
 * rmsnorm.h — C ABI of the MI355X (gfx950) RMSNorm-for-training library.
 *
 * The operation (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a
 * dw-accuracy backward routes", opening description):
 *   forward   x[T, H] BF16, w[H] BF16 or FP32  ->  y[T, H] BF16, rstd[T] FP32
 *             rstd_t = 1/sqrt(mean_j(x_tj^2) + eps),  y_tj = x_tj * rstd_t * w_j
 *   backward  dy[T, H] BF16                     ->  dx[T, H] BF16, dw[H] FP32
 *             xhat = x*rstd, c_t = mean_j(dy_tj * w_j * xhat_tj),
 *             dx_tj = rstd_t * (dy_tj * w_j - xhat_tj * c_t),
 *             dw_j = sum_t dy_tj * xhat_tj
 * Both backward modes (deterministic = 1 or 0) run after one and the same
 * forward; what may differ between them is only the reduction of the dw
 * column sum over T. Forms (same page, opening description and "Key"): rows
 * of [T, H] with a weight in BF16 or FP32; a residual add fused ahead of the
 * norm, whose rounded BF16 sum is both written out and normalised; and
 * per-head views [T, heads, H], strided or contiguous, all heads sharing one
 * w[H], with dw summed over T and over the heads. Output dtypes ("Workload"
 * paragraph): y, dx and the residual sum BF16; rstd and dw FP32.
 *
 * Conventions for every entry point:
 * - All tensor pointers are DEVICE pointers on the current HIP device; the
 *   caller owns every buffer. The library never allocates, frees or
 *   synchronises; each call enqueues kernels on `stream` and returns.
 * - BF16 tensors are raw 16-bit patterns (void*). Sizes and strides are in
 *   ELEMENTS (int64_t).
 * - A view describes rows = T * heads rows of H contiguous elements; row
 *   (t, head) starts at t * stride_t + head * stride_h. rstd is always a
 *   contiguous FP32 array of T * heads values, index t * heads + head.
 * - Requirements: H a positive multiple of 8 and at most 16384; T >= 0 and
 *   heads >= 1 (rows == T*heads == 0: the forward does nothing, the backward
 *   writes dw = 0); rows < 2^31; BF16 tensor base pointers
 *   and strides 16-byte aligned (strides multiples of 8 elements); weight
 *   pointers 16-byte aligned; rstd/dw 4-byte aligned; eps finite and >= 0.
 * - Outputs are written in full (dw is overwritten, never accumulated into).
 *   An output may alias an input only exactly (same pointer, same view), and
 *   only in the forward: y over x, or h over x in the residual form. Any
 *   other overlap of the byte spans of an output with another tensor, and
 *   any output view whose rows overlap each other, is RMSN_ERR_ALIAS.
 * - Errors are returned as negative status codes before anything is
 *   enqueued (RMSN_ERR_LAUNCH is reported after a failed launch).
 *   rmsnorm_status_string() names them. Nothing is printed.
 * - Workspace: the backward entry points take a device workspace of at
 *   least rmsnorm_bwd_workspace_bytes(...) bytes, 256-byte aligned, as
 *   scratch: it needs no initialisation and its contents after a call are
 *   unspecified. Two calls that may run concurrently must not share one.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight dtype. The two outer enumerators are never valid; they make every
 * int value a value of this type, so that a caller may pass any int (a C
 * caller, or a binding) and get RMSN_ERR_DTYPE back for unsupported ones
 * rather than undefined behaviour in the C++ implementation. */
typedef enum {
    RMSN_DTYPE_INVALID_ = -1,
    RMSN_BF16 = 0,
    RMSN_F32 = 1,
    RMSN_DTYPE_MAX_ = 0x7fffffff
} rmsn_dtype_t;

enum {
    RMSN_OK = 0,
    RMSN_ERR_NULL = -1,      /* a required pointer is NULL */
    RMSN_ERR_DTYPE = -2,     /* weight dtype is neither RMSN_BF16 nor RMSN_F32 */
    RMSN_ERR_SHAPE = -3,     /* H not in 8..16384 step 8, negative T/heads, views disagree */
    RMSN_ERR_ALIGN = -4,     /* pointer or stride misaligned */
    RMSN_ERR_WORKSPACE = -5, /* workspace NULL, misaligned or smaller than required */
    RMSN_ERR_OVERFLOW = -6,  /* element offsets or byte sizes overflow int64 */
    RMSN_ERR_ALIAS = -7,     /* an output overlaps another tensor (not exact in-place) */
    RMSN_ERR_LAUNCH = -8,    /* a kernel launch failed (hipGetLastError) */
    RMSN_ERR_EPS = -9,       /* eps negative, NaN or infinite */
    RMSN_ERR_SCRATCH = -10   /* the no-alloc entry point's fixed scratch is too small
                                (or its address could not be looked up) */
};

typedef struct {
    int64_t T;        /* tokens */
    int64_t heads;    /* rows per token (1 for plain [T, H]) */
    int64_t H;        /* normalised width */
    int64_t stride_t; /* elements between tokens */
    int64_t stride_h; /* elements between heads of one token */
} rmsn_view_t;

/* ---------------------------------------------------------------- forward */

/* Plain forward over contiguous x[T, H] -> y[T, H], rstd[T].
 * (flashinfer PR #8827 description: forward returns y BF16, rstd FP32.) */
int rmsnorm_fwd(const void* x, const void* w, rmsn_dtype_t w_dtype, float eps,
                void* y, float* rstd, int64_t T, int64_t H, hipStream_t stream);

/* Forward over arbitrary views (per-head [T, heads, H], strided or not).
 * x and y views must agree on T, heads and H; rstd has T*heads entries.
 * (Same page, opening description: per-head views, 24 heads of 256 in a
 * strided buffer or 4 heads of 256 contiguous, that share one weight.) */
int rmsnorm_fwd_strided(const void* x, rmsn_view_t xv, const void* w,
                        rmsn_dtype_t w_dtype, float eps, void* y, rmsn_view_t yv,
                        float* rstd, hipStream_t stream);

/* Fused residual forward on contiguous [T, H]: h = BF16(x + r) is written,
 * then y, rstd = RMSNorm(h). (Same page, "Key": the fused residual form
 * rounds the sum of the two BF16 inputs once to BF16.) */
int rmsnorm_residual_fwd(const void* x, const void* r, const void* w,
                         rmsn_dtype_t w_dtype, float eps, void* h, void* y,
                         float* rstd, int64_t T, int64_t H, hipStream_t stream);

/* The same over views: x, r, h and y each have their own view, and the four
 * agree on T, heads and H; rstd has T*heads entries. h may be x itself (same
 * pointer and view); no other output may overlap an input. (Same page,
 * opening description: the residual form, and the per-head views that share
 * one weight.) */
int rmsnorm_residual_fwd_strided(const void* x, rmsn_view_t xv, const void* r, rmsn_view_t rv,
                                 const void* w, rmsn_dtype_t w_dtype, float eps, void* h,
                                 rmsn_view_t hv, void* y, rmsn_view_t yv, float* rstd,
                                 hipStream_t stream);

/* --------------------------------------------------------------- backward */

/* Bytes of workspace the backward needs for this shape and mode, enough for
 * every backward entry point below (0 when none of their kernels needs any;
 * callers may still pass a larger buffer). */
size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype,
                                   int deterministic);

/* Zero-fill a device buffer with a kernel on `stream` (no memset node, so it
 * is safe inside graph capture). Not needed before the backward calls. */
int rmsnorm_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Plain backward on contiguous [T, H]. rstd is the forward's FP32 output.
 * deterministic != 0: dw is bit-identical run to run for the same inputs and
 * does not depend on the device's CU count. deterministic == 0 allows an
 * order of the dw reduction that may vary between runs; this library's
 * route table currently serves both values with the same fixed-order
 * kernels (an atomic reduction measured slower on this part), so today both
 * modes return the same dw bits. dx is bit-identical between the two modes.
 * (Same page, opening description: the two modes run one forward and differ
 * in the backward only; "Changed windows by reason": every dw element must
 * lie within 1e-4 absolute plus 1e-4 relative of the FP64 result.) */
int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* w,
                rmsn_dtype_t w_dtype, int deterministic, void* dx, float* dw,
                int64_t T, int64_t H, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* Backward over views: dy, x and dx views agree on T, heads and H; dw[H]
 * sums over T and heads. dx may be a strided view into a wider buffer; only
 * the elements the view covers are written. Modes and workspace as in
 * rmsnorm_bwd. (Same page, opening description: per-head views with 24
 * heads of 256 in a strided buffer and 4 heads of 256 contiguous, both
 * modes, one shared w[256].) */
int rmsnorm_bwd_strided(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                        const float* rstd, const void* w, rmsn_dtype_t w_dtype,
                        int deterministic, void* dx, rmsn_view_t dxv, float* dw,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate (code under graph capture, tight
 * serving loops, harnesses that forbid allocation): rmsnorm_bwd_strided
 * with no workspace argument. The dw partial rows go to a fixed device array
 * of 32 MiB inside the library, enough for every shape at the default
 * routes; a problem needing more returns RMSN_ERR_SCRATCH before anything is
 * enqueued. Each device holds its own array until the process ends. All
 * calls on one device share that array, so calls that may overlap on one
 * device (other streams, other host threads) race and must be serialised
 * by the caller. Everything else as rmsnorm_bwd_strided; the results are
 * bit-identical to it. Makes no allocation. */
int rmsnorm_bwd_strided_noalloc(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                                const float* rstd, const void* w, rmsn_dtype_t w_dtype,
                                int deterministic, void* dx, rmsn_view_t dxv, float* dw,
                                hipStream_t stream);

/* Backward that takes no rstd: each row's rstd is recomputed from x inside
 * the backward kernel, while the row is in registers, with the forward's own
 * arithmetic (FP32 sums of squares over 8-element groups, added in FP64,
 * 1/sqrt(mean + eps) in FP64 rounded once to FP32). For activation
 * recompute: the pages time a checkpointed training step as forward,
 * forward recompute, backward ("2xfwd+bwd", flashinfer PR #8827 "Key"); a
 * caller that kept x and needs no second y can replace the recompute
 * forward and the backward with this one call, saving the recompute's
 * read of x and write of y. The recomputed rstd equals the forward's
 * whenever the FP64 sum of a row's FP32 group sums is exact in both
 * summation orders, which holds unless those group sums span more than
 * 2^(29 - log2(H/8)) in magnitude; otherwise it can differ in the last bit.
 * Views, outputs, modes and workspace as in rmsnorm_bwd_strided; eps as
 * in the forward (RMSN_ERR_EPS if negative or not finite). At every T this
 * runs the row kernel (no small-T column-task kernel). */
int rmsnorm_bwd_recompute(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                          const void* w, rmsn_dtype_t w_dtype, float eps, int deterministic,
                          void* dx, rmsn_view_t dxv, float* dw, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Residual backward on contiguous [T, H]: h is the forward's BF16 h_new;
 * dres (nullable) is the gradient arriving at h_new from the residual
 * stream. Returns dh = BF16(dres + dRMSNorm/dh) — the one "combined grad"
 * that flows to both x and r — and dw. (Same page, "Key": fused residual
 * add, combined grad.) */
int rmsnorm_residual_bwd(const void* dy, const void* h, const void* dres,
                         const float* rstd, const void* w, rmsn_dtype_t w_dtype,
                         int deterministic, void* dh, float* dw, int64_t T, int64_t H,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same over views: dy, h, dres (when not NULL) and dh each have their
 * own view, agreeing on T, heads and H; dresv is ignored when dres is NULL;
 * rstd has T*heads entries; dw sums over T and heads. Modes and workspace as
 * in rmsnorm_bwd. (Same page, opening description and "Key".) */
int rmsnorm_residual_bwd_strided(const void* dy, rmsn_view_t dyv, const void* h, rmsn_view_t hv,
                                 const void* dres, rmsn_view_t dresv, const float* rstd,
                                 const void* w, rmsn_dtype_t w_dtype, int deterministic, void* dh,
                                 rmsn_view_t dhv, float* dw, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- deferred dw reduction
 *
 * The deterministic backward is a row kernel that leaves per-block partial
 * rows of dw, then a fixed-order reduce of those rows into dw (the pages'
 * "chunk-partials pair": flashinfer PR "fix(cake_rmsnorm): sm_100a and
 * sm_107a dw-accuracy backward routes", "Changed windows by reason"). A
 * training step needs dw only at the optimizer, after the whole backward, so
 * these calls split the pair: each norm's backward leaves its partial rows in
 * a caller buffer, and one rmsnorm_dw_reduce_batch call later reduces the
 * partials of many norms in one launch. Each job's dw then has exactly the
 * bits rmsnorm_bwd_strided (or rmsnorm_residual_bwd_strided) returns in
 * deterministic mode for the same call; dx (dh) is the same as there too.
 */

/* Bytes of the partial-rows buffer a deferred backward of `rows` rows of H
 * needs (0 for an invalid shape). The layout is a function of (rows, H) and
 * the route table: keep route overrides unchanged between the backward and
 * its reduce. */
size_t rmsnorm_bwd_partials_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype);

/* rmsnorm_bwd_strided (deterministic) without its dw reduction: dx is
 * written, and the dw partial rows are left in `partials` (256-byte
 * aligned, at least rmsnorm_bwd_partials_bytes bytes, owned by the caller
 * until the reduce has run). */
int rmsnorm_bwd_strided_partials(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                                 const float* rstd, const void* w, rmsn_dtype_t w_dtype, void* dx,
                                 rmsn_view_t dxv, void* partials, size_t partials_bytes,
                                 hipStream_t stream);

/* rmsnorm_residual_bwd_strided (deterministic) without its dw reduction; the
 * partials as above. */
int rmsnorm_residual_bwd_strided_partials(const void* dy, rmsn_view_t dyv, const void* h,
                                          rmsn_view_t hv, const void* dres, rmsn_view_t dresv,
                                          const float* rstd, const void* w, rmsn_dtype_t w_dtype,
                                          void* dh, rmsn_view_t dhv, void* partials,
                                          size_t partials_bytes, hipStream_t stream);

/* One deferred reduction: the partial rows of one earlier call (rows = its
 * T*heads, H and w_dtype as passed to it) and the dw [H] FP32 to write. */
typedef struct {
    const void* partials;
    size_t partials_bytes;
    int64_t rows;
    int64_t H;
    rmsn_dtype_t w_dtype;
    float* dw;
} rmsn_dw_job_t;

/* Reduce n deferred jobs into their dw on `stream`, in as few launches as
 * the job table allows (one per 32 jobs of each partial precision). Every
 * job is checked before anything is enqueued: a buffer smaller than its
 * layout needs is RMSN_ERR_WORKSPACE, a dw overlapping any job's partials or
 * another dw is RMSN_ERR_ALIAS. n == 0 does nothing. */
int rmsnorm_dw_reduce_batch(const rmsn_dw_job_t* jobs, int n, hipStream_t stream);

/* -------------------------------------------------------------- LayerNorm
 *
 * The adjacent normalisation of the same training stacks (ROCm
 * TransformerEngine PR "Microbenchmarking and CI performance regression
 * test", benchmark_normalization table: RMSNorm and LayerNorm forward and
 * backward, BF16, on MI355). Contiguous x[T, H] BF16; gamma and beta [H] BF16
 * or FP32 (the same dtype):
 *   forward   mean_t = (1/H) sum_j x_tj, var_t = (1/H) sum_j (x_tj - mean_t)^2,
 *             rstd_t = 1/sqrt(var_t + eps),
 *             y_tj = BF16((x_tj - mean_t) * rstd_t * gamma_j + beta_j)
 *   backward  xhat = (x - mean) * rstd, g = dy * gamma,
 *             dx = BF16(rstd * (g - mean_j(g) - xhat * mean_j(g * xhat))),
 *             dgamma_j = sum_t dy_tj * xhat_tj,  dbeta_j = sum_t dy_tj
 * Conventions, modes and errors as for RMSNorm above (deterministic != 0:
 * dgamma and dbeta bit-identical run to run and across devices).
 */

/* Forward: y [T, H] BF16 (may be x itself, exactly), mean and rstd [T]
 * FP32. beta may be NULL (no bias). */
int layernorm_fwd(const void* x, const void* gamma, const void* beta, rmsn_dtype_t w_dtype,
                  float eps, void* y, float* mean, float* rstd, int64_t T, int64_t H,
                  hipStream_t stream);

/* Workspace bytes layernorm_bwd needs (its [P, 2H] partial sums). */
size_t layernorm_bwd_workspace_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype,
                                     int deterministic);

/* Backward at the forward's mean and rstd: dx [T, H] BF16, dgamma and dbeta
 * [H] FP32 (overwritten; zero when T == 0). The workspace is scratch, as
 * for rmsnorm_bwd. */
int layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                  const void* gamma, rmsn_dtype_t w_dtype, int deterministic, void* dx,
                  float* dgamma, float* dbeta, int64_t T, int64_t H, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------ diagnostics */

/* Static description of an error code (never NULL). */
const char* rmsnorm_status_string(int status);

/* Kernel kinds a route can name. */
enum {
    RMSN_KIND_FWD_ROW = 1,      /* one-pass row forward */
    RMSN_KIND_BWD_ROW_DET = 2,  /* row backward + per-block dw partials, then fixed-order reduce */
    RMSN_KIND_BWD_ROW_ATOMIC = 3, /* row backward + FP64 atomic dw, last block finalises */
    RMSN_KIND_BWD_COLTASK = 4   /* small T: fixed column tasks for dw + row tasks for dx */
};

typedef struct {
    int kind;            /* RMSN_KIND_* */
    int vec_per_lane;    /* 16-byte vectors each lane owns per row */
    int lanes_per_row;   /* threads that share one row */
    int rows_per_block;  /* row groups in a block */
    int unroll;          /* rows a row group holds per iteration */
    int block_threads;
    int partial_f64;     /* dw partials in FP64 (1) or FP32 (0) */
    int reduce_threads;  /* block size of the dw reduce kernel */
    int64_t grid;        /* blocks of the main kernel */
    int64_t partials;    /* dw partial rows written (0 if none) */
    int64_t reduce_grid; /* blocks of the dw reduce (column-task blocks for small T) */
    int stream_loads;    /* row kernels' non-temporal loads, a function of the shape:
                            backward 1 dy/dres, 2 every input; forward 2 x and r
                            (residual form only); 0 none */
} rmsn_route_t;

/* The route table: which kernel and launch shape serve this problem.
 * op: 0 forward, 1 backward, 2 LayerNorm forward, 3 LayerNorm backward.
 * form (ops 0 and 1; ignored otherwise): 0 plain (rmsnorm_fwd*, rmsnorm_bwd,
 * rmsnorm_bwd_strided), 1 residual (rmsnorm_residual_fwd/bwd), 2 recompute
 * (rmsnorm_bwd_recompute).
 * Pure host function; needs no GPU.
 * Returns RMSN_OK or RMSN_ERR_SHAPE / RMSN_ERR_DTYPE / RMSN_ERR_NULL. */
int rmsnorm_route_query(int op, int64_t rows, int64_t H, rmsn_dtype_t w_dtype,
                        int deterministic, int form, rmsn_route_t* out);

/* Launch-shape knobs for benchmarks and tuning sweeps (not part of the
 * method). A zero field keeps the table's choice. The route is still derived
 * and checked by the same code, so a knob the kernels cannot honour makes
 * the next call of that op fail with RMSN_ERR_SHAPE instead of launching.
 * Overriding the backward changes the deterministic partition, hence the dw
 * bits (they stay reproducible for a fixed setting). The small-T column-task
 * route is not affected. op as for rmsnorm_route_query. Process-wide, and
 * not synchronised: set it while no other host thread is calling the
 * library. NULL clears. */
typedef struct {
    int vec_per_lane;   /* 1, 2 or 4 (the backwards: 4 only with unroll 1) */
    int unroll;         /* 1, 2, 4 or 8, with vec_per_lane * unroll <= 8 (RMSNorm
                           backward <= 4; LayerNorm backward: unroll <= 2) */
    int rows_per_block; /* row groups per block. Block size <= 256 threads when a
                           row fits in one wave, else <= 1024, and <= 512 once
                           vec_per_lane * unroll >= 4 (the backwards: >= 2) */
    int blocks_per_cu;  /* grid cap = 256 * blocks_per_cu */
    int partial_f64;    /* backward: 1 FP64 partials, 2 FP32 partials */
    int kind;           /* backward: RMSN_KIND_BWD_ROW_DET or RMSN_KIND_BWD_ROW_ATOMIC */
    int stream_loads;   /* 1 + the stream_loads level to force (0 keeps the route's) */
} rmsn_route_knobs_t;
int rmsnorm_route_override(int op, const rmsn_route_knobs_t* knobs);

/* Per-kernel timing with HIP events on the caller's stream (for benchmarks).
 * While enabled, every kernel the library launches is bracketed by two
 * events; rmsnorm_timing_read waits for them and returns, per kernel kind
 * (index 0..7, see RMSN_TIMER_*), the number of launches and their summed
 * duration in milliseconds, then clears the counters. Not thread-safe;
 * off by default. */
enum {
    RMSN_TIMER_FWD = 0,
    RMSN_TIMER_BWD_ROW = 1,
    RMSN_TIMER_DW_REDUCE = 2,
    RMSN_TIMER_BWD_SMALL = 3,
    RMSN_TIMER_INIT = 4,
    RMSN_TIMER_COUNT = 8
};
int rmsnorm_timing_enable(int enable);
int rmsnorm_timing_read(int64_t* launches, double* total_ms, int n);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
