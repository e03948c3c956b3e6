// Route table: which kernel and launch shape serve (op, rows, H, weight
// dtype, mode, form). Host-only and deterministic: a function of its
// arguments alone (never of the device), so the deterministic backward's
// row partition — and with it the dw bits — is fixed by the shape.
//
// The pages pick among kernel kinds by windows of T per (GPU, H, weight
// dtype) (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
// backward routes", "Changed windows by reason"). The kinds kept here are
// the ones that still hold on gfx950: a column-task kernel for small T
// ("the fixed-claim column-task kernel runs T 1 to 64"), and a row kernel
// with per-block dw partials plus a reduce (the "chunk-partials pair") or
// with atomics for the non-deterministic mode. No dw-accuracy cut is needed
// above that: FP64 dw accumulation keeps every shape inside the budget.
#include <string.h>

#include "rmsn_internal.h"

namespace rmsn {

namespace {

// Rows at or below this use the column-task kernel (both modes).
constexpr int64_t kSmallRows = 64;
// Deterministic partials are stored in FP32 up to this many rows, FP64 above
// (the FP32 rounding of each partial adds ~3e-8 * sqrt(T) absolute error).
constexpr int64_t kPartialF32MaxRows = 8192;
// Threads per CU the launch shapes aim to fill.
constexpr int kThreadsPerCU = 2048;
constexpr int kBwdThreadsPerCU = 1024;

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Lanes per row for `nvec` 16-byte vectors at `nv` vectors per lane: a power
// of two up to one wave, else a whole number of waves.
int lanes_per_row(int nvec, int nv) {
    const int need = ceil_div(nvec, nv);
    if (need <= 64) {
        int t = 1;
        while (t < need) t <<= 1;
        return t;
    }
    return ceil_div(need, 64) * 64;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

int route(int op, int64_t rows, int64_t H, rmsn_dtype_t wdt, int det, int residual,
          Route* out) {
    if (!out) return RMSN_ERR_NULL;
    memset(out, 0, sizeof(*out));
    if (wdt != RMSN_BF16 && wdt != RMSN_F32) return RMSN_ERR_DTYPE;
    if (H < kVec || H > kMaxH || H % kVec != 0 || rows < 0 || rows > INT32_MAX)
        return RMSN_ERR_SHAPE;
    if (op != 0 && op != 1) return RMSN_ERR_SHAPE;
    (void)residual;
    const int nvec = (int)(H / kVec);
    rmsn_route_t& r = out->r;

    if (op == 0) {
        // One-pass row forward; up to 1024 lanes per row.
        const int nv = nvec <= 1024 ? 1 : 2;
        const int tpr = lanes_per_row(nvec, nv);
        const int rpb = tpr <= 256 ? 256 / tpr : 1;
        r.kind = RMSN_KIND_FWD_ROW;
        r.vec_per_lane = nv;
        r.lanes_per_row = tpr;
        r.rows_per_block = rpb;
        r.block_threads = tpr * rpb;
        const int64_t cap = (int64_t)kPartitionCUs * (kThreadsPerCU / r.block_threads);
        int64_t g = ceil_div(rows, rpb);
        r.grid = g < cap ? g : cap;
        if (r.grid < 1) r.grid = 1;
        return RMSN_OK;
    }

    if (rows <= kSmallRows) {
        // Column tasks for dw + row tasks for dx in one launch of 256 threads.
        const int nv = nvec <= 256 ? 1 : (nvec <= 512 ? 2 : (nvec <= 1024 ? 4 : 8));
        const int tpr = lanes_per_row(nvec, nv);
        const int rpb = tpr <= 256 ? 256 / tpr : 1;
        const int splits = 8;
        const int vb = 256 / splits;
        r.kind = RMSN_KIND_BWD_COLTASK;
        r.vec_per_lane = nv;
        r.lanes_per_row = tpr;
        r.rows_per_block = rpb;
        r.block_threads = 256;
        const int ncol = ceil_div(nvec, vb);
        r.grid = ncol + ceil_div(rows, rpb);
        r.partials = 0;
        r.reduce_grid = ncol;  // reported: blocks that run column tasks
        out->workspace = 0;
        return RMSN_OK;
    }

    // Large T: row kernel with register dw sums per block.
    const int nv = nvec <= 1024 ? 1 : 2;
    const int tpr = lanes_per_row(nvec, nv);
    const int rpb = tpr <= 256 ? 256 / tpr : 1;
    r.vec_per_lane = nv;
    r.lanes_per_row = tpr;
    r.rows_per_block = rpb;
    r.block_threads = tpr * rpb;
    // Every block must be resident at once (the partition is fixed, so a
    // second round of blocks would double the tail): aim at 16 waves per CU.
    int per_cu = kBwdThreadsPerCU / r.block_threads;
    if (per_cu < 1) per_cu = 1;
    const int64_t cap = (int64_t)kPartitionCUs * per_cu;
    int64_t g = ceil_div(rows, 4 * rpb);  // at least ~4 rows per slot
    r.grid = g < cap ? g : cap;
    if (r.grid < 1) r.grid = 1;
    if (det) {
        r.kind = RMSN_KIND_BWD_ROW_DET;
        r.partial_f64 = rows > kPartialF32MaxRows ? 1 : 0;
        r.partials = r.grid;
        const int cpc = r.partial_f64 ? 2 : 4;
        r.reduce_grid = ceil_div(H, 16 * cpc);
        out->workspace = align256((size_t)r.partials * (size_t)H * (r.partial_f64 ? 8 : 4));
    } else {
        r.kind = RMSN_KIND_BWD_ROW_ATOMIC;
        r.partial_f64 = 1;
        r.partials = 0;
        r.reduce_grid = 0;
        out->workspace = align256((size_t)H * 8) + 256;
    }
    return RMSN_OK;
}

}  // namespace rmsn
