// Route table: which kernel and launch shape serve (op, rows, H, weight
// dtype, mode, form). Host-only and deterministic: a function of its
// arguments (and of an explicit tuning override, if one is set), never of
// the device, so the deterministic backward's row partition — and with it
// the dw bits — is fixed by the shape.
//
// The pages pick among kernel kinds by windows of T per (GPU, H, weight
// dtype) (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a dw-accuracy
// backward routes", "Changed windows by reason"). The kinds kept here are
// the ones that still hold on gfx950: a column-task kernel for small T (the
// page serves T from 1 to 64 with its column-task kernel), and a row kernel
// with per-block dw partials plus a reduce (the "chunk-partials pair") for
// both modes, or with atomics when an override asks for them. No
// dw-accuracy cut is needed above that: FP64 dw accumulation keeps every
// shape inside the budget.
#include <string.h>

#include "rmsn_internal.h"

namespace rmsn {

namespace {

// Rows at or below this use the column-task kernel (both modes).
constexpr int64_t kSmallRows = 64;
// Deterministic partials are stored in FP32 up to this many rows, FP64 above
// (the FP32 rounding of each partial adds ~3e-8 * sqrt(T) absolute error).
constexpr int64_t kPartialF32MaxRows = 8192;

// LayerNorm's backward keeps twice the FP64 accumulators (dgamma and
// dbeta): one vector per lane where the RMSNorm table takes two for wide rows.
constexpr int kOps = 4;
bool g_have_knobs[kOps] = {false, false, false, false};
rmsn_route_knobs_t g_knobs[kOps];
// Largest dynamic LDS a block asks for (the LayerNorm slot combine holds 2H
// doubles when a block has several row groups).
constexpr size_t kMaxLds = 64 * 1024;
// MI355X's Infinity Cache (the memory-side cache behind the L2s).
constexpr double kMallBytes = 256.0 * 1024 * 1024;

// Cache policy of the row kernels' loads (RMSNorm and LayerNorm), a
// function of the shape only. When the forward's tensors (x and y, plus r
// and h in the residual form) fill the Infinity Cache, the backward loads
// every large input non-temporally (2): it is their last reader in the step.
// Otherwise x can still be found by the backward: from 32M elements only
// the tensors read once (dy, dres) are streamed (1), which keeps them from
// evicting x; below that (0) plain loads measured no faster. The forward
// streams only inputs that no later kernel reads, x and r of the residual
// form (whose backward reads h), and only at level 2: streaming the plain
// form's x, which the backward reads again, made the step slower at every
// size measured (up to 6 %). Step times, fwd + deterministic bwd in
// 200-step graphs, against plain loads everywhere: 131072 x 2048 -2.7 %,
// 16384 x 6144 residual -3.7 %, 32768 x 24 x 256 strided -11.3 %,
// 32768 x 4 x 256 -2.1 %, 1048576 x 512 -6.4 %, 262144 x 1536 -8.2 %,
// 65536 x 5120 -3.3 %, 8192 x 16384 -12.4 %, 4096 x 4096 unchanged;
// LayerNorm 65536 x 4096 -10.3 %, 8192 x 16384 -1.8 %.
int stream_level(int64_t rows, int64_t H, bool residual) {
    const double e = (double)rows * (double)H;
    const double fwd_bytes = e * 2.0 * (residual ? 4.0 : 2.0);
    if (fwd_bytes >= kMallBytes) return 2;
    if (e >= 32.0 * 1024 * 1024) return 1;
    return 0;
}

// The RMSNorm backward streams dy and dres at every size below that cache
// size too. Retimed with the current launch shapes (same-process A/B, four
// repetitions, steps in 400-step graphs): 4096 x 4096 -1.7 %, 8192 x 2048
// -6.8 %, 8192 x 1024 -6.2 %, 4096 x 6144 -1.0 %, 2048 x 4096 -1.6 %,
// 1024 x 4096 -0.6 %, residual 4096 x 4096 -1.9 %, 65536 x 256 -2.7 %.
// LayerNorm's backward keeps the 32M-element rule above: the same change
// gave it -2.2 % to +1.7 %.
int rms_bwd_stream_level(int64_t rows, int64_t H, bool residual) {
    const int lvl = stream_level(rows, H, residual);
    return lvl > 1 ? lvl : 1;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Lanes per row for `nvec` 16-byte vectors at `nv` vectors per lane: a power
// of two up to one wave, else a whole number of waves.
int lanes_per_row(int nvec, int nv) {
    const int need = (int)ceil_div(nvec, nv);
    if (need <= 64) {
        int t = 1;
        while (t < need) t <<= 1;
        return t;
    }
    return (int)ceil_div(need, 64) * 64;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Default launch shapes of the row kernels by width (nvec 16-byte vectors
// per row), chosen by timing every compiled shape on MI355X in step mode
// (forward then backward in graphs, as training runs them, with the load
// policy above) at the workloads of each width: H 256 (per-head views), 512,
// 1536, 2048, 4096, 5120, 6144 (plain and residual), 8192 and 16384, then
// confirming each change with an in-process A/B.
// rpb_threads sets the row groups per block (threads / lanes per row).
struct Shape {
    int nv, unroll, rpb, bpc;
};
struct Entry {
    int max_nvec, nv, unroll, rpb_threads, bpc;
};
constexpr Entry kFwdTable[] = {
    {32, 4, 1, 256, 2},     // H <= 256: 8 lanes per row, 32 rows per block
    {64, 4, 1, 256, 2},     // H <= 512: 16 lanes per row, 16 rows per block
    {192, 4, 2, 256, 1},    // H <= 1536: 64 lanes per row, 4 row groups, 2 rows per iteration
    {256, 2, 1, 512, 4},    // H <= 2048: 4 row groups of 128 lanes, 4 blocks per CU
    {512, 2, 4, 256, 4},    // H <= 4096: 256 lanes per row, 4 rows per iteration
    {640, 2, 1, 640, 2},    // H <= 5120: 2 row groups of 320 lanes, 2 blocks per CU
    {768, 2, 1, 768, 1},    // H <= 6144: 2 row groups of 384 lanes
    {1024, 2, 1, 0, 2},     // H <= 8192
    {1 << 30, 4, 1, 0, 1},  // H <= 16384
};
constexpr Entry kBwdTable[] = {
    {32, 2, 1, 256, 2},     // H <= 256: 16 lanes per row, 16 rows per block, 2 blocks per CU
    {64, 2, 2, 256, 1},     // H <= 512: 32 lanes per row, 8 row groups, 2 rows per iteration
    {192, 1, 1, 768, 1},    // H <= 1536: one lane per vector, 768-thread blocks
    {256, 1, 1, 1024, 1},   // H <= 2048: 4 row groups of 256 lanes, 1 block per CU
    {512, 1, 1, 1024, 1},   // H <= 4096: 2 row groups of 512 lanes (3 of 320 up to 2560), 1 block per CU
    {640, 4, 1, 384, 1},    // H <= 5120: 2 row groups of 192 lanes, four vectors each
    {768, 1, 1, 0, 1},      // H <= 6144: 768 lanes, one row per block
    {1024, 1, 1, 0, 1},     // H <= 8192: 1024 lanes, one row per block
    {1 << 30, 4, 1, 0, 1},  // H <= 16384: 512 lanes, four vectors each
};

// Recompute-form backward (rmsnorm_bwd_recompute), timed as forward +
// recompute backward in step graphs at the workloads of each width class
// (T 4096 to 1048576). Its rows end in a serial chain (FP64 sum of squares,
// exchange, square root and division) that the plain backward does not
// have, so it wants more rows in flight per CU: more vectors per lane,
// smaller blocks, more of them.
constexpr Entry kRcBwdTable[] = {
    {32, 2, 1, 256, 2},     // H <= 256: as the plain backward
    {64, 4, 1, 64, 4},      // H <= 512: 16 lanes per row, 4 rows per block
    {192, 2, 2, 128, 4},    // H <= 1536: 128 lanes, 2 rows per iteration, 4 blocks per CU
    {256, 2, 2, 256, 2},    // H <= 2048: 2 row groups of 128 lanes, 2 blocks per CU
    {512, 2, 2, 256, 2},    // H <= 4096: 256 lanes, 2 rows per iteration
    {640, 4, 1, 384, 1},    // H <= 5120: 2 row groups of 192 lanes
    {768, 4, 1, 0, 2},      // H <= 6144: 192 lanes, one row per block, 2 blocks per CU
    {1024, 4, 1, 0, 2},     // H <= 8192: 256 lanes, one row per block, 2 blocks per CU
    {1 << 30, 4, 1, 0, 1},  // H <= 16384: as the plain backward
};

template <size_t N>
Shape lookup(const Entry (&t)[N], int nvec) {
    for (const Entry& e : t) {
        if (nvec <= e.max_nvec) {
            Shape s{e.nv, e.unroll, 0, e.bpc};
            const int need = (nvec + e.nv - 1) / e.nv;
            int tpr = 1;
            if (need <= 64) {
                while (tpr < need) tpr <<= 1;
            } else {
                tpr = (need + 63) / 64 * 64;
            }
            int threads = e.rpb_threads;
            if (tpr <= 64 && threads > 256) threads = 256;
            if (threads > 0 && threads / tpr >= 1) s.rpb = threads / tpr;
            return s;
        }
    }
    return Shape{1, 1, 0, 0};
}

// LayerNorm, timed in step mode at the shapes of the TE page's
// normalization table (8192 tokens x 3584, 4096, 8192, 16384) and at
// 65536 x 2048. Its forward holds no FP64 accumulators and does two row
// exchanges, so it takes four vectors per lane and fewer lanes per row.
constexpr Entry kLnFwdTable[] = {
    {32, 4, 1, 256, 2},     // H <= 256
    {64, 4, 1, 256, 2},     // H <= 512
    {256, 4, 1, 256, 2},    // H <= 2048
    {512, 4, 1, 256, 2},    // H <= 4096: 128 lanes per row, 2 rows per block
    {1024, 4, 1, 256, 2},   // H <= 8192: 256 lanes, one row per block, 2 blocks per CU
    {1 << 30, 4, 1, 0, 1},  // H <= 16384
};
constexpr Entry kLnBwdTable[] = {
    {32, 2, 1, 128, 4},     // H <= 256
    {64, 2, 1, 128, 4},     // H <= 512
    {192, 1, 1, 768, 1},    // H <= 1536
    {256, 2, 2, 256, 2},    // H <= 2048: 128 lanes, 2 rows per iteration, 2 blocks per CU
    {512, 1, 1, 0, 2},      // H <= 4096
    {640, 1, 1, 0, 1},      // H <= 5120
    {1024, 1, 1, 0, 1},     // H <= 8192: 1024 lanes, one row per block
    {1 << 30, 4, 1, 0, 1},  // H <= 16384: 512 lanes, four vectors each
};

Shape default_fwd(int nvec) { return lookup(kFwdTable, nvec); }
Shape default_bwd(int nvec) { return lookup(kBwdTable, nvec); }
Shape default_rc_bwd(int nvec) { return lookup(kRcBwdTable, nvec); }
Shape default_ln_fwd(int nvec) { return lookup(kLnFwdTable, nvec); }
Shape default_ln_bwd(int nvec) { return lookup(kLnBwdTable, nvec); }

// Fill the row-kernel part of a route from a shape; 0 fields take defaults.
// The checks mirror what the kernels are compiled for: (NV, U) pairs with
// NV * U <= 8 (the backwards' NV 4 only with U = 1, and NV * U <= 4 for the
// RMSNorm backward), blocks of <= 256 threads when a row fits in one wave;
// for wider rows <= 512 when NV * U >= 4 (the backwards: >= 2), else <= 1024.
int row_shape(int op, int nvec, Shape sh, rmsn_route_t& r) {
    const int nv = sh.nv;
    // NV 4: the forwards (ops 0, 2), and the backwards (ops 1, 3) with U = 1
    const bool nv_ok = nv == 1 || nv == 2 || (nv == 4 && (op == 0 || op == 2)) ||
                       (nv == 4 && (op == 1 || op == 3) && sh.unroll == 1);
    if (!nv_ok) return RMSN_ERR_SHAPE;
    const int tpr = lanes_per_row(nvec, nv);
    if (tpr > 1024) return RMSN_ERR_SHAPE;
    const int u = sh.unroll;
    if (!(u == 1 || u == 2 || u == 4 || u == 8)) return RMSN_ERR_SHAPE;
    if (nv * u > 8) return RMSN_ERR_SHAPE;
    if (op == 1 && nv * u > 4) return RMSN_ERR_SHAPE;
    int rpb = sh.rpb;
    if (rpb <= 0) rpb = tpr <= 256 ? 256 / tpr : 1;
    if ((int64_t)rpb * tpr > 1024) return RMSN_ERR_SHAPE;
    const int threads = rpb * tpr;
    if (threads % 64 != 0) return RMSN_ERR_SHAPE;
    if (tpr <= 64 && threads > 256) return RMSN_ERR_SHAPE;
    const bool bwd = op == 1 || op == 3;
    if (tpr > 64 && nv * u >= (bwd ? 2 : 4) && threads > 512) return RMSN_ERR_SHAPE;
    r.vec_per_lane = nv;
    r.lanes_per_row = tpr;
    r.rows_per_block = rpb;
    r.unroll = u;
    r.block_threads = threads;
    return RMSN_OK;
}

void apply_knobs(const rmsn_route_knobs_t& k, Shape& sh) {
    if (k.vec_per_lane && k.vec_per_lane != sh.nv) {
        // the table's rows per iteration and row groups per block were sized
        // for its own vector width
        sh.nv = k.vec_per_lane;
        sh.unroll = 1;
        sh.rpb = 0;
    }
    if (k.unroll) sh.unroll = k.unroll;
    if (k.rows_per_block) sh.rpb = k.rows_per_block;
    if (k.blocks_per_cu) sh.bpc = k.blocks_per_cu;
}

}  // namespace

int set_route_knobs(int op, const rmsn_route_knobs_t* k) {
    if (op < 0 || op >= kOps) return RMSN_ERR_SHAPE;
    if (!k) {
        g_have_knobs[op] = false;
        return RMSN_OK;
    }
    if (k->blocks_per_cu < 0 || k->blocks_per_cu > 32 || k->rows_per_block < 0 ||
        k->rows_per_block > 1024 || k->vec_per_lane < 0 || k->unroll < 0 || k->partial_f64 < 0 ||
        k->partial_f64 > 2 || k->stream_loads < 0 || k->stream_loads > 3)
        return RMSN_ERR_SHAPE;
    if (k->kind != 0 && k->kind != RMSN_KIND_BWD_ROW_DET && k->kind != RMSN_KIND_BWD_ROW_ATOMIC)
        return RMSN_ERR_SHAPE;
    g_knobs[op] = *k;
    g_have_knobs[op] = true;
    return RMSN_OK;
}

int route(int op, int64_t rows, int64_t H, rmsn_dtype_t wdt, int det, int form, Route* out) {
    if (!out) return RMSN_ERR_NULL;
    memset(out, 0, sizeof(*out));
    if (wdt != RMSN_BF16 && wdt != RMSN_F32) return RMSN_ERR_DTYPE;
    if (H < kVec || H > kMaxH || H % kVec != 0 || rows < 0 || rows > INT32_MAX)
        return RMSN_ERR_SHAPE;
    if (op < 0 || op >= kOps) return RMSN_ERR_SHAPE;
    if (form != kFormPlain && form != kFormResidual && form != kFormRecompute) return RMSN_ERR_SHAPE;
    const int nvec = (int)(H / kVec);
    rmsn_route_t& r = out->r;
    int st;

    if (op == 2) {  // LayerNorm forward
        Shape sh = default_ln_fwd(nvec);
        if (g_have_knobs[2]) apply_knobs(g_knobs[2], sh);
        if ((st = row_shape(0, nvec, sh, r)) != RMSN_OK) return st;
        const int nv = r.vec_per_lane, u = r.unroll;  // compiled pairs
        if (!((nv == 1 && u <= 2) || (nv == 2 && u <= 4 && u != 3) || (nv == 4 && u == 1)))
            return RMSN_ERR_SHAPE;
        r.kind = RMSN_KIND_FWD_ROW;
        r.stream_loads = 0;  // the backward reads x again
        if (g_have_knobs[2] && g_knobs[2].stream_loads) r.stream_loads = g_knobs[2].stream_loads - 1;
        const int bpc = sh.bpc > 0 ? sh.bpc : (2048 / r.block_threads > 0 ? 2048 / r.block_threads : 1);
        const int64_t cap = (int64_t)kPartitionCUs * bpc;
        const int64_t g = ceil_div(rows, (int64_t)r.rows_per_block * r.unroll);
        r.grid = g < cap ? g : cap;
        if (r.grid < 1) r.grid = 1;
        return RMSN_OK;
    }

    if (op == 3) {  // LayerNorm backward: row kernel + [P, 2H] partials at every T
        Shape sh = default_ln_bwd(nvec);
        const rmsn_route_knobs_t* k = g_have_knobs[3] ? &g_knobs[3] : nullptr;
        if (k) apply_knobs(*k, sh);
        if ((st = row_shape(3, nvec, sh, r)) != RMSN_OK) return st;
        if (r.unroll > 2) return RMSN_ERR_SHAPE;  // compiled pairs
        if (r.rows_per_block > 1 && (size_t)16 * H > kMaxLds) return RMSN_ERR_SHAPE;
        int bpc = sh.bpc > 0 ? sh.bpc : 1024 / r.block_threads;
        if (bpc < 1) bpc = 1;
        const int64_t cap = (int64_t)kPartitionCUs * bpc;
        const int64_t g = ceil_div(rows, 4LL * r.rows_per_block * r.unroll);
        r.grid = g < cap ? g : cap;
        if (r.grid < 1) r.grid = 1;
        r.kind = RMSN_KIND_BWD_ROW_DET;
        r.stream_loads = stream_level(rows, H, false);
        if (k && k->stream_loads) r.stream_loads = k->stream_loads - 1;
        r.partial_f64 = rows > kPartialF32MaxRows ? 1 : 0;
        if (k && k->partial_f64) r.partial_f64 = k->partial_f64 == 1 ? 1 : 0;
        r.partials = r.grid;
        const int psize = r.partial_f64 ? 8 : 4;
        r.reduce_grid = ceil_div(2 * H * psize, 16 * kReduceChunks);
        r.reduce_threads = kReduceThreads;
        out->workspace = align256((size_t)r.partials * (size_t)(2 * H) * psize);
        (void)det;
        return RMSN_OK;
    }

    if (op == 0) {
        Shape sh = default_fwd(nvec);
        if (g_have_knobs[0]) apply_knobs(g_knobs[0], sh);
        if ((st = row_shape(0, nvec, sh, r)) != RMSN_OK) return st;
        r.kind = RMSN_KIND_FWD_ROW;
        r.stream_loads = form == kFormResidual && stream_level(rows, H, true) == 2 ? 2 : 0;
        if (g_have_knobs[0] && g_knobs[0].stream_loads) r.stream_loads = g_knobs[0].stream_loads - 1;
        const int bpc = sh.bpc > 0 ? sh.bpc : (2048 / r.block_threads > 0 ? 2048 / r.block_threads : 1);
        const int64_t cap = (int64_t)kPartitionCUs * bpc;
        const int64_t g = ceil_div(rows, (int64_t)r.rows_per_block * r.unroll);
        r.grid = g < cap ? g : cap;
        if (r.grid < 1) r.grid = 1;
        return RMSN_OK;
    }

    if (rows <= kSmallRows && form != kFormRecompute) {
        // Column tasks for dw + row tasks for dx in one launch of 256 threads.
        // (The recompute form takes the row kernel at every T: its column
        // tasks would need every row's rstd before they start.)
        const int nv = nvec <= 256 ? 1 : (nvec <= 512 ? 2 : (nvec <= 1024 ? 4 : 8));
        const int tpr = lanes_per_row(nvec, nv);
        const int rpb = tpr <= 256 ? 256 / tpr : 1;
        const int splits = 8;
        const int vb = 256 / splits;
        r.kind = RMSN_KIND_BWD_COLTASK;
        r.vec_per_lane = nv;
        r.lanes_per_row = tpr;
        r.rows_per_block = rpb;
        r.unroll = 1;
        r.block_threads = 256;
        const int64_t ncol = ceil_div(nvec, vb);
        r.grid = ncol + ceil_div(rows, rpb);
        r.partials = 0;
        r.reduce_grid = ncol;  // reported: blocks that run column tasks
        out->workspace = 0;
        return RMSN_OK;
    }

    // Large T: row kernel with register dw sums per block.
    Shape sh = form == kFormRecompute ? default_rc_bwd(nvec) : default_bwd(nvec);
    const rmsn_route_knobs_t* k = g_have_knobs[1] ? &g_knobs[1] : nullptr;
    if (k) apply_knobs(*k, sh);
    if ((st = row_shape(1, nvec, sh, r)) != RMSN_OK) return st;
    if (r.rows_per_block > 1 && (size_t)8 * H > kMaxLds) return RMSN_ERR_SHAPE;
    // Every block should be resident at once (the partition is fixed, so a
    // second round of blocks would lengthen the tail): by default 16 waves
    // per CU.
    int bpc = sh.bpc > 0 ? sh.bpc : 1024 / r.block_threads;
    if (bpc < 1) bpc = 1;
    const int64_t cap = (int64_t)kPartitionCUs * bpc;
    const int64_t g = ceil_div(rows, 4LL * r.rows_per_block * r.unroll);  // ~4 iterations or more
    r.grid = g < cap ? g : cap;
    if (r.grid < 1) r.grid = 1;
    r.stream_loads = rms_bwd_stream_level(rows, H, form == kFormResidual);
    if (k && k->stream_loads) r.stream_loads = k->stream_loads - 1;
    // Both modes take the fixed-order two-stage path: the atomic finalise,
    // the one reduction that would differ, measured slower on this part at
    // every workload (4096 x 4096: 160 against 36.8 us per step). It stays
    // reachable for non-deterministic calls through the tuning override.
    int kind = RMSN_KIND_BWD_ROW_DET;
    if (k && k->kind && !det) kind = k->kind;
    if (kind == RMSN_KIND_BWD_ROW_DET) {
        r.kind = RMSN_KIND_BWD_ROW_DET;
        r.partial_f64 = rows > kPartialF32MaxRows ? 1 : 0;
        if (k && k->partial_f64) r.partial_f64 = k->partial_f64 == 1 ? 1 : 0;
        r.partials = r.grid;
        const int psize = r.partial_f64 ? 8 : 4;
        r.reduce_grid = ceil_div(H * psize, 16 * kReduceChunks);
        r.reduce_threads = kReduceThreads;
        out->workspace = align256((size_t)r.partials * (size_t)H * psize);
    } else {
        if (r.vec_per_lane != 1 || r.unroll > 2) return RMSN_ERR_SHAPE;  // compiled variants
        r.kind = RMSN_KIND_BWD_ROW_ATOMIC;
        r.partial_f64 = 1;
        r.partials = 0;
        r.reduce_grid = 0;
        out->workspace = align256((size_t)H * 8) + 256;
    }
    return RMSN_OK;
}

}  // namespace rmsn
