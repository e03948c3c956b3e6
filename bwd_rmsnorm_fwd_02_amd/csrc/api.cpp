// C ABI of the RMSNorm library: argument validation, routing and launches.
// Every check happens on the host before anything is enqueued; the kernels
// assume the shapes, strides and alignments validated here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "rmsn_internal.h"

using namespace rmsn;

namespace {

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

bool view_extent(const rmsn_view_t& v, int64_t* last_plus_one) {
    // offset of the element one past the last row's end
    int64_t a = 0, b = 0, e = 0;
    if (v.T == 0 || v.heads == 0) {
        *last_plus_one = 0;
        return true;
    }
    if (__builtin_mul_overflow(v.T - 1, v.stride_t, &a)) return false;
    if (__builtin_mul_overflow(v.heads - 1, v.stride_h, &b)) return false;
    if (__builtin_add_overflow(a, b, &e)) return false;
    if (__builtin_add_overflow(e, v.H, &e)) return false;
    int64_t bytes;
    if (__builtin_mul_overflow(e, (int64_t)2, &bytes)) return false;
    *last_plus_one = e;
    return true;
}

Span span_of(const void* p, int64_t elems, int64_t esize) {
    uintptr_t lo = (uintptr_t)p;
    return Span{lo, lo + (uintptr_t)(elems * esize)};
}

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool same_view(const rmsn_view_t& a, const rmsn_view_t& b) {
    return a.T == b.T && a.heads == b.heads && a.H == b.H && a.stride_t == b.stride_t &&
           a.stride_h == b.stride_h;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_dtype(rmsn_dtype_t d) { return (d == RMSN_BF16 || d == RMSN_F32) ? RMSN_OK : RMSN_ERR_DTYPE; }

int check_shape(const rmsn_view_t& v) {
    if (v.H < kVec || v.H > kMaxH || v.H % kVec != 0) return RMSN_ERR_SHAPE;
    if (v.T < 0 || v.heads < 1) return RMSN_ERR_SHAPE;
    if (v.stride_t < 0 || v.stride_h < 0) return RMSN_ERR_SHAPE;
    int64_t rows;
    if (__builtin_mul_overflow(v.T, v.heads, &rows)) return RMSN_ERR_OVERFLOW;
    if (rows > INT32_MAX) return RMSN_ERR_SHAPE;
    return RMSN_OK;
}

bool same_shape(const rmsn_view_t& a, const rmsn_view_t& b) {
    return a.T == b.T && a.heads == b.heads && a.H == b.H;
}

// Layout checks for one BF16 tensor view: base and strides 16-byte aligned.
int check_layout(const void* p, const rmsn_view_t& v, int64_t* extent) {
    if (!aligned(p, 16)) return RMSN_ERR_ALIGN;
    if (v.stride_t % kVec != 0 || v.stride_h % kVec != 0) return RMSN_ERR_ALIGN;
    if (!view_extent(v, extent)) return RMSN_ERR_OVERFLOW;
    return RMSN_OK;
}

// Rows of an output view must not overlap one another.
bool rows_disjoint(const rmsn_view_t& v) {
    if (v.heads > 1 && v.stride_h < v.H) return false;
    if (v.T > 1 && v.stride_t < (v.heads - 1) * v.stride_h + v.H) return false;
    return true;
}

rmsn_view_t contiguous(int64_t T, int64_t H) { return rmsn_view_t{T, 1, H, H, 0}; }

int64_t wsize(rmsn_dtype_t d) { return d == RMSN_BF16 ? 2 : 4; }

int check_eps(float eps) { return (isfinite(eps) && eps >= 0.f) ? RMSN_OK : RMSN_ERR_EPS; }

// ------------------------------------------------------------------ timers

struct TimerState {
    bool enabled = false;
    std::vector<hipEvent_t> start, stop;
    std::vector<int> kind;
    size_t used = 0;
    int64_t launches[RMSN_TIMER_COUNT] = {};
    double ms[RMSN_TIMER_COUNT] = {};
    int pending_kind = -1;
};
TimerState g_timer;
constexpr size_t kTimerPool = 4096;

}  // namespace

namespace rmsn {

void timer_begin(int kind, hipStream_t) {
    g_timer.pending_kind = g_timer.enabled ? kind : -1;
}

void timer_end(int, hipStream_t) { g_timer.pending_kind = -1; }

bool timer_take(hipEvent_t* start, hipEvent_t* stop) {
    if (!g_timer.enabled || g_timer.pending_kind < 0 || g_timer.used >= g_timer.start.size()) return false;
    *start = g_timer.start[g_timer.used];
    *stop = g_timer.stop[g_timer.used];
    g_timer.kind[g_timer.used] = g_timer.pending_kind;
    g_timer.used++;
    g_timer.pending_kind = -1;
    return true;
}

}  // namespace rmsn

namespace {

void drain_timers() {
    for (size_t i = 0; i < g_timer.used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_timer.stop[i]) == hipSuccess &&
            hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]) == hipSuccess) {
            g_timer.launches[g_timer.kind[i]] += 1;
            g_timer.ms[g_timer.kind[i]] += ms;
        }
    }
    g_timer.used = 0;
}

// ---------------------------------------------------------------- forward

int fwd_impl(const void* x, const rmsn_view_t& xv, const void* r, const rmsn_view_t* rv,
             void* h, const rmsn_view_t* hv, const void* w, rmsn_dtype_t wdt, float eps,
             void* y, const rmsn_view_t& yv, float* rstd, hipStream_t s) {
    const bool residual = (r != nullptr) || (rv != nullptr);
    int st;
    if ((st = check_dtype(wdt)) != RMSN_OK) return st;
    if ((st = check_shape(xv)) != RMSN_OK) return st;
    if ((st = check_shape(yv)) != RMSN_OK) return st;
    if (!same_shape(xv, yv)) return RMSN_ERR_SHAPE;
    if (residual) {
        if ((st = check_shape(*rv)) != RMSN_OK) return st;
        if ((st = check_shape(*hv)) != RMSN_OK) return st;
        if (!same_shape(xv, *rv) || !same_shape(xv, *hv)) return RMSN_ERR_SHAPE;
    }
    if ((st = check_eps(eps)) != RMSN_OK) return st;
    const int64_t rows = xv.T * xv.heads;
    if (rows == 0) return RMSN_OK;
    if (!x || !w || !y || !rstd) return RMSN_ERR_NULL;
    if (residual && (!r || !h)) return RMSN_ERR_NULL;
    int64_t ex, ey, er = 0, eh = 0;
    if ((st = check_layout(x, xv, &ex)) != RMSN_OK) return st;
    if ((st = check_layout(y, yv, &ey)) != RMSN_OK) return st;
    if (residual) {
        if ((st = check_layout(r, *rv, &er)) != RMSN_OK) return st;
        if ((st = check_layout(h, *hv, &eh)) != RMSN_OK) return st;
    }
    if (!aligned(w, 16) || !aligned(rstd, 4)) return RMSN_ERR_ALIGN;
    if (!rows_disjoint(yv) || (residual && !rows_disjoint(*hv))) return RMSN_ERR_ALIAS;

    const Span sx = span_of(x, ex, 2), sy = span_of(y, ey, 2);
    const Span sw = span_of(w, xv.H, wsize(wdt)), srs = span_of(rstd, rows, 4);
    const Span sr = residual ? span_of(r, er, 2) : Span{0, 0};
    const Span sh = residual ? span_of(h, eh, 2) : Span{0, 0};
    // y: may alias x exactly (plain form only)
    const bool y_inplace = !residual && x == y && same_view(xv, yv);
    if (!y_inplace && overlap(sy, sx)) return RMSN_ERR_ALIAS;
    if (overlap(sy, sw) || overlap(sy, srs)) return RMSN_ERR_ALIAS;
    if (overlap(srs, sx) || overlap(srs, sw)) return RMSN_ERR_ALIAS;
    if (residual) {
        const bool h_inplace = x == h && same_view(xv, *hv);
        if (!h_inplace && overlap(sh, sx)) return RMSN_ERR_ALIAS;
        if (overlap(sh, sr) || overlap(sh, sw) || overlap(sh, sy) || overlap(sh, srs)) return RMSN_ERR_ALIAS;
        if (overlap(sy, sr) || overlap(srs, sr)) return RMSN_ERR_ALIAS;
    }

    Route rt;
    if ((st = route(0, rows, xv.H, wdt, 1, residual ? kFormResidual : kFormPlain, &rt)) != RMSN_OK)
        return st;
    FwdParams p;
    memset(&p, 0, sizeof p);
    p.x = static_cast<const uint16_t*>(x);
    p.r = static_cast<const uint16_t*>(r);
    p.h = static_cast<uint16_t*>(h);
    p.y = static_cast<uint16_t*>(y);
    p.rstd = rstd;
    p.w = w;
    p.ax = RowAddr{xv.stride_t, xv.stride_h};
    p.ay = RowAddr{yv.stride_t, yv.stride_h};
    if (residual) {
        p.ar = RowAddr{rv->stride_t, rv->stride_h};
        p.ah = RowAddr{hv->stride_t, hv->stride_h};
    }
    p.rows = rows;
    p.heads = (int32_t)xv.heads;
    p.H = (int32_t)xv.H;
    p.nvec = (int32_t)(xv.H / kVec);
    p.tpr = rt.r.lanes_per_row;
    p.rpb = rt.r.rows_per_block;
    p.eps = eps;
    timer_begin(RMSN_TIMER_FWD, s);
    st = launch_fwd(p, rt, wdt, residual, s);
    timer_end(RMSN_TIMER_FWD, s);
    return st;
}

// --------------------------------------------------------------- backward

// Layout of the partial rows a deferred backward leaves for (rows, H): P
// rows of H FP64 or FP32 values in `bytes` bytes. Token counts up to the
// column-task limit leave one FP32 row holding the final dw.
int deferred_layout(int64_t rows, int64_t H, rmsn_dtype_t wdt, int64_t* P, int* f64,
                    size_t* bytes) {
    Route rt;
    const int st = route(1, rows, H, wdt, 1, kFormPlain, &rt);
    if (st != RMSN_OK) return st;
    if (rt.r.kind != RMSN_KIND_BWD_ROW_DET) {
        *P = 1;
        *f64 = 0;
        *bytes = ((size_t)H * 4 + 255) & ~(size_t)255;
        return RMSN_OK;
    }
    *P = rt.r.partials;
    *f64 = rt.r.partial_f64;
    *bytes = rt.workspace;
    return RMSN_OK;
}

// defer: leave the dw partial rows in `ws` (the caller's, laid out as
// deferred_layout says) instead of reducing them into dw, which is unused.
int bwd_impl(const void* dy, const rmsn_view_t& dyv, const void* x, const rmsn_view_t& xv,
             const void* dres, const rmsn_view_t* resv, const float* rstd, const void* w,
             rmsn_dtype_t wdt, int det, void* dx, const rmsn_view_t& dxv, float* dw,
             void* ws, size_t ws_bytes, int form, float eps, hipStream_t s, bool defer = false) {
    const bool residual = form == kFormResidual;
    if (defer) det = 1;
    const bool rc = form == kFormRecompute;  // rstd recomputed from x, none passed
    int st;
    if ((st = check_dtype(wdt)) != RMSN_OK) return st;
    if (rc && (st = check_eps(eps)) != RMSN_OK) return st;
    if ((st = check_shape(xv)) != RMSN_OK) return st;
    if ((st = check_shape(dyv)) != RMSN_OK) return st;
    if ((st = check_shape(dxv)) != RMSN_OK) return st;
    if (!same_shape(xv, dyv) || !same_shape(xv, dxv)) return RMSN_ERR_SHAPE;
    if (dres) {
        if ((st = check_shape(*resv)) != RMSN_OK) return st;
        if (!same_shape(xv, *resv)) return RMSN_ERR_SHAPE;
    }
    const int64_t rows = xv.T * xv.heads;
    const int64_t H = xv.H;
    if (defer) {
        int64_t P;
        int f64;
        size_t need;
        if ((st = deferred_layout(rows, H, wdt, &P, &f64, &need)) != RMSN_OK) return st;
        if (!ws || !aligned(ws, 256) || ws_bytes < need) return RMSN_ERR_WORKSPACE;
        if (rows == 0) {
            // one FP32 partial row of zeros: the column sum over no rows
            timer_begin(RMSN_TIMER_INIT, s);
            st = launch_fill_zero(ws, (size_t)H * 4, s);
            timer_end(RMSN_TIMER_INIT, s);
            return st;
        }
    } else {
        if (!dw) return RMSN_ERR_NULL;
        if (!aligned(dw, 4)) return RMSN_ERR_ALIGN;
    }
    if (rows == 0) {
        // the column sum over zero rows is zero
        timer_begin(RMSN_TIMER_INIT, s);
        st = launch_fill_zero(dw, (size_t)H * 4, s);
        timer_end(RMSN_TIMER_INIT, s);
        return st;
    }
    if (!x || !dy || (!rc && !rstd) || !w || !dx) return RMSN_ERR_NULL;
    if (residual && resv && !dres) return RMSN_ERR_NULL;
    if (!aligned(w, 16) || (!rc && !aligned(rstd, 4))) return RMSN_ERR_ALIGN;
    int64_t ex, edy, edx, eres = 0;
    if ((st = check_layout(x, xv, &ex)) != RMSN_OK) return st;
    if ((st = check_layout(dy, dyv, &edy)) != RMSN_OK) return st;
    if ((st = check_layout(dx, dxv, &edx)) != RMSN_OK) return st;
    if (dres && (st = check_layout(dres, *resv, &eres)) != RMSN_OK) return st;
    if (!rows_disjoint(dxv)) return RMSN_ERR_ALIAS;

    const Span sx = span_of(x, ex, 2), sdy = span_of(dy, edy, 2), sdx = span_of(dx, edx, 2);
    const Span sw = span_of(w, H, wsize(wdt));
    const Span srs = rc ? Span{0, 0} : span_of(rstd, rows, 4);
    const Span sdw = defer ? Span{0, 0} : span_of(dw, H, 4);
    const Span sres = dres ? span_of(dres, eres, 2) : Span{0, 0};
    if (overlap(sdx, sx) || overlap(sdx, sdy) || overlap(sdx, sw) || overlap(sdx, srs) ||
        overlap(sdx, sdw) || overlap(sdx, sres))
        return RMSN_ERR_ALIAS;
    if (overlap(sdw, sx) || overlap(sdw, sdy) || overlap(sdw, sw) || overlap(sdw, srs) || overlap(sdw, sres))
        return RMSN_ERR_ALIAS;

    Route rt;
    if ((st = route(1, rows, H, wdt, det, form, &rt)) != RMSN_OK) return st;
    // a deferred call's partial rows need room even where the route itself
    // needs no workspace (the column-task kernel's one dw row)
    const size_t ws_need = defer ? (rt.workspace > (size_t)H * 4 ? rt.workspace : (size_t)H * 4)
                                 : rt.workspace;
    if (ws_need > 0) {
        if (!ws || !aligned(ws, 256) || ws_bytes < ws_need) return RMSN_ERR_WORKSPACE;
        const Span sws = span_of(ws, (int64_t)ws_need, 1);
        if (overlap(sws, sx) || overlap(sws, sdy) || overlap(sws, sdx) || overlap(sws, sw) ||
            overlap(sws, srs) || overlap(sws, sdw) || overlap(sws, sres))
            return RMSN_ERR_ALIAS;
    }

    BwdParams p;
    memset(&p, 0, sizeof p);
    p.dy = static_cast<const uint16_t*>(dy);
    p.x = static_cast<const uint16_t*>(x);
    p.dres = static_cast<const uint16_t*>(dres);
    p.rstd = rstd;
    p.w = w;
    p.dx = static_cast<uint16_t*>(dx);
    p.dw = dw;
    p.ady = RowAddr{dyv.stride_t, dyv.stride_h};
    p.ax = RowAddr{xv.stride_t, xv.stride_h};
    p.adx = RowAddr{dxv.stride_t, dxv.stride_h};
    if (dres) p.ares = RowAddr{resv->stride_t, resv->stride_h};
    p.rows = rows;
    p.heads = (int32_t)xv.heads;
    p.H = (int32_t)H;
    p.nvec = (int32_t)(H / kVec);
    p.tpr = rt.r.lanes_per_row;
    p.rpb = rt.r.rows_per_block;
    p.eps = eps;

    if (rt.r.kind == RMSN_KIND_BWD_COLTASK) {
        if (defer) p.dw = static_cast<float*>(ws);  // the one partial row
        p.ncol_blocks = (int32_t)rt.r.reduce_grid;
        p.col_splits = 8;
        timer_begin(RMSN_TIMER_BWD_SMALL, s);
        st = launch_bwd_small(p, rt, wdt, residual, s);
        timer_end(RMSN_TIMER_BWD_SMALL, s);
        return st;
    }
    if (rt.r.kind == RMSN_KIND_BWD_ROW_DET) {
        p.partial = ws;
        timer_begin(RMSN_TIMER_BWD_ROW, s);
        st = launch_bwd_row(p, rt, wdt, form, s);
        timer_end(RMSN_TIMER_BWD_ROW, s);
        if (st != RMSN_OK || defer) return st;
        timer_begin(RMSN_TIMER_DW_REDUCE, s);
        st = launch_dw_reduce(p, rt, s);
        timer_end(RMSN_TIMER_DW_REDUCE, s);
        return st;
    }
    // atomic route: accumulator [H] doubles then the ticket, cleared first so
    // the workspace needs no initialisation by the caller
    p.acc = static_cast<double*>(ws);
    p.ticket = reinterpret_cast<unsigned int*>(static_cast<char*>(ws) + (((size_t)H * 8 + 255) & ~(size_t)255));
    timer_begin(RMSN_TIMER_INIT, s);
    st = launch_fill_zero(ws, rt.workspace, s);
    timer_end(RMSN_TIMER_INIT, s);
    if (st != RMSN_OK) return st;
    timer_begin(RMSN_TIMER_BWD_ROW, s);
    st = launch_bwd_row(p, rt, wdt, form, s);
    timer_end(RMSN_TIMER_BWD_ROW, s);
    return st;
}

// --------------------------------------------------------------- LayerNorm

int ln_fwd_impl(const void* x, const void* gamma, const void* beta, rmsn_dtype_t wdt, float eps,
                void* y, float* mean, float* rstd, int64_t T, int64_t H, hipStream_t s) {
    int st;
    if ((st = check_dtype(wdt)) != RMSN_OK) return st;
    const rmsn_view_t v = contiguous(T, H);
    if ((st = check_shape(v)) != RMSN_OK) return st;
    if ((st = check_eps(eps)) != RMSN_OK) return st;
    if (T == 0) return RMSN_OK;
    if (!x || !gamma || !y || !mean || !rstd) return RMSN_ERR_NULL;
    int64_t ex, ey;
    if ((st = check_layout(x, v, &ex)) != RMSN_OK) return st;
    if ((st = check_layout(y, v, &ey)) != RMSN_OK) return st;
    if (!aligned(gamma, 16) || (beta && !aligned(beta, 16)) || !aligned(mean, 4) || !aligned(rstd, 4))
        return RMSN_ERR_ALIGN;
    const Span sx = span_of(x, ex, 2), sy = span_of(y, ey, 2);
    const Span sg = span_of(gamma, H, wsize(wdt));
    const Span sb = beta ? span_of(beta, H, wsize(wdt)) : Span{0, 0};
    const Span sm = span_of(mean, T, 4), sr = span_of(rstd, T, 4);
    if (!(x == y) && overlap(sy, sx)) return RMSN_ERR_ALIAS;  // y may overwrite x exactly
    if (overlap(sy, sg) || overlap(sy, sb) || overlap(sy, sm) || overlap(sy, sr)) return RMSN_ERR_ALIAS;
    for (const Span& o : {sm, sr})
        if (overlap(o, sx) || overlap(o, sg) || overlap(o, sb)) return RMSN_ERR_ALIAS;
    if (overlap(sm, sr)) return RMSN_ERR_ALIAS;

    Route rt;
    if ((st = route(2, T, H, wdt, 1, kFormPlain, &rt)) != RMSN_OK) return st;
    LnFwdParams p;
    memset(&p, 0, sizeof p);
    p.x = static_cast<const uint16_t*>(x);
    p.y = static_cast<uint16_t*>(y);
    p.mean = mean;
    p.rstd = rstd;
    p.gamma = gamma;
    p.beta = beta;
    p.rows = T;
    p.H = (int32_t)H;
    p.nvec = (int32_t)(H / kVec);
    p.tpr = rt.r.lanes_per_row;
    p.rpb = rt.r.rows_per_block;
    p.eps = eps;
    timer_begin(RMSN_TIMER_FWD, s);
    st = launch_ln_fwd(p, rt, wdt, s);
    timer_end(RMSN_TIMER_FWD, s);
    return st;
}

int ln_bwd_impl(const void* dy, const void* x, const float* mean, const float* rstd,
                const void* gamma, rmsn_dtype_t wdt, int det, void* dx, float* dgamma,
                float* dbeta, int64_t T, int64_t H, void* ws, size_t ws_bytes, hipStream_t s) {
    int st;
    if ((st = check_dtype(wdt)) != RMSN_OK) return st;
    const rmsn_view_t v = contiguous(T, H);
    if ((st = check_shape(v)) != RMSN_OK) return st;
    if (!dgamma || !dbeta) return RMSN_ERR_NULL;
    if (!aligned(dgamma, 4) || !aligned(dbeta, 4)) return RMSN_ERR_ALIGN;
    const Span sdg = span_of(dgamma, H, 4), sdb = span_of(dbeta, H, 4);
    if (overlap(sdg, sdb)) return RMSN_ERR_ALIAS;
    if (T == 0) {
        // column sums over zero rows are zero
        timer_begin(RMSN_TIMER_INIT, s);
        st = launch_fill_zero(dgamma, (size_t)H * 4, s);
        if (st == RMSN_OK) st = launch_fill_zero(dbeta, (size_t)H * 4, s);
        timer_end(RMSN_TIMER_INIT, s);
        return st;
    }
    if (!dy || !x || !mean || !rstd || !gamma || !dx) return RMSN_ERR_NULL;
    int64_t ex, edy, edx;
    if ((st = check_layout(x, v, &ex)) != RMSN_OK) return st;
    if ((st = check_layout(dy, v, &edy)) != RMSN_OK) return st;
    if ((st = check_layout(dx, v, &edx)) != RMSN_OK) return st;
    if (!aligned(gamma, 16) || !aligned(mean, 4) || !aligned(rstd, 4)) return RMSN_ERR_ALIGN;
    const Span sx = span_of(x, ex, 2), sdy = span_of(dy, edy, 2), sdx = span_of(dx, edx, 2);
    const Span sg = span_of(gamma, H, wsize(wdt));
    const Span sm = span_of(mean, T, 4), sr = span_of(rstd, T, 4);
    for (const Span& o : {sdx, sdg, sdb}) {
        if (overlap(o, sx) || overlap(o, sdy) || overlap(o, sg) || overlap(o, sm) || overlap(o, sr))
            return RMSN_ERR_ALIAS;
    }
    if (overlap(sdx, sdg) || overlap(sdx, sdb)) return RMSN_ERR_ALIAS;

    Route rt;
    if ((st = route(3, T, H, wdt, det, kFormPlain, &rt)) != RMSN_OK) return st;
    if (!ws || !aligned(ws, 256) || ws_bytes < rt.workspace) return RMSN_ERR_WORKSPACE;
    const Span sws = span_of(ws, (int64_t)rt.workspace, 1);
    for (const Span& o : {sx, sdy, sdx, sg, sm, sr, sdg, sdb})
        if (overlap(sws, o)) return RMSN_ERR_ALIAS;

    LnBwdParams p;
    memset(&p, 0, sizeof p);
    p.dy = static_cast<const uint16_t*>(dy);
    p.x = static_cast<const uint16_t*>(x);
    p.mean = mean;
    p.rstd = rstd;
    p.gamma = gamma;
    p.dx = static_cast<uint16_t*>(dx);
    p.partial = ws;
    p.rows = T;
    p.H = (int32_t)H;
    p.nvec = (int32_t)(H / kVec);
    p.tpr = rt.r.lanes_per_row;
    p.rpb = rt.r.rows_per_block;
    timer_begin(RMSN_TIMER_BWD_ROW, s);
    st = launch_ln_bwd_row(p, rt, wdt, s);
    timer_end(RMSN_TIMER_BWD_ROW, s);
    if (st != RMSN_OK) return st;
    timer_begin(RMSN_TIMER_DW_REDUCE, s);
    st = launch_col_reduce(ws, rt, (int32_t)(2 * H), dgamma, dbeta, (int32_t)H, s);
    timer_end(RMSN_TIMER_DW_REDUCE, s);
    return st;
}

}  // namespace

// ==================================================================== C ABI

extern "C" {

int rmsnorm_fwd(const void* x, const void* w, rmsn_dtype_t w_dtype, float eps, void* y,
                float* rstd, int64_t T, int64_t H, hipStream_t stream) {
    const rmsn_view_t v = contiguous(T, H);
    return fwd_impl(x, v, nullptr, nullptr, nullptr, nullptr, w, w_dtype, eps, y, v, rstd, stream);
}

int rmsnorm_fwd_strided(const void* x, rmsn_view_t xv, const void* w, rmsn_dtype_t w_dtype,
                        float eps, void* y, rmsn_view_t yv, float* rstd, hipStream_t stream) {
    return fwd_impl(x, xv, nullptr, nullptr, nullptr, nullptr, w, w_dtype, eps, y, yv, rstd, stream);
}

int rmsnorm_residual_fwd(const void* x, const void* r, const void* w, rmsn_dtype_t w_dtype,
                         float eps, void* h, void* y, float* rstd, int64_t T, int64_t H,
                         hipStream_t stream) {
    const rmsn_view_t v = contiguous(T, H);
    if (!r && T * H != 0) return RMSN_ERR_NULL;
    return fwd_impl(x, v, r ? r : x, &v, h, &v, w, w_dtype, eps, y, v, rstd, stream);
}

int rmsnorm_residual_fwd_strided(const void* x, rmsn_view_t xv, const void* r, rmsn_view_t rv,
                                 const void* w, rmsn_dtype_t w_dtype, float eps, void* h,
                                 rmsn_view_t hv, void* y, rmsn_view_t yv, float* rstd,
                                 hipStream_t stream) {
    if (!r && xv.T * xv.heads != 0) return RMSN_ERR_NULL;
    return fwd_impl(x, xv, r ? r : x, &rv, h, &hv, w, w_dtype, eps, y, yv, rstd, stream);
}

size_t rmsnorm_bwd_workspace_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype,
                                   int deterministic) {
    // the largest need over the three backward forms
    size_t need = 0;
    for (int form : {kFormPlain, kFormResidual, kFormRecompute}) {
        Route rt;
        if (route(1, rows, H, w_dtype, deterministic, form, &rt) == RMSN_OK && rt.workspace > need)
            need = rt.workspace;
    }
    return need;
}

int rmsnorm_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (workspace_bytes == 0) return RMSN_OK;
    if (!workspace) return RMSN_ERR_NULL;
    timer_begin(RMSN_TIMER_INIT, stream);
    int st = launch_fill_zero(workspace, workspace_bytes, stream);
    timer_end(RMSN_TIMER_INIT, stream);
    return st;
}

int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* w,
                rmsn_dtype_t w_dtype, int deterministic, void* dx, float* dw, int64_t T,
                int64_t H, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const rmsn_view_t v = contiguous(T, H);
    return bwd_impl(dy, v, x, v, nullptr, nullptr, rstd, w, w_dtype, deterministic, dx, v, dw,
                    workspace, workspace_bytes, kFormPlain, 0.f, stream);
}

int rmsnorm_bwd_strided(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                        const float* rstd, const void* w, rmsn_dtype_t w_dtype, int deterministic,
                        void* dx, rmsn_view_t dxv, float* dw, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(dy, dyv, x, xv, nullptr, nullptr, rstd, w, w_dtype, deterministic, dx, dxv, dw,
                    workspace, workspace_bytes, kFormPlain, 0.f, stream);
}

int rmsnorm_bwd_recompute(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                          const void* w, rmsn_dtype_t w_dtype, float eps, int deterministic,
                          void* dx, rmsn_view_t dxv, float* dw, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(dy, dyv, x, xv, nullptr, nullptr, nullptr, w, w_dtype, deterministic, dx, dxv,
                    dw, workspace, workspace_bytes, kFormRecompute, eps, stream);
}

int rmsnorm_residual_bwd(const void* dy, const void* h, const void* dres, const float* rstd,
                         const void* w, rmsn_dtype_t w_dtype, int deterministic, void* dh,
                         float* dw, int64_t T, int64_t H, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    const rmsn_view_t v = contiguous(T, H);
    return bwd_impl(dy, v, h, v, dres, dres ? &v : nullptr, rstd, w, w_dtype, deterministic, dh, v,
                    dw, workspace, workspace_bytes, kFormResidual, 0.f, stream);
}

int rmsnorm_residual_bwd_strided(const void* dy, rmsn_view_t dyv, const void* h, rmsn_view_t hv,
                                 const void* dres, rmsn_view_t dresv, const float* rstd,
                                 const void* w, rmsn_dtype_t w_dtype, int deterministic, void* dh,
                                 rmsn_view_t dhv, float* dw, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return bwd_impl(dy, dyv, h, hv, dres, dres ? &dresv : nullptr, rstd, w, w_dtype, deterministic,
                    dh, dhv, dw, workspace, workspace_bytes, kFormResidual, 0.f, stream);
}

size_t rmsnorm_bwd_partials_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype) {
    int64_t P;
    int f64;
    size_t bytes;
    if (deferred_layout(rows, H, w_dtype, &P, &f64, &bytes) != RMSN_OK) return 0;
    return bytes;
}

int rmsnorm_bwd_strided_partials(const void* dy, rmsn_view_t dyv, const void* x, rmsn_view_t xv,
                                 const float* rstd, const void* w, rmsn_dtype_t w_dtype, void* dx,
                                 rmsn_view_t dxv, void* partials, size_t partials_bytes,
                                 hipStream_t stream) {
    return bwd_impl(dy, dyv, x, xv, nullptr, nullptr, rstd, w, w_dtype, 1, dx, dxv, nullptr,
                    partials, partials_bytes, kFormPlain, 0.f, stream, true);
}

int rmsnorm_residual_bwd_strided_partials(const void* dy, rmsn_view_t dyv, const void* h,
                                          rmsn_view_t hv, const void* dres, rmsn_view_t dresv,
                                          const float* rstd, const void* w, rmsn_dtype_t w_dtype,
                                          void* dh, rmsn_view_t dhv, void* partials,
                                          size_t partials_bytes, hipStream_t stream) {
    return bwd_impl(dy, dyv, h, hv, dres, dres ? &dresv : nullptr, rstd, w, w_dtype, 1, dh, dhv,
                    nullptr, partials, partials_bytes, kFormResidual, 0.f, stream, true);
}

int rmsnorm_dw_reduce_batch(const rmsn_dw_job_t* jobs, int n, hipStream_t stream) {
    if (n < 0) return RMSN_ERR_SHAPE;
    if (n == 0) return RMSN_OK;
    if (!jobs) return RMSN_ERR_NULL;
    // validate every job, and that no dw overlaps any job's partials or
    // another dw, before anything is enqueued
    std::vector<DwJob> f32, f64;
    std::vector<Span> parts, dws;
    for (int i = 0; i < n; ++i) {
        const rmsn_dw_job_t& jb = jobs[i];
        int st;
        if ((st = check_dtype(jb.w_dtype)) != RMSN_OK) return st;
        if (jb.H < kVec || jb.H > kMaxH || jb.H % kVec != 0 || jb.rows < 0 || jb.rows > INT32_MAX)
            return RMSN_ERR_SHAPE;
        if (!jb.partials || !jb.dw) return RMSN_ERR_NULL;
        if (!aligned(jb.partials, 16) || !aligned(jb.dw, 4)) return RMSN_ERR_ALIGN;
        int64_t P;
        int pf64;
        size_t bytes;
        if ((st = deferred_layout(jb.rows, jb.H, jb.w_dtype, &P, &pf64, &bytes)) != RMSN_OK) return st;
        const size_t used = (size_t)P * (size_t)jb.H * (pf64 ? 8 : 4);
        if (jb.partials_bytes < used) return RMSN_ERR_WORKSPACE;
        parts.push_back(span_of(jb.partials, (int64_t)used, 1));
        dws.push_back(span_of(jb.dw, jb.H, 4));
        DwJob d;
        d.part = jb.partials;
        d.P = P;
        d.H = (int32_t)jb.H;
        d.f64 = pf64;
        d.dw = jb.dw;
        d.block0 = 0;
        (pf64 ? f64 : f32).push_back(d);
    }
    for (int i = 0; i < n; ++i) {
        for (int k = 0; k < n; ++k) {
            if (overlap(dws[i], parts[k])) return RMSN_ERR_ALIAS;
            if (k != i && overlap(dws[i], dws[k])) return RMSN_ERR_ALIAS;
        }
    }
    // one launch per precision and per kMaxBatchJobs jobs; job blocks as in
    // the single reduce (16-byte chunks of kReduceChunks per block)
    for (std::vector<DwJob>* group : {&f32, &f64}) {
        for (size_t at = 0; at < group->size(); at += kMaxBatchJobs) {
            DwJobs t;
            memset(&t, 0, sizeof t);
            int64_t blocks = 0;
            const size_t m = std::min(group->size() - at, (size_t)kMaxBatchJobs);
            for (size_t q = 0; q < m; ++q) {
                DwJob d = (*group)[at + q];
                d.block0 = blocks;
                const int64_t psize = d.f64 ? 8 : 4;
                blocks += (d.H * psize + 16 * kReduceChunks - 1) / (16 * kReduceChunks);
                t.j[q] = d;
            }
            t.n = (int32_t)m;
            timer_begin(RMSN_TIMER_DW_REDUCE, stream);
            const int st = launch_dw_reduce_batch(t, blocks, stream);
            timer_end(RMSN_TIMER_DW_REDUCE, stream);
            if (st != RMSN_OK) return st;
        }
    }
    return RMSN_OK;
}

int layernorm_fwd(const void* x, const void* gamma, const void* beta, rmsn_dtype_t w_dtype,
                  float eps, void* y, float* mean, float* rstd, int64_t T, int64_t H,
                  hipStream_t stream) {
    return ln_fwd_impl(x, gamma, beta, w_dtype, eps, y, mean, rstd, T, H, stream);
}

size_t layernorm_bwd_workspace_bytes(int64_t rows, int64_t H, rmsn_dtype_t w_dtype,
                                     int deterministic) {
    Route rt;
    if (route(3, rows, H, w_dtype, deterministic, kFormPlain, &rt) != RMSN_OK) return 0;
    return rt.workspace;
}

int layernorm_bwd(const void* dy, const void* x, const float* mean, const float* rstd,
                  const void* gamma, rmsn_dtype_t w_dtype, int deterministic, void* dx,
                  float* dgamma, float* dbeta, int64_t T, int64_t H, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
    return ln_bwd_impl(dy, x, mean, rstd, gamma, w_dtype, deterministic, dx, dgamma, dbeta, T, H,
                       workspace, workspace_bytes, stream);
}

const char* rmsnorm_status_string(int status) {
    switch (status) {
        case RMSN_OK: return "ok";
        case RMSN_ERR_NULL: return "a required pointer is NULL";
        case RMSN_ERR_DTYPE: return "weight dtype must be RMSN_BF16 or RMSN_F32";
        case RMSN_ERR_SHAPE:
            return "bad shape: H must be a multiple of 8 in [8, 16384], T >= 0, heads >= 1, "
                   "rows <= 2^31-1, and all views must agree on T, heads and H";
        case RMSN_ERR_ALIGN:
            return "misaligned: BF16 tensors and weights need 16-byte aligned bases and strides "
                   "that are multiples of 8 elements; FP32 rstd/dw need 4-byte alignment";
        case RMSN_ERR_WORKSPACE:
            return "workspace is NULL, not 256-byte aligned, or smaller than "
                   "rmsnorm_bwd_workspace_bytes()";
        case RMSN_ERR_OVERFLOW: return "element offsets or byte sizes overflow int64";
        case RMSN_ERR_ALIAS:
            return "an output overlaps another tensor (only exact in-place y==x / h==x in the "
                   "forward is allowed) or an output view's rows overlap each other";
        case RMSN_ERR_LAUNCH: return "a HIP kernel launch failed";
        case RMSN_ERR_EPS: return "eps must be finite and >= 0";
        case RMSN_ERR_SCRATCH:
            return "the problem needs more dw partial rows than the no-alloc entry point's fixed "
                   "32 MiB scratch holds (or its device address could not be looked up)";
        default: return "unknown status";
    }
}

int rmsnorm_route_query(int op, int64_t rows, int64_t H, rmsn_dtype_t w_dtype, int deterministic,
                        int form, rmsn_route_t* out) {
    if (!out) return RMSN_ERR_NULL;
    Route rt;
    const int st = route(op, rows, H, w_dtype, deterministic, op <= 1 ? form : kFormPlain, &rt);
    *out = rt.r;
    return st;
}

int rmsnorm_route_override(int op, const rmsn_route_knobs_t* knobs) {
    return set_route_knobs(op, knobs);
}

int rmsnorm_timing_enable(int enable) {
    if (enable) {
        if (g_timer.start.empty()) {
            g_timer.start.resize(kTimerPool);
            g_timer.stop.resize(kTimerPool);
            g_timer.kind.resize(kTimerPool);
            for (size_t i = 0; i < kTimerPool; ++i) {
                if (hipEventCreate(&g_timer.start[i]) != hipSuccess ||
                    hipEventCreate(&g_timer.stop[i]) != hipSuccess) {
                    g_timer.start.resize(i);
                    g_timer.stop.resize(i);
                    break;
                }
            }
        }
        g_timer.enabled = true;
    } else {
        g_timer.enabled = false;
    }
    return RMSN_OK;
}

int rmsnorm_timing_read(int64_t* launches, double* total_ms, int n) {
    drain_timers();
    for (int i = 0; i < n && i < RMSN_TIMER_COUNT; ++i) {
        if (launches) launches[i] = g_timer.launches[i];
        if (total_ms) total_ms[i] = g_timer.ms[i];
    }
    for (int i = 0; i < RMSN_TIMER_COUNT; ++i) {
        g_timer.launches[i] = 0;
        g_timer.ms[i] = 0.0;
    }
    return RMSN_OK;
}

}  // extern "C"
