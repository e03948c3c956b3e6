// Host-sanitizer driver for the C ABI layer (test infrastructure), built with
// api.cpp, route.cpp and tests/abi_sanitize_stubs.cpp under AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_abi_sanitize_cpu.py. It queries
// the route table over a grid of shapes, including out-of-range ones, and
// calls every entry point with bad and with well-formed arguments (device
// pointers are never dereferenced on the host; well-formed calls end at the
// stubbed launch). Exit status 0 when every status code is the expected one.
#include <stdint.h>
#include <stdio.h>

#include "../include/rmsnorm.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const int got_ = (call);                                                    \
        if (got_ != (want)) {                                                       \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__,     \
                    #call, got_, (int)(want));                                      \
            ++g_fail;                                                               \
        }                                                                           \
    } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
    // route table over a grid of shapes (every status is valid; the sanitizers
    // watch the arithmetic and indexing)
    const int64_t rows[] = {-1, 0, 1, 63, 64, 65, 4096, 8192, 8193, 131072, 786432,
                            (int64_t)1 << 31, ((int64_t)1 << 31) - 1, (int64_t)1 << 62};
    const int64_t Hs[] = {-8, 0, 7, 8, 24, 256, 1032, 2048, 4096, 6144, 8192, 16384, 16392};
    long ok = 0;
    for (int op = -1; op <= 4; ++op)
        for (int64_t r : rows)
            for (int64_t H : Hs)
                for (int dt = 0; dt <= 2; ++dt)
                    for (int det = 0; det <= 1; ++det)
                        for (int form = 0; form <= 3; ++form) {
                            rmsn_route_t rt;
                            const int st = rmsnorm_route_query(op, r, H, (rmsn_dtype_t)dt, det, form, &rt);
                            if (st == RMSN_OK) {
                                ++ok;
                                if (rt.block_threads <= 0 || rt.block_threads > 1024 || rt.grid < 1) {
                                    fprintf(stderr, "bad route op %d rows %lld H %lld\n", op,
                                            (long long)r, (long long)H);
                                    ++g_fail;
                                }
                            }
                            (void)rmsnorm_bwd_workspace_bytes(r, H, (rmsn_dtype_t)dt, det);
                            (void)layernorm_bwd_workspace_bytes(r, H, (rmsn_dtype_t)dt, det);
                        }
    if (ok == 0) ++g_fail;
    EXPECT(rmsnorm_route_query(0, 64, 64, RMSN_BF16, 1, 0, nullptr), RMSN_ERR_NULL);
    for (int s = -20; s <= 5; ++s)
        if (!rmsnorm_status_string(s)) ++g_fail;

    // route knobs: set, use, clear
    rmsn_route_knobs_t k = {2, 2, 0, 0, 0, 0, 0};
    EXPECT(rmsnorm_route_override(1, &k), RMSN_OK);
    rmsn_route_t rt;
    (void)rmsnorm_route_query(1, 4096, 4096, RMSN_BF16, 1, 0, &rt);
    k.blocks_per_cu = 99;
    EXPECT(rmsnorm_route_override(1, &k), RMSN_ERR_SHAPE);
    EXPECT(rmsnorm_route_override(1, nullptr), RMSN_OK);
    EXPECT(rmsnorm_route_override(7, nullptr), RMSN_ERR_SHAPE);

    const hipStream_t s = nullptr;
    const uintptr_t A = 0x10000000;
    const int64_t T = 4096, H = 4096;
    const uintptr_t G = (uintptr_t)1 << 30;  // 1 GiB apart: no tensor here spans more
    void *X = fake(A), *Y = fake(A + G), *DY = fake(A + 2 * G), *DX = fake(A + 3 * G),
         *W = fake(A + 4 * G), *RS = fake(A + 5 * G), *DW = fake(A + 6 * G), *WS = fake(A + 7 * G),
         *R = fake(A + 8 * G), *MU = fake(A + 9 * G), *DB = fake(A + 10 * G);
    float *rs = static_cast<float*>(RS), *dw = static_cast<float*>(DW), *mu = static_cast<float*>(MU),
          *db = static_cast<float*>(DB);
    const size_t need = rmsnorm_bwd_workspace_bytes(T, H, RMSN_BF16, 1);

    // forward
    EXPECT(rmsnorm_fwd(X, W, RMSN_BF16, 1e-6f, Y, rs, T, H, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_fwd(X, W, RMSN_BF16, 1e-6f, X, rs, T, H, s), RMSN_ERR_LAUNCH);  // in place
    EXPECT(rmsnorm_fwd(X, W, RMSN_BF16, 1e-6f, Y, rs, T, 7, s), RMSN_ERR_SHAPE);
    EXPECT(rmsnorm_fwd(X, W, (rmsn_dtype_t)5, 1e-6f, Y, rs, T, H, s), RMSN_ERR_DTYPE);
    EXPECT(rmsnorm_fwd(nullptr, W, RMSN_BF16, 1e-6f, Y, rs, T, H, s), RMSN_ERR_NULL);
    EXPECT(rmsnorm_fwd(fake(A + 2), W, RMSN_BF16, 1e-6f, Y, rs, T, H, s), RMSN_ERR_ALIGN);
    EXPECT(rmsnorm_fwd(X, W, RMSN_BF16, -1.f, Y, rs, T, H, s), RMSN_ERR_EPS);
    EXPECT(rmsnorm_fwd(X, W, RMSN_BF16, 1e-6f, fake(A + 64), rs, T, H, s), RMSN_ERR_ALIAS);
    EXPECT(rmsnorm_fwd(nullptr, nullptr, RMSN_BF16, 1e-6f, nullptr, nullptr, 0, H, s), RMSN_OK);
    const rmsn_view_t xv = {32768, 24, 256, 8192, 256}, yv = {32768, 24, 256, 24 * 256, 256};
    EXPECT(rmsnorm_fwd_strided(X, xv, W, RMSN_F32, 1e-6f, Y, yv, rs, s), RMSN_ERR_LAUNCH);
    const rmsn_view_t huge = {10, 24, 256, (int64_t)1 << 62, 256};
    EXPECT(rmsnorm_fwd_strided(X, huge, W, RMSN_F32, 1e-6f, Y, yv, rs, s), RMSN_ERR_SHAPE);
    EXPECT(rmsnorm_residual_fwd(X, R, W, RMSN_BF16, 1e-6f, DX, Y, rs, T, H, s), RMSN_ERR_LAUNCH);

    // backward
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DX, dw, T, H, WS, need, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 0, DX, dw, T, H, WS, need, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DX, dw, T, H, WS, 4096, s), RMSN_ERR_WORKSPACE);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DY, dw, T, H, WS, need, s), RMSN_ERR_ALIAS);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DX, nullptr, T, H, WS, need, s), RMSN_ERR_NULL);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DX, dw, 64, 256, nullptr, 0, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd(DY, X, rs, W, RMSN_BF16, 1, DX, dw, 0, H, nullptr, 0, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd_strided(DY, yv, X, xv, rs, W, RMSN_F32, 1, DX, xv, dw, WS,
                               rmsnorm_bwd_workspace_bytes(32768 * 24, 256, RMSN_F32, 1), s),
           RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd_recompute(DY, yv, X, xv, W, RMSN_F32, 1e-6f, 1, DX, yv, dw, WS,
                                 rmsnorm_bwd_workspace_bytes(32768 * 24, 256, RMSN_F32, 1), s),
           RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_residual_bwd(DY, X, R, rs, W, RMSN_BF16, 1, DX, dw, T, H, WS, need, s),
           RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_workspace_init(WS, need, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_workspace_init(nullptr, 16, s), RMSN_ERR_NULL);

    // deferred dw reduction
    const rmsn_view_t pv = {T, 1, H, H, 0};
    const size_t pneed = rmsnorm_bwd_partials_bytes(T, H, RMSN_BF16);
    if (pneed == 0 || rmsnorm_bwd_partials_bytes(T, 7, RMSN_BF16) != 0) ++g_fail;
    EXPECT(rmsnorm_bwd_strided_partials(DY, pv, X, pv, rs, W, RMSN_BF16, DX, pv, WS, pneed, s),
           RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_bwd_strided_partials(DY, pv, X, pv, rs, W, RMSN_BF16, DX, pv, WS, pneed - 1, s),
           RMSN_ERR_WORKSPACE);
    EXPECT(rmsnorm_bwd_strided_partials(DY, pv, X, pv, rs, W, RMSN_BF16, DX, pv, fake(A + 7 * G + 16),
                                        pneed, s), RMSN_ERR_WORKSPACE);
    EXPECT(rmsnorm_bwd_strided_partials(DY, pv, X, pv, rs, W, RMSN_BF16, DX, pv, DX, pneed, s),
           RMSN_ERR_ALIAS);
    EXPECT(rmsnorm_residual_bwd_strided_partials(DY, pv, X, pv, R, pv, rs, W, RMSN_BF16, DX, pv, WS,
                                                 pneed, s), RMSN_ERR_LAUNCH);
    {
        const rmsn_view_t small = {64, 1, 256, 256, 0}, none = {0, 1, 256, 256, 0};
        const size_t sneed = rmsnorm_bwd_partials_bytes(64, 256, RMSN_F32);
        EXPECT(rmsnorm_bwd_strided_partials(DY, small, X, small, rs, W, RMSN_F32, DX, small, WS,
                                            sneed, s), RMSN_ERR_LAUNCH);
        EXPECT(rmsnorm_bwd_strided_partials(DY, none, X, none, rs, W, RMSN_F32, DX, none, WS, sneed, s),
               RMSN_ERR_LAUNCH);  // zero rows: the fill of one zero partial row
    }
    rmsn_dw_job_t jobs[40];
    for (int i = 0; i < 40; ++i)
        jobs[i] = rmsn_dw_job_t{fake(A + 7 * G + (uintptr_t)i * (pneed + 256)), pneed, T, H, RMSN_BF16,
                                static_cast<float*>(fake(A + 6 * G + (uintptr_t)i * H * 4))};
    EXPECT(rmsnorm_dw_reduce_batch(jobs, 40, s), RMSN_ERR_LAUNCH);
    EXPECT(rmsnorm_dw_reduce_batch(jobs, 0, s), RMSN_OK);
    EXPECT(rmsnorm_dw_reduce_batch(nullptr, 1, s), RMSN_ERR_NULL);
    EXPECT(rmsnorm_dw_reduce_batch(jobs, -1, s), RMSN_ERR_SHAPE);
    {
        rmsn_dw_job_t bad[2] = {jobs[0], jobs[1]};
        bad[1].partials_bytes = pneed / 2;
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_WORKSPACE);
        bad[1] = jobs[1];
        bad[1].dw = bad[0].dw;  // two jobs write one dw
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_ALIAS);
        bad[1] = jobs[1];
        bad[1].dw = static_cast<float*>(const_cast<void*>(bad[0].partials));  // dw over partials
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_ALIAS);
        bad[1] = jobs[1];
        bad[1].H = 12;
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_SHAPE);
        bad[1] = jobs[1];
        bad[1].w_dtype = (rmsn_dtype_t)3;
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_DTYPE);
        bad[1] = jobs[1];
        bad[1].partials = fake(A + 7 * G + 8);
        EXPECT(rmsnorm_dw_reduce_batch(bad, 2, s), RMSN_ERR_ALIGN);
    }

    // LayerNorm
    const size_t lneed = layernorm_bwd_workspace_bytes(T, H, RMSN_BF16, 1);
    EXPECT(layernorm_fwd(X, W, R, RMSN_BF16, 1e-5f, Y, mu, rs, T, H, s), RMSN_ERR_LAUNCH);
    EXPECT(layernorm_bwd(DY, X, mu, rs, W, RMSN_BF16, 1, DX, dw, db, T, H, WS, lneed, s),
           RMSN_ERR_LAUNCH);
    EXPECT(layernorm_bwd(DY, X, mu, rs, W, RMSN_BF16, 1, DX, dw, db, T, H, WS, lneed - 1, s),
           RMSN_ERR_WORKSPACE);

    // timers with no GPU events taken
    int64_t launches[8];
    double ms[8];
    EXPECT(rmsnorm_timing_read(launches, ms, 8), RMSN_OK);

    if (g_fail) {
        fprintf(stderr, "%d failures\n", g_fail);
        return 1;
    }
    printf("abi sanitizer driver: %ld routes queried, all status codes as expected\n", ok);
    return 0;
}
