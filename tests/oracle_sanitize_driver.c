/*
 * Host-sanitizer driver for the FP64 oracle (test infrastructure). Built with
 * gcc -fsanitize=address,undefined by tests/test_oracle_sanitize_cpu.py; it
 * calls every oracle entry point on shapes from empty to ragged, each buffer
 * allocated at its exact size so that any access past its end is reported,
 * and checks that finite inputs give finite outputs. Exit status 0 on
 * success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/rmsnorm_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double next_unit(void) { /* xorshift64*, uniform in [-2, 2) */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    const uint64_t r = g_state * 0x2545F4914F6CDD1Dull;
    return 4.0 * (double)(r >> 11) / 9007199254740992.0 - 2.0;
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint16_t* bf16_array(int64_t n) {
    double* v = xmalloc(sizeof(double) * (size_t)n);
    uint16_t* b = xmalloc(sizeof(uint16_t) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) v[i] = next_unit();
    orc_round_bf16(n, v, b);
    free(v);
    return b;
}

static double* f64_array(int64_t n, double base) {
    double* v = xmalloc(sizeof(double) * (size_t)n);
    for (int64_t i = 0; i < n; ++i) v[i] = base + 0.1 * next_unit();
    return v;
}

static int all_finite(const double* v, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i])) return 0;
    return 1;
}

#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            fprintf(stderr, "check failed: %s (rows %lld H %lld)\n", #cond,     \
                    (long long)rows, (long long)H);                             \
            return 1;                                                           \
        }                                                                       \
    } while (0)

static int run_shape(int64_t rows, int64_t H) {
    const int64_t n = rows * H;
    uint16_t* x = bf16_array(n);
    uint16_t* dy = bf16_array(n);
    uint16_t* r = bf16_array(n);
    uint16_t* h = xmalloc(sizeof(uint16_t) * (size_t)n);
    double* w = f64_array(H, 1.0);
    double* beta = f64_array(H, 0.0);
    double* xw = xmalloc(sizeof(double) * (size_t)n);
    double* rstd = xmalloc(sizeof(double) * (size_t)rows);
    double* mu = xmalloc(sizeof(double) * (size_t)rows);
    double* y = xmalloc(sizeof(double) * (size_t)n);
    double* dx = xmalloc(sizeof(double) * (size_t)n);
    double* c = xmalloc(sizeof(double) * (size_t)(2 * rows));
    double* dw = xmalloc(sizeof(double) * (size_t)H);
    double* db = xmalloc(sizeof(double) * (size_t)H);
    float* f = xmalloc(sizeof(float) * (size_t)rows);
    uint16_t* yb = xmalloc(sizeof(uint16_t) * (size_t)n);

    orc_bf16_to_double(n, x, xw);
    orc_fwd(rows, H, x, w, 1e-6, rstd, y);
    CHECK(all_finite(rstd, rows) && all_finite(y, n));
    orc_round_bf16(n, y, yb);
    orc_round_f32(rows, rstd, f);
    orc_bwd(rows, H, dy, x, rstd, w, dx, c, dw);
    CHECK(all_finite(dx, n) && all_finite(c, rows) && all_finite(dw, H));
    orc_bwd(rows, H, dy, x, rstd, w, NULL, NULL, dw); /* dw-only pass */
    CHECK(all_finite(dw, H));
    orc_fwd_f64(rows, H, xw, w, 1e-6, rstd, y);
    orc_bwd_f64(rows, H, xw, xw, rstd, w, dx, c, dw);
    CHECK(all_finite(dx, n) && all_finite(dw, H));
    orc_residual_add(n, x, r, h);
    orc_ln_fwd(rows, H, h, w, beta, 1e-5, mu, rstd, y);
    CHECK(all_finite(mu, rows) && all_finite(rstd, rows) && all_finite(y, n));
    orc_ln_fwd(rows, H, h, w, NULL, 1e-5, mu, rstd, y); /* no bias */
    orc_ln_bwd(rows, H, dy, h, mu, rstd, w, dx, c, dw, db);
    CHECK(all_finite(dx, n) && all_finite(c, 2 * rows) && all_finite(dw, H) && all_finite(db, H));
    orc_ln_bwd(rows, H, dy, h, mu, rstd, w, NULL, NULL, dw, db);
    orc_ln_fwd_f64(rows, H, xw, w, beta, 1e-5, mu, rstd, y);
    orc_ln_bwd_f64(rows, H, xw, xw, mu, rstd, w, dx, c, dw, db);
    CHECK(all_finite(dx, n) && all_finite(dw, H) && all_finite(db, H));

    free(x); free(dy); free(r); free(h); free(w); free(beta); free(xw); free(rstd);
    free(mu); free(y); free(dx); free(c); free(dw); free(db); free(f); free(yb);
    return 0;
}

int main(void) {
    static const int64_t shapes[][2] = {{0, 8}, {1, 1}, {3, 5}, {17, 64}, {64, 256},
                                        {5, 1032}, {2, 16384}, {129, 24}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        if (run_shape(shapes[i][0], shapes[i][1])) return 1;
    printf("oracle sanitizer driver: all shapes ok\n");
    return 0;
}
