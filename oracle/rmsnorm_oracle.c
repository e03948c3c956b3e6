/*
 * FP64 CPU oracle for RMSNorm training. TEST INFRASTRUCTURE ONLY: see the
 * header for who may use it and for the layout conventions.
 *
 * The method reaches a result with a plain definition (RMSNorm forward and
 * its exact gradient), so this file is that definition written out in
 * double precision, one row at a time, with no blocking or fusion:
 *
 *   forward   rstd_t = 1/sqrt((1/H) sum_j x_tj^2 + eps)
 *             y_tj   = (x_tj * rstd_t) * w_j
 *   backward  xhat   = x * rstd,  g = dy * w,
 *             c_t    = (1/H) sum_j g_tj * xhat_tj
 *             dx_tj  = rstd_t * (g_tj - xhat_tj * c_t)
 *             dw_j   = sum_t dy_tj * xhat_tj
 *   residual  h      = BF16(x + r) before the forward; the backward of the
 *             residual form adds the gradient arriving at h (done by the
 *             caller on the FP64 dx, so it is not repeated here).
 *
 * Source of the definition: flashinfer PR "fix(cake_rmsnorm): sm_100a and
 * sm_107a dw-accuracy backward routes" (opening description: outputs y and
 * rstd forward, dx and dw backward; "Key": h_new = BF16(h + u); "Workload":
 * eps 1e-6, y/dx/h_new BF16, rstd/dw FP32). The closed forms for rstd, dx
 * and dw are the usual RMSNorm ones; the tests pin them by finite
 * differences and invariants.
 *
 * Every sum uses Neumaier's compensated summation (an improved Kahan
 * summation), in index order. This keeps the dw reference, a sum over up to
 * about a million rows, within a few FP64 ulps of the exact sum.
 */
#include "rmsnorm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Running compensated sum (Neumaier). */
typedef struct {
    double s;
    double c;
} nsum_t;

static void nsum_add(nsum_t* a, double v) {
    double t = a->s + v;
    /* The correction term is defined for finite sums only: once the sum is
     * infinite or NaN it is the plain sum's value (inf - inf in the
     * correction would turn an infinite sum into NaN). */
    if (isfinite(t)) {
        if (fabs(a->s) >= fabs(v)) {
            a->c += (a->s - t) + v;
        } else {
            a->c += (v - t) + a->s;
        }
    }
    a->s = t;
}

static double nsum_value(const nsum_t* a) { return a->s + a->c; }

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void orc_bf16_to_double(int64_t n, const uint16_t* bits, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits_to_double(bits[i]);
}

/*
 * BF16 has 8 significant bits and the FP32 exponent range. Round-to-nearest-
 * even straight from the double, with one rounding: scale |v| by the BF16
 * quantum of its binade (an exact power-of-two scaling), round the quotient
 * to an integer with ties to even (rint in the default rounding mode), and
 * scale back. Values at or above the midpoint between the largest finite
 * BF16 and 2^128 round to infinity (the largest finite BF16 has an odd
 * significand, so a tie there goes up).
 */
static uint16_t double_to_bf16_bits(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int binade = e - 1;
    if (binade < -126) binade = -126; /* subnormal BF16: fixed quantum */
    double quantum = ldexp(1.0, binade - 7);
    double k = rint(a / quantum);
    double r = k * quantum; /* a BF16 value, exactly representable in FP32 */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

void orc_round_bf16(int64_t n, const double* v, uint16_t* bits) {
    for (int64_t i = 0; i < n; ++i) bits[i] = double_to_bf16_bits(v[i]);
}

void orc_round_f32(int64_t n, const double* v, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (float)v[i];
}

/*
 * One row of the forward on double inputs: returns rstd and writes y when
 * y is not NULL.
 */
static double row_fwd(int64_t H, const double* x, const double* w, double eps,
                      double* y) {
    nsum_t ss = {0.0, 0.0};
    for (int64_t j = 0; j < H; ++j) nsum_add(&ss, x[j] * x[j]);
    double ms = nsum_value(&ss) / (double)H;
    double rstd = 1.0 / sqrt(ms + eps);
    if (y) {
        for (int64_t j = 0; j < H; ++j) {
            double xhat = x[j] * rstd;
            y[j] = xhat * w[j];
        }
    }
    return rstd;
}

/*
 * One row of the backward on double inputs at the given rstd. Writes dx and
 * c when asked, and adds this row's dy*xhat into the per-column compensated
 * accumulators of dw.
 */
static void row_bwd(int64_t H, const double* dy, const double* x, double rstd,
                    const double* w, double* dx, double* c_out, nsum_t* dw_acc) {
    if (dx || c_out) {
        nsum_t dot = {0.0, 0.0};
        for (int64_t j = 0; j < H; ++j) {
            double xhat = x[j] * rstd;
            double g = dy[j] * w[j];
            nsum_add(&dot, g * xhat);
        }
        double c = nsum_value(&dot) / (double)H;
        if (c_out) *c_out = c;
        if (dx) {
            for (int64_t j = 0; j < H; ++j) {
                double xhat = x[j] * rstd;
                double g = dy[j] * w[j];
                dx[j] = rstd * (g - xhat * c);
            }
        }
    }
    for (int64_t j = 0; j < H; ++j) {
        double xhat = x[j] * rstd;
        nsum_add(&dw_acc[j], dy[j] * xhat);
    }
}

static void* xalloc(size_t n, size_t sz) {
    void* p = calloc(n ? n : 1, sz);
    if (!p) abort();
    return p;
}

void orc_fwd_f64(int64_t rows, int64_t H, const double* x, const double* w,
                 double eps, double* rstd_out, double* y_out) {
    for (int64_t t = 0; t < rows; ++t)
        rstd_out[t] = row_fwd(H, x + t * H, w, eps, y_out ? y_out + t * H : NULL);
}

void orc_bwd_f64(int64_t rows, int64_t H, const double* dy, const double* x,
                 const double* rstd, const double* w, double* dx_out,
                 double* c_out, double* dw_out) {
    nsum_t* acc = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    for (int64_t t = 0; t < rows; ++t)
        row_bwd(H, dy + t * H, x + t * H, rstd[t], w, dx_out ? dx_out + t * H : NULL,
                c_out ? c_out + t : NULL, acc);
    for (int64_t j = 0; j < H; ++j) dw_out[j] = nsum_value(&acc[j]);
    free(acc);
}

/* BF16 entry points: widen one row at a time (exactly) and run the same rows. */
void orc_fwd(int64_t rows, int64_t H, const uint16_t* x, const double* w,
             double eps, double* rstd_out, double* y_out) {
    double* xr = (double*)xalloc((size_t)H, sizeof(double));
    for (int64_t t = 0; t < rows; ++t) {
        orc_bf16_to_double(H, x + t * H, xr);
        rstd_out[t] = row_fwd(H, xr, w, eps, y_out ? y_out + t * H : NULL);
    }
    free(xr);
}

void orc_bwd(int64_t rows, int64_t H, const uint16_t* dy, const uint16_t* x,
             const double* rstd, const double* w, double* dx_out,
             double* c_out, double* dw_out) {
    nsum_t* acc = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    double* xr = (double*)xalloc((size_t)H, sizeof(double));
    double* dyr = (double*)xalloc((size_t)H, sizeof(double));
    for (int64_t t = 0; t < rows; ++t) {
        orc_bf16_to_double(H, x + t * H, xr);
        orc_bf16_to_double(H, dy + t * H, dyr);
        row_bwd(H, dyr, xr, rstd[t], w, dx_out ? dx_out + t * H : NULL,
                c_out ? c_out + t : NULL, acc);
    }
    for (int64_t j = 0; j < H; ++j) dw_out[j] = nsum_value(&acc[j]);
    free(dyr);
    free(xr);
    free(acc);
}

/*
 * The sum of two BF16 values is formed in double. It is exact unless the
 * exponents differ by more than the double significand can span, and in that
 * case the smaller term is far below half a BF16 ulp of the larger, so the
 * rounded result is the same. One rounding to BF16 follows.
 */
void orc_residual_add(int64_t n, const uint16_t* x, const uint16_t* r,
                      uint16_t* h_out) {
    for (int64_t i = 0; i < n; ++i) {
        double s = bf16_bits_to_double(x[i]) + bf16_bits_to_double(r[i]);
        h_out[i] = double_to_bf16_bits(s);
    }
}

/* ------------------------------------------------------------ LayerNorm
 *
 * The adjacent normalisation in the same training stacks (ROCm
 * TransformerEngine PR "Microbenchmarking and CI performance regression
 * test", benchmark_normalization table: RMSNorm and LayerNorm forward and
 * backward on MI355). The usual definition, per row:
 *
 *   forward   mu = (1/H) sum_j x_j,  var = (1/H) sum_j (x_j - mu)^2,
 *             rstd = 1/sqrt(var + eps),  xhat = (x - mu) * rstd,
 *             y = xhat * gamma + beta
 *   backward  g = dy * gamma,  c1 = (1/H) sum_j g_j,
 *             c2 = (1/H) sum_j g_j * xhat_j,
 *             dx = rstd * (g - c1 - xhat * c2)
 *             dgamma_j = sum_t dy_tj * xhat_tj,  dbeta_j = sum_t dy_tj
 *
 * The variance is the two-pass one (deviations from the mean), as a plain
 * reading of the definition.
 */

static void ln_row_fwd(int64_t H, const double* x, const double* gamma, const double* beta,
                       double eps, double* mu_out, double* rstd_out, double* y) {
    nsum_t s = {0.0, 0.0};
    for (int64_t j = 0; j < H; ++j) nsum_add(&s, x[j]);
    double mu = nsum_value(&s) / (double)H;
    nsum_t v = {0.0, 0.0};
    for (int64_t j = 0; j < H; ++j) nsum_add(&v, (x[j] - mu) * (x[j] - mu));
    double var = nsum_value(&v) / (double)H;
    double rstd = 1.0 / sqrt(var + eps);
    *mu_out = mu;
    *rstd_out = rstd;
    if (y) {
        for (int64_t j = 0; j < H; ++j) {
            double xhat = (x[j] - mu) * rstd;
            y[j] = xhat * gamma[j] + (beta ? beta[j] : 0.0);
        }
    }
}

static void ln_row_bwd(int64_t H, const double* dy, const double* x, double mu, double rstd,
                       const double* gamma, double* dx, double* c_out, nsum_t* dg_acc,
                       nsum_t* db_acc) {
    if (dx || c_out) {
        nsum_t s1 = {0.0, 0.0}, s2 = {0.0, 0.0};
        for (int64_t j = 0; j < H; ++j) {
            double xhat = (x[j] - mu) * rstd;
            double g = dy[j] * gamma[j];
            nsum_add(&s1, g);
            nsum_add(&s2, g * xhat);
        }
        double c1 = nsum_value(&s1) / (double)H;
        double c2 = nsum_value(&s2) / (double)H;
        if (c_out) {
            c_out[0] = c1;
            c_out[1] = c2;
        }
        if (dx) {
            for (int64_t j = 0; j < H; ++j) {
                double xhat = (x[j] - mu) * rstd;
                double g = dy[j] * gamma[j];
                dx[j] = rstd * (g - c1 - xhat * c2);
            }
        }
    }
    for (int64_t j = 0; j < H; ++j) {
        double xhat = (x[j] - mu) * rstd;
        nsum_add(&dg_acc[j], dy[j] * xhat);
        nsum_add(&db_acc[j], dy[j]);
    }
}

void orc_ln_fwd_f64(int64_t rows, int64_t H, const double* x, const double* gamma,
                    const double* beta, double eps, double* mu_out, double* rstd_out,
                    double* y_out) {
    for (int64_t t = 0; t < rows; ++t)
        ln_row_fwd(H, x + t * H, gamma, beta, eps, mu_out + t, rstd_out + t,
                   y_out ? y_out + t * H : NULL);
}

void orc_ln_bwd_f64(int64_t rows, int64_t H, const double* dy, const double* x,
                    const double* mu, const double* rstd, const double* gamma, double* dx_out,
                    double* c_out, double* dgamma_out, double* dbeta_out) {
    nsum_t* dg = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    nsum_t* db = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    for (int64_t t = 0; t < rows; ++t)
        ln_row_bwd(H, dy + t * H, x + t * H, mu[t], rstd[t], gamma,
                   dx_out ? dx_out + t * H : NULL, c_out ? c_out + 2 * t : NULL, dg, db);
    for (int64_t j = 0; j < H; ++j) {
        dgamma_out[j] = nsum_value(&dg[j]);
        dbeta_out[j] = nsum_value(&db[j]);
    }
    free(db);
    free(dg);
}

void orc_ln_fwd(int64_t rows, int64_t H, const uint16_t* x, const double* gamma,
                const double* beta, double eps, double* mu_out, double* rstd_out,
                double* y_out) {
    double* xr = (double*)xalloc((size_t)H, sizeof(double));
    for (int64_t t = 0; t < rows; ++t) {
        orc_bf16_to_double(H, x + t * H, xr);
        ln_row_fwd(H, xr, gamma, beta, eps, mu_out + t, rstd_out + t,
                   y_out ? y_out + t * H : NULL);
    }
    free(xr);
}

void orc_ln_bwd(int64_t rows, int64_t H, const uint16_t* dy, const uint16_t* x,
                const double* mu, const double* rstd, const double* gamma, double* dx_out,
                double* c_out, double* dgamma_out, double* dbeta_out) {
    nsum_t* dg = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    nsum_t* db = (nsum_t*)xalloc((size_t)H, sizeof(nsum_t));
    double* xr = (double*)xalloc((size_t)H, sizeof(double));
    double* dyr = (double*)xalloc((size_t)H, sizeof(double));
    for (int64_t t = 0; t < rows; ++t) {
        orc_bf16_to_double(H, x + t * H, xr);
        orc_bf16_to_double(H, dy + t * H, dyr);
        ln_row_bwd(H, dyr, xr, mu[t], rstd[t], gamma, dx_out ? dx_out + t * H : NULL,
                   c_out ? c_out + 2 * t : NULL, dg, db);
    }
    for (int64_t j = 0; j < H; ++j) {
        dgamma_out[j] = nsum_value(&dg[j]);
        dbeta_out[j] = nsum_value(&db[j]);
    }
    free(dyr);
    free(xr);
    free(db);
    free(dg);
}
