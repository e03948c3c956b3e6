/*
 * FP64 CPU oracle for RMSNorm training (forward, backward, fused residual).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no source with the HIP
 * library.
 *
 * What it follows (flashinfer PR "fix(cake_rmsnorm): sm_100a and sm_107a
 * dw-accuracy backward routes", opening description): the forward of
 * RMSNorm-for-training returns y and rstd, the backward returns dx and dw;
 * the fused residual form first forms h_new = BF16(h + u) (same page, "Key"
 * paragraph); accuracy is judged against FP64 ("Changed windows by reason").
 *
 * Layout: every array is contiguous row-major [rows, H]; a per-head view is
 * flattened by the caller so that row r = t * heads + head. BF16 tensors are
 * passed as their 16-bit patterns and widened exactly. w is passed widened
 * to double (BF16 and FP32 values are exact in FP64).
 */
#ifndef RMSNORM_ORACLE_H
#define RMSNORM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact widening of BF16 bit patterns to double. */
void orc_bf16_to_double(int64_t n, const uint16_t* bits, double* out);

/* Round doubles to BF16, round-to-nearest-even, one rounding. */
void orc_round_bf16(int64_t n, const double* v, uint16_t* bits);

/* Round doubles to FP32, round-to-nearest-even. */
void orc_round_f32(int64_t n, const double* v, float* out);

/* Forward. For each row: rstd = 1/sqrt(mean(x^2) + eps), y = (x*rstd)*w.
 * x: BF16 bits [rows, H]; w: [H]; rstd_out: [rows]; y_out: [rows, H] or NULL. */
void orc_fwd(int64_t rows, int64_t H, const uint16_t* x, const double* w,
             double eps, double* rstd_out, double* y_out);

/* Backward at a given rstd (the caller chooses FP64-recomputed or the
 * forward's FP32 value). For each row t:
 *   xhat = x*rstd, g = dy*w, c_t = (1/H) sum_j g*xhat,
 *   dx = rstd*(g - xhat*c_t)
 * and dw_j = sum over all rows of dy*xhat (compensated, rows in order).
 * dx_out and c_out may be NULL (dw-only pass over large inputs). */
void orc_bwd(int64_t rows, int64_t H, const uint16_t* dy, const uint16_t* x,
             const double* rstd, const double* w, double* dx_out,
             double* c_out, double* dw_out);

/* The same forward and backward on double inputs (used with unrounded
 * inputs, e.g. for finite-difference checks). */
void orc_fwd_f64(int64_t rows, int64_t H, const double* x, const double* w,
                 double eps, double* rstd_out, double* y_out);
void orc_bwd_f64(int64_t rows, int64_t H, const double* dy, const double* x,
                 const double* rstd, const double* w, double* dx_out,
                 double* c_out, double* dw_out);

/* Residual pre-step: h = BF16(x + r), as bits. */
void orc_residual_add(int64_t n, const uint16_t* x, const uint16_t* r,
                      uint16_t* h_out);

/* LayerNorm (the adjacent normalisation of the same benchmark suite: ROCm
 * TransformerEngine PR "Microbenchmarking and CI performance regression
 * test", benchmark_normalization). Forward per row: mu = mean(x),
 * var = mean((x - mu)^2), rstd = 1/sqrt(var + eps),
 * y = (x - mu)*rstd*gamma + beta (beta may be NULL: zero). */
void orc_ln_fwd(int64_t rows, int64_t H, const uint16_t* x, const double* gamma,
                const double* beta, double eps, double* mu_out, double* rstd_out,
                double* y_out);
/* Backward at given mu and rstd: xhat = (x - mu)*rstd, g = dy*gamma,
 * c1 = mean(g), c2 = mean(g*xhat), dx = rstd*(g - c1 - xhat*c2);
 * dgamma_j = sum_t dy*xhat, dbeta_j = sum_t dy. c_out (nullable) receives
 * [c1, c2] per row; dx_out may be NULL. */
void orc_ln_bwd(int64_t rows, int64_t H, const uint16_t* dy, const uint16_t* x,
                const double* mu, const double* rstd, const double* gamma, double* dx_out,
                double* c_out, double* dgamma_out, double* dbeta_out);
void orc_ln_fwd_f64(int64_t rows, int64_t H, const double* x, const double* gamma,
                    const double* beta, double eps, double* mu_out, double* rstd_out,
                    double* y_out);
void orc_ln_bwd_f64(int64_t rows, int64_t H, const double* dy, const double* x,
                    const double* mu, const double* rstd, const double* gamma, double* dx_out,
                    double* c_out, double* dgamma_out, double* dbeta_out);

#ifdef __cplusplus
}
#endif

#endif
