/*
 * layernorm.h -- C ABI of the MI355X (gfx950) LayerNorm forward, plain and
 * fused with the residual add that precedes it, in the same library as
 * rmsnorm.h (librmsnorm.so) and with its status codes and conventions:
 * row-major (M, H) matrices with row strides in ELEMENTS, device pointers on
 * the current HIP device, nothing allocated, freed or synchronised, argument
 * errors found on the host before any HIP call, identical bits on every run;
 * an output may be the very same buffer as an input of the same shape, any
 * other overlap is rejected; M == 0 enqueues nothing.
 *
 * The page "SpeedROCm: shape-aware Triton acceleration for Transformer
 * inference" ("How the solution addresses the problem", item 4) fuses each
 * residual add of a pre-LayerNorm transformer with the LayerNorm that
 * consumes it.  LayerNorm is torch.nn's, which the same page lists among its
 * runtime interfaces: over the trailing dimension,
 *
 *   h     = x                         (layernorm_fwd)
 *   h     = float32(x) + float32(r)   (layernorm_fwd_residual; the sum is
 *                                      also written, rounded to x_dtype, to
 *                                      residual_out when that is not NULL)
 *   mean  = sum_j h[j] / H
 *   var   = sum_j (h[j] - mean)^2 / H       (population variance)
 *   rstd  = 1 / sqrt(var + eps)
 *   y[j]  = (h[j] - mean) * rstd * w[j] + b[j]
 *
 * in float32 from the unrounded h; the variance is taken about the computed
 * mean (a second reduction), never as a difference of mean squares; y is
 * formed as fma((h - mean) * rstd, w, b) and rounded once to x_dtype.
 *
 *   w, b        (H,) weight and bias, each optional (NULL = 1 and 0), both
 *               in w_dtype: x_dtype or RMSN_F32.
 *   mean, rstd  (M,) float32 per-row statistics, each optional (the inputs
 *               a backward pass would need).
 *   eps         > 0 and finite; H >= 1 and <= 2^30.
 */
#ifndef LAYERNORM_H
#define LAYERNORM_H

#include <stddef.h>
#include <stdint.h>

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

rmsn_status_t layernorm_fwd(const void *x, int64_t x_stride, const void *w, const void *b, void *y,
                            int64_t y_stride, float *mean, float *rstd, int64_t M, int64_t H, float eps,
                            rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream);

/*
 *   residual      (M, H) input, rows r_stride apart.
 *   residual_out  (M, H) output or NULL; may be residual or x itself.
 *   y             may be x or residual itself.
 */
rmsn_status_t layernorm_fwd_residual(const void *x, int64_t x_stride, const void *residual, int64_t r_stride,
                                     const void *w, const void *b, void *y, int64_t y_stride, void *residual_out,
                                     int64_t ro_stride, float *mean, float *rstd, int64_t M, int64_t H, float eps,
                                     rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LAYERNORM_H */
