/*
 * rmsnorm.h -- C ABI of the MI355X (gfx950) RMSNorm library.
 *
 * RMSNorm over the trailing (hidden) dimension of an (M, H) row-major matrix:
 *
 *     y[i, j] = x[i, j] * rrms[i] * w[j],   rrms[i] = 1 / sqrt(sum_j x[i, j]^2 / H + eps)
 *
 * as defined on the page "Skill: Write a Triton RMSNorm Kernel" (ahel.ai),
 * section "Purpose" and "Required reasoning process" steps 1-10: the mean
 * divides by the full row length H, eps sits inside the square root, the
 * weight has shape (H,) and is indexed by column only, there is no bias and
 * no mean subtraction, squares and sums are taken in float32 whatever the
 * storage format.  The weightless form (w == NULL, y = x * rrms) follows the
 * page "rocm-kernels" (skillselion.com), "Core Kernel Implementations",
 * RMSNorm, where LTX-Video's norms carry no weight.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are row-major (M, H) with unit stride along H.  *_stride
 *    arguments are the distance between consecutive rows, in ELEMENTS, and
 *    must be >= H.  Rows may be padded (stride > H) or be a strided view.
 *  - Every data pointer is a DEVICE pointer on the current HIP device
 *    (hipGetDevice).  The caller owns all memory.  The library never
 *    allocates, frees or synchronises; it only validates the arguments and
 *    enqueues kernels on `stream` (0 = the null stream), so results are ready
 *    when that stream reaches them.
 *  - x_dtype is the storage format of every (M, H) matrix of a call; outputs
 *    are written in that same format, rounded to nearest even.  w_dtype is
 *    the weight's format: either x_dtype or RMSN_F32.  rrms and dw are
 *    always float32.
 *  - M == 0 is valid and enqueues nothing (after the other arguments pass
 *    validation), except that rmsnorm_bwd with dw != NULL writes dw = 0,
 *    the sum over zero rows.
 *  - An output may be the very same buffer as an input of the same shape
 *    (same pointer and same stride; e.g. y == x): every element is read
 *    before it is written.  Any other overlap between an output and another
 *    buffer of the call is rejected with RMSN_ERR_INVALID_ARG.
 *  - Argument errors are detected on the host before any HIP call, so they
 *    are reported without touching the device.  RMSN_ERR_HIP reports a failed
 *    device query or kernel launch (asynchronous faults surface later, on
 *    the stream, as with any HIP kernel).  rmsnorm_last_error() returns a
 *    message for the most recent failure on the calling thread.
 *  - All entry points are thread-safe and keep no state between calls,
 *    apart from a per-device cache of the compute-unit count.  The one
 *    process-wide setting is the development override of rmsnorm_tuning.h,
 *    which is off unless a caller sets it through that header's functions
 *    (no environment variable or other input reaches it).
 *  - Results do not depend on the stream, on timing or on other calls: the
 *    same inputs in the same layout give the same bits on the same device.
 *    The order of the float32 sums follows the tile, which depends on H, the
 *    formats and whether rows sit on the 16-byte grid; a backward on rows off
 *    it whose tensors share one offset within their 16-byte blocks also
 *    follows that offset.  Other layouts of the same values may then differ
 *    in the last bits, within the same tolerances; so may a tile forced
 *    through rmsnorm_tuning_set_geometry().
 */
#ifndef RMSNORM_H
#define RMSNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums are int-sized, and their two range markers make every int value
 * a valid value of the type (also in C++, where a value outside an enum's
 * range is undefined): a caller may pass any int, and the library rejects
 * the ones it does not know with RMSN_ERR_UNSUPPORTED instead of misbehaving.
 * The markers are never valid arguments. */
typedef enum {
    RMSN_F32 = 0,  /* IEEE binary32 */
    RMSN_F16 = 1,  /* IEEE binary16 */
    RMSN_BF16 = 2, /* bfloat16 (upper half of a binary32) */
    RMSN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    RMSN_DTYPE_RANGE_MAX_ = 2147483647
} rmsn_dtype_t;

typedef enum {
    RMSN_OK = 0,
    RMSN_ERR_INVALID_ARG = 1, /* NULL required pointer, bad size/stride/eps, overlap */
    RMSN_ERR_UNSUPPORTED = 2, /* dtype combination, H too large, device not gfx950 */
    RMSN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    RMSN_ERR_HIP = 4,         /* device query or kernel launch failed */
    RMSN_STATUS_RANGE_MIN_ = -2147483647 - 1,
    RMSN_STATUS_RANGE_MAX_ = 2147483647
} rmsn_status_t;

/*
 * Forward RMSNorm ("Skill: Write a Triton RMSNorm Kernel", "Required reasoning
 * process" steps 1-10; weightless form: "rocm-kernels", "Core Kernel
 * Implementations").
 *
 *   x     (M, H) input, rows x_stride elements apart.
 *   w     (H,) weight, contiguous, or NULL for the weightless norm.
 *   y     (M, H) output, rows y_stride elements apart; may equal x (same
 *         pointer and stride).
 *   rrms  (M,) float32 output of the per-row 1/sqrt(mean(x^2) + eps) -- the
 *         statistic the backward pass reads (step 10) -- or NULL.
 *   eps   > 0 and finite; added inside the square root.
 *   H     >= 1 and <= 2^30.
 */
rmsn_status_t rmsnorm_fwd(const void *x, int64_t x_stride, const void *w, void *y,
                          int64_t y_stride, float *rrms, int64_t M, int64_t H, float eps,
                          rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream);

/*
 * Fused residual pre-norm ("Skill: Write a Triton RMSNorm Kernel", "Use this
 * when" and "Kernel design rules": the residual is added in float32 after
 * both inputs are widened and before squaring; the post-add sum may be
 * written back as the next residual stream).
 *
 *   h[i, j]            = float32(x[i, j]) + float32(residual[i, j])
 *   residual_out[i, j] = h[i, j] rounded to x_dtype (nearest even)
 *   y                  = RMSNorm of the UNROUNDED h, as rmsnorm_fwd
 *
 *   residual      (M, H) input, rows r_stride apart.
 *   residual_out  (M, H) output, rows ro_stride apart, or NULL to skip the
 *                 write-back; may equal residual or x (same pointer/stride).
 *   y, w, rrms, eps, M, H  as rmsnorm_fwd; y may equal x or residual.
 */
rmsn_status_t rmsnorm_fwd_residual(const void *x, int64_t x_stride, const void *residual,
                                   int64_t r_stride, const void *w, void *y, int64_t y_stride,
                                   void *residual_out, int64_t ro_stride, float *rrms, int64_t M,
                                   int64_t H, float eps, rmsn_dtype_t x_dtype,
                                   rmsn_dtype_t w_dtype, hipStream_t stream);

/*
 * AdaLN-RMSNorm, the DiT conditioning step fused with the norm ("rocm-kernels",
 * "Core Kernel Implementations", 4. AdaLN, and "Triton kernel templates",
 * Template 4: norm(x) * weight * (1 + scale) + shift):
 *
 *   y[i, j] = (x[i, j] * rrms[i]) * w[j] * (1 + scale[c, j]) + shift[c, j],
 *   c = i / rows_per_cond
 *
 * rows_per_cond = 1 gives one conditioning row per row ([B, S, H] scale and
 * shift); rows_per_cond = S gives one per batch of S rows ([B, 1, H]).
 *
 *   scale, shift  (ceil(M / rows_per_cond), H), rows cond_stride elements
 *                 apart (both tensors share the stride, as when they are two
 *                 slices of one modulation tensor).
 *   w             (H,) weight or NULL.
 *   param_dtype   format of w, scale and shift: x_dtype or RMSN_F32.
 *   x, y, rrms, eps, M, H  as rmsnorm_fwd; the product with (1 + scale) and
 *                 the addition of shift are one float32 fused multiply-add.
 */
rmsn_status_t rmsnorm_adaln_fwd(const void *x, int64_t x_stride, const void *w, const void *scale,
                                const void *shift, int64_t cond_stride, int64_t rows_per_cond, void *y,
                                int64_t y_stride, float *rrms, int64_t M, int64_t H, float eps,
                                rmsn_dtype_t x_dtype, rmsn_dtype_t param_dtype, hipStream_t stream);

/*
 * Bytes of device workspace rmsnorm_bwd needs for (M, H) when a weight
 * gradient is requested (0 when M <= 0 or H <= 0): min(M, Pmax(H)) * H * 4,
 * where Pmax(H) = clamp(8 MiB / (4 H), 1024, 8192) is the most float32 rows
 * of partial column sums a call may use.  The value depends only on M and H,
 * never on the device, so it can be sized once per shape.
 */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t H);

/*
 * Backward RMSNorm ("Skill: Write a Triton RMSNorm Kernel", "Required
 * reasoning process" step 12, and "Correctness requirements": the saved rrms
 * is read, never recomputed).  With xn = x * rrms[i] and g = dy * w:
 *
 *   dx[i, j] = rrms[i] * g[i, j] - xn[i, j] * (rrms[i] / H) * sum_j g[i, j] * xn[i, j]
 *   dw[j]    = sum_i dy[i, j] * xn[i, j]          (shape (H,), float32)
 *
 *   dy, x     (M, H) inputs, rows dy_stride / x_stride apart.
 *   w         (H,) weight, or NULL for the weightless norm (then g = dy and dw
 *             must be NULL).
 *   rrms      (M,) float32 saved by the forward pass.
 *   dx        (M, H) output in x_dtype, rows dx_stride apart; may equal dy or
 *             x (same pointer and stride).
 *   dw        (H,) float32 output, OVERWRITTEN (not accumulated), or NULL to
 *             skip the weight gradient.  The column sums are reduced in a
 *             fixed order: no atomics, the same bits on every run.
 *   workspace device scratch of at least rmsnorm_bwd_workspace_bytes(M, H)
 *             bytes, 16-byte aligned (hipMalloc and torch allocations are),
 *             when dw != NULL (ignored otherwise).
 *             Its contents on entry do not matter; it must not overlap any
 *             other argument, and it must not be used by another call that
 *             may run at the same time.
 */
rmsn_status_t rmsnorm_bwd(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride,
                          const void *w, const float *rrms, void *dx, int64_t dx_stride, float *dw,
                          void *workspace, size_t workspace_bytes, int64_t M, int64_t H,
                          rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream);

/*
 * rmsnorm_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation, kernels and bits as rmsnorm_bwd, with no workspace
 * argument: the dw partial rows live in a static device array of this
 * library, 32 MiB, of which every device the library runs on holds one copy
 * until the process ends.  Nothing is allocated or freed by the call.
 *
 *   Arguments as rmsnorm_bwd.  The call needs P x H x 4 bytes of that array
 *   when dw != NULL, with P the number of partial rows rmsnorm_bwd takes for
 *   the shape on this device (256 for bf16 8192 x 6144 on a 256-CU MI355X: 6
 *   MiB); a call needing more than 32 MiB is rejected with
 *   RMSN_ERR_WORKSPACE before anything is enqueued.  With dw == NULL the
 *   array is not used.
 *   Every call on a device shares that device's array, and it keeps the last
 *   call's partial rows; each call writes every row it reads, so nothing has
 *   to be cleared.  Calls that may overlap in time on one device (other
 *   streams, other threads) race on the array: order them on one stream.
 */
rmsn_status_t rmsnorm_bwd_noalloc(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride,
                                  const void *w, const float *rrms, void *dx, int64_t dx_stride, float *dw,
                                  int64_t M, int64_t H, rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype,
                                  hipStream_t stream);

/*
 * Backward of the fused residual pre-norm.  Its forward (rmsnorm_fwd_residual)
 * computes h = x + residual, y = RMSNorm(h) and writes h back as the next
 * residual stream, so h reaches the loss twice: through y and through
 * residual_out.  By the chain rule through the sum, x and residual receive the
 * same gradient
 *
 *   dh[i, j] = dx[i, j] (as rmsnorm_bwd, with h in place of x) + dres[i, j]
 *
 * formed in float32 and rounded once.  (The page "Skill: Write a Triton
 * RMSNorm Kernel" gives the forward fusion, "Use this when" and "Kernel design
 * rules", and the norm's backward, step 12; the added term is the derivative
 * of the residual write-back.)
 *
 *   h         (M, H) the residual_out the forward wrote (the post-add stream
 *             as stored), rows h_stride apart.  The forward's rrms was
 *             computed from the unrounded sum; for float32 the two agree.
 *   dres      (M, H) gradient arriving on residual_out, rows dres_stride
 *             apart, or NULL when residual_out feeds nothing (then this call
 *             is rmsnorm_bwd).
 *   dh        (M, H) output, rows dh_stride apart; may equal dy, h or dres
 *             (same pointer and stride).
 *   dy, w, rrms, dw, workspace, workspace_bytes, M, H, dtypes
 *             as rmsnorm_bwd (the workspace size is the same).
 */
rmsn_status_t rmsnorm_bwd_residual(const void *dy, int64_t dy_stride, const void *h, int64_t h_stride,
                                   const void *dres, int64_t dres_stride, const void *w, const float *rrms,
                                   void *dh, int64_t dh_stride, float *dw, void *workspace,
                                   size_t workspace_bytes, int64_t M, int64_t H, rmsn_dtype_t x_dtype,
                                   rmsn_dtype_t w_dtype, hipStream_t stream);

/* Fixed text for a status code (never NULL). */
const char *rmsnorm_status_string(rmsn_status_t status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char *rmsnorm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_H */
