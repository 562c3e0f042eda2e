/*
 * rope.h -- C ABI of the MI355X (gfx950) RoPE apply step, in the same library
 * as rmsnorm.h (librmsnorm.so) and with its status codes and conventions:
 * device pointers on the current HIP device, strides in ELEMENTS, nothing
 * allocated, freed or synchronised, argument errors found on the host before
 * any HIP call, results identical on every run.
 *
 * The operation is the rotate-half rotary embedding of the page "rocm-kernels"
 * (skillselion.com), "Core Kernel Implementations", 2. RoPE 3D, and "Triton
 * kernel templates", Template 2: q or k laid out [batch, seq_len, heads,
 * head_dim] is rotated in pairs (element j with element j + head_dim/2) by
 * the angle whose cosine and sine the caller has tabulated per position in
 * [seq_len, head_dim] tables.  For video the positions are the t*h*w latent
 * patches and the tables carry the temporal and spatial frequencies; the
 * apply step is the same.  With the batch folded into the rows, row r reads
 * table row r mod seq_len (the same page, "Common Pitfalls", 7: reading row r
 * itself runs past the tables when batch > 1).
 *
 * For token row r = b * seq_len + s, head h and j < head_dim / 2, with
 * x0 = x[r, h, j], x1 = x[r, h, j + head_dim/2], c = cos[s, j], sn = sin[s, j]
 * (sn = -sin[s, j] when transpose != 0), in float32:
 *
 *   out[r, h, j]              = x0 * c - x1 * sn
 *   out[r, h, j + head_dim/2] = x1 * c + x0 * sn
 *
 * each rounded once to x_dtype (nearest even); the product with c is fused
 * with the sum (one fma each: fma(x0, c, x1 * -sn) and fma(x1, c, x0 * sn)).
 * Only the first head_dim/2 columns of a table row are read: the rotate-half
 * layout repeats the same angles in both halves, so [seq_len, head_dim/2]
 * tables work too.  The transposed rotation
 * is the inverse rotation and the gradient of the rotation with respect to x.
 */
#ifndef ROPE_H
#define ROPE_H

#include <stddef.h>
#include <stdint.h>

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   x            input; token row r = b * seq_len + s starts at
 *                x + r * x_row_stride, head h at + h * x_head_stride, and the
 *                head_dim elements of a head are contiguous.
 *   cos, sin     (seq_len, >= head_dim/2) tables, rows table_stride elements
 *                apart (the same stride for both), in table_dtype.
 *   out          output laid out as x with its own strides; it may be x itself
 *                (same pointer and strides).  Every other overlap of the byte
 *                ranges spanned by out and an input is rejected.
 *   batch        >= 0 (0 enqueues nothing); seq_len >= 1; num_heads >= 1;
 *   head_dim     even, 2 .. 65536.
 *   strides      head strides >= head_dim; row strides >= (num_heads - 1) *
 *                head stride + head_dim; table_stride >= head_dim / 2.
 *   transpose    0: rotate by the tabulated angle; nonzero: by its negative.
 *   x_dtype      RMSN_F32, RMSN_F16 or RMSN_BF16 (also the output format);
 *   table_dtype  x_dtype or RMSN_F32.
 */
rmsn_status_t rope_apply(const void *x, int64_t x_row_stride, int64_t x_head_stride, const void *cos,
                         const void *sin, int64_t table_stride, void *out, int64_t out_row_stride,
                         int64_t out_head_stride, int64_t batch, int64_t seq_len, int64_t num_heads,
                         int64_t head_dim, int transpose, rmsn_dtype_t x_dtype, rmsn_dtype_t table_dtype,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_H */
