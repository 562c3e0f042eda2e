/*
 * rmsnorm_tuning.h -- development hook of librmsnorm.so for launch-geometry
 * sweeps and for tests that must reach every kernel path at small sizes.
 * Not needed for normal use: without it the library picks the geometry
 * itself from H, the storage format and the device.
 *
 * The override changes which threads handle which elements, and therefore
 * the order of the float32 sums, but never what is computed.  It is
 * process-wide; set it only while no other thread is calling the library.
 */
#ifndef RMSNORM_TUNING_H
#define RMSNORM_TUNING_H

#include <stdint.h>

#include "rmsnorm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * which = 0: forward and fused residual.  A row is owned by wpr waves of 64
 *            threads, each thread holding vpt 16-byte vectors (single elements
 *            when rows are not 16-byte aligned); third = rows per workgroup;
 *            grid > 0 caps the number of workgroups (they then walk the rows
 *            grid-stride), 0 = one workgroup per group of rows.
 * which = 1: backward.  vpt and wpr as above (one row per workgroup at a
 *            time); third = number of workgroups P, each owning one row of
 *            dw partial sums (0 = default); grid selects which rows a
 *            workgroup owns: 0 = default, 1 = interleaved (b, b+P, ...),
 *            2 = a contiguous block.
 * which = 2: RoPE apply.  vpt = wpr = 1 sets the override; third = 1 forces
 *            the split layout (each thread reads both halves of a head)
 *            instead of the lane exchange; grid > 0 caps the number of
 *            workgroups along the positions (they then walk the position
 *            blocks grid-stride), 0 = one workgroup per block.
 * vpt <= 0 or wpr <= 0 clears the override.  A tile too small for the row
 * takes the two-pass path, which requires vpt = 4 (8 for single elements).
 * An override the shape cannot use makes the call fail with
 * RMSN_ERR_INVALID_ARG.
 */
void rmsnorm_tuning_set_geometry(int which, int vpt, int wpr, int third, int64_t grid);

/*
 * Host only (touches no device): the tile a call takes with no forced
 * geometry.  op: 0 RMSNorm forward, 1 fused residual, 2 AdaLN, 3 LayerNorm,
 * 4 backward, 5 residual backward, 6 LayerNorm fused with the residual add.  layout 0: every row start 16-byte
 * aligned; 1: row starts only element-aligned (parameters 16-byte aligned);
 * 2: as 1, with every row stream of the call (x, dy, dres, dx) at one shared
 * offset within its 16-byte chunks, the same for every row a backward
 * workgroup owns (the backward then sets its vectors on memory's 16-byte
 * grid; the forward ops take layout 1's tile).
 * The parameters (weight, AdaLN's rows, LayerNorm's bias) are taken in x's
 * format; a float32 weight on 16-bit data can give another tile (a smaller
 * register budget).  Writes out[0] elements per access, out[1] accesses per thread, out[2] waves
 * per row, out[3] rows per workgroup, out[4] 1 when rows off the 16-byte grid
 * take 16-byte vectors at each row's byte offset, 2 when a backward takes
 * them on memory's 16-byte grid (layout 2, one pass; the tile then covers the
 * one more vector such a row may touch), 0 for single elements or rows on
 * the grid, out[5] 1 when the row takes the multi-pass path (out[1] and
 * out[2] are then 0).  RMSN_ERR_INVALID_ARG for a bad op, layout, H or a NULL
 * out; RMSN_ERR_UNSUPPORTED for an unknown format or H > 2^30.
 */
rmsn_status_t rmsnorm_tuning_tile(int op, int64_t H, rmsn_dtype_t x_dtype, int layout, int32_t out[6]);

/*
 * Streaming accesses: the (M, H) inputs and outputs can be read and written
 * with non-temporal hints, which keep them out of the caches.  mode < 0 (the
 * default) streams when a call moves at least 64 MiB of such data, 0 never,
 * > 0 always.  Results are identical either way.
 */
void rmsnorm_tuning_set_streaming(int mode);

/*
 * Speed-of-light reference for measurements: copies `bytes` from src to dst
 * (device pointers, 2-byte aligned, bytes a multiple of 16, the two ranges
 * disjoint) with the forward kernels' access pattern -- 256-thread
 * workgroups, two 16-byte vectors per thread, non-temporal loads and stores
 * -- and no arithmetic, so that a kernel's HBM rate can be compared with the
 * rate of moving the same bytes in the same way.  When src and dst are both
 * 16-byte aligned every access is an aligned 16-byte one; otherwise every
 * access is a 16-byte access at the element-aligned address, as the kernels
 * for rows off the 16-byte grid make.  Enqueued on `stream`; returns
 * RMSN_ERR_INVALID_ARG for a bad argument.
 */
rmsn_status_t rmsnorm_tuning_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_TUNING_H */
