// kernel_tables.hpp -- lookup of kernel instantiations by format and tile.
// Each kernel family is instantiated in its own translation unit
// (kernels_fwd.hip, kernels_fwd_residual.hip, kernels_adaln.hip,
// kernels_fwd_mis.hip, kernels_bwd.hip, kernels_bwd_residual.hip, kernels_bwd_mis.hip,
// kernels_rope.hip, kernels_ln.hip,
// kernels_ln_mis.hip)
// so that they compile in parallel; the host code only sees these functions.
#pragma once

#include "bwd_kernels.hpp"
#include "fwd_kernels.hpp"
#include "ln_kernels.hpp"
#include "rmsnorm.h"
#include "rope_kernels.hpp"

namespace rmsn {

typedef void (*fwd_fn)(const FwdParams);
typedef void (*bwd_fn)(const BwdParams);
typedef void (*rope_fn)(const RopeParams);
typedef void (*ln_fn)(const LnParams);

// nullptr when no instantiation matches (vec: elements per access; vpt:
// accesses per thread; nt: streaming accesses)
fwd_fn fwd_lookup_plain(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt);
fwd_fn fwd_lookup_resid(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt);
// the forward for rows off the 16-byte grid (16-byte vectors at the row's
// byte offset; mode: MODE_PLAIN, MODE_RESID or MODE_ADALN), resident or, for
// rows longer than a tile, in two passes (vpt 4)
fwd_fn fwd_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, int mode, bool nt);
// AdaLN: wdt is the format of the weight, scale and shift
fwd_fn fwd_lookup_adaln(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt);
// deep: the one-vector tile with three rows prefetched per wave (rmsnorm_bwd_kernel's DEEP)
bwd_fn bwd_lookup_plain(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt, bool deep);
// the backward of the fused residual pre-norm (adds the residual-stream gradient)
bwd_fn bwd_lookup_res(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt);
// the backward for rows off the 16-byte grid (16-byte vectors at the row's
// byte offset; x, dy, dres and dx element-aligned, w 16-byte aligned), one
// pass or, for rows longer than a tile, two (vpt 4)
bwd_fn bwd_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, bool res, bool nt, bool deep);
const void *dw_finalize_kernel();
// vec: 16 / element size, or 1 for single elements; tdt: x's format or
// float32; xchg: the lane-exchange layout (vectors only)
// LayerNorm forward, plain or fused with the residual add (resid)
ln_fn ln_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt, bool resid);
// LayerNorm for rows off the 16-byte grid in 16-byte vectors at the row's
// byte offset, resident or, for rows longer than a tile, in passes (vpt 4)
ln_fn ln_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, bool nt, bool resid);
rope_fn rope_lookup(rmsn_dtype_t xdt, rmsn_dtype_t tdt, int vec, bool nt, bool xchg);

}  // namespace rmsn
