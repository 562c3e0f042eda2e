// kernels_bwd_residual.hip -- instantiations of the backward of the fused
// residual pre-norm (bwd_kernels.hpp with RES: the residual-stream gradient
// is added to dx).
#include "bwd_table.hpp"

namespace rmsn {

bwd_fn bwd_lookup_res(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt) {
    return nt ? tables::bwd_lookup_nt<true, true>(xdt, wdt, vec, vpt, two_pass, false)
              : tables::bwd_lookup_nt<true, false>(xdt, wdt, vec, vpt, two_pass, false);
}

}  // namespace rmsn
