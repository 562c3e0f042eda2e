// kernels_fwd_residual.hip -- instantiations of the fused residual pre-norm kernels (fwd_kernels.hpp).
#include "fwd_table.hpp"

namespace rmsn {

fwd_fn fwd_lookup_resid(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt) {
    return nt ? tables::fwd_lookup_nt<MODE_RESID, true>(xdt, wdt, vec, vpt, two_pass)
              : tables::fwd_lookup_nt<MODE_RESID, false>(xdt, wdt, vec, vpt, two_pass);
}

}  // namespace rmsn
