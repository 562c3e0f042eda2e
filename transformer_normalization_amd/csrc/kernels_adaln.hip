// kernels_adaln.hip -- instantiations of the AdaLN-RMSNorm kernels (fwd_kernels.hpp).
#include "fwd_table.hpp"

namespace rmsn {

fwd_fn fwd_lookup_adaln(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt) {
    return nt ? tables::fwd_lookup_nt<MODE_ADALN, true>(xdt, wdt, vec, vpt, two_pass)
              : tables::fwd_lookup_nt<MODE_ADALN, false>(xdt, wdt, vec, vpt, two_pass);
}

}  // namespace rmsn
