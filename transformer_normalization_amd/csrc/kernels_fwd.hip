// kernels_fwd.hip -- instantiations of the plain forward kernels (fwd_kernels.hpp).
#include "fwd_table.hpp"

namespace rmsn {

fwd_fn fwd_lookup_plain(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt) {
    return nt ? tables::fwd_lookup_nt<MODE_PLAIN, true>(xdt, wdt, vec, vpt, two_pass)
              : tables::fwd_lookup_nt<MODE_PLAIN, false>(xdt, wdt, vec, vpt, two_pass);
}

}  // namespace rmsn
