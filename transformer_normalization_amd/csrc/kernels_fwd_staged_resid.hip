// kernels_fwd_staged_resid.hip -- instantiations of the staged forward
// (staged_kernels.hpp) for the fused residual pre-norm.
#include "kernel_tables.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, bool NT>
fwd_fn staged_for(int vpt) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    constexpr bool R = true;
    switch (vpt) {
    case 1: return rmsnorm_fwd_staged_kernel<XDT, WDT, 1, R, NT, fwd_max_threads(1 * V, R ? 1 : 0)>;
    case 2: return rmsnorm_fwd_staged_kernel<XDT, WDT, 2, R, NT, fwd_max_threads(2 * V, R ? 1 : 0)>;
    case 3: return rmsnorm_fwd_staged_kernel<XDT, WDT, 3, R, NT, fwd_max_threads(3 * V, R ? 1 : 0)>;
    case 4: return rmsnorm_fwd_staged_kernel<XDT, WDT, 4, R, NT, fwd_max_threads(4 * V, R ? 1 : 0)>;
    case 6: return rmsnorm_fwd_staged_kernel<XDT, WDT, 6, R, NT, fwd_max_threads(6 * V, R ? 1 : 0)>;
    default: return nullptr;
    }
}

template <bool NT>
fwd_fn staged_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return staged_for<DT_F32, DT_F32, NT>(vpt);
    case RMSN_F16: return wf32 ? staged_for<DT_F16, DT_F32, NT>(vpt) : staged_for<DT_F16, DT_F16, NT>(vpt);
    case RMSN_BF16: return wf32 ? staged_for<DT_BF16, DT_F32, NT>(vpt) : staged_for<DT_BF16, DT_BF16, NT>(vpt);
    default: return nullptr;
    }
}

}  // namespace

fwd_fn fwd_staged_lookup_resid(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool nt) {
    return nt ? staged_nt<true>(xdt, wdt, vpt) : staged_nt<false>(xdt, wdt, vpt);
}

}  // namespace rmsn
