// kernels_ln_staged.hip -- instantiations of the staged LayerNorm
// (staged_kernels.hpp), plain and fused with the residual add.
#include "kernel_tables.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, bool R, bool NT>
ln_fn staged_for(int vpt) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    switch (vpt) {
    case 1: return layernorm_fwd_staged_kernel<XDT, WDT, 1, R, NT, ln_max_threads(1 * V)>;
    case 2: return layernorm_fwd_staged_kernel<XDT, WDT, 2, R, NT, ln_max_threads(2 * V)>;
    case 3: return layernorm_fwd_staged_kernel<XDT, WDT, 3, R, NT, ln_max_threads(3 * V)>;
    case 4: return layernorm_fwd_staged_kernel<XDT, WDT, 4, R, NT, ln_max_threads(4 * V)>;
    case 6: return layernorm_fwd_staged_kernel<XDT, WDT, 6, R, NT, ln_max_threads(6 * V)>;
    default: return nullptr;
    }
}

template <bool R, bool NT>
ln_fn staged_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return staged_for<DT_F32, DT_F32, R, NT>(vpt);
    case RMSN_F16: return wf32 ? staged_for<DT_F16, DT_F32, R, NT>(vpt) : staged_for<DT_F16, DT_F16, R, NT>(vpt);
    case RMSN_BF16: return wf32 ? staged_for<DT_BF16, DT_F32, R, NT>(vpt) : staged_for<DT_BF16, DT_BF16, R, NT>(vpt);
    default: return nullptr;
    }
}

}  // namespace

ln_fn ln_staged_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool nt, bool resid) {
    if (resid) return nt ? staged_nt<true, true>(xdt, wdt, vpt) : staged_nt<true, false>(xdt, wdt, vpt);
    return nt ? staged_nt<false, true>(xdt, wdt, vpt) : staged_nt<false, false>(xdt, wdt, vpt);
}

}  // namespace rmsn
