// kernels_fwd_mis.hip -- instantiations of the forward (plain, fused residual
// and AdaLN) for rows off the 16-byte grid: 16-byte vectors read and written
// at the row's byte offset (fwd_kernels.hpp, MIS), resident or in two passes.
#include "kernel_tables.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, int MODE, bool NT>
fwd_fn mis_kernel(int vpt, bool tp) {
    // 2: x and its parameters are all 16-bit (the register budget)
    constexpr int ES2 = Fmt<XDT>::bytes == 2 && Fmt<WDT>::bytes == 2 ? 2 : 4;
    constexpr int V = 16 / Fmt<XDT>::bytes;
    if (tp) return vpt == 4 ? rmsnorm_fwd_kernel<XDT, WDT, V, 4, MODE, true, NT, 1024, true> : nullptr;
    switch (vpt) {
    case 1: return rmsnorm_fwd_kernel<XDT, WDT, V, 1, MODE, false, NT, fwd_max_threads(1 * V, MODE, ES2), true>;
    case 2: return rmsnorm_fwd_kernel<XDT, WDT, V, 2, MODE, false, NT, fwd_max_threads(2 * V, MODE, ES2), true>;
    case 3: return rmsnorm_fwd_kernel<XDT, WDT, V, 3, MODE, false, NT, fwd_max_threads(3 * V, MODE, ES2), true>;
    case 4: return rmsnorm_fwd_kernel<XDT, WDT, V, 4, MODE, false, NT, fwd_max_threads(4 * V, MODE, ES2), true>;
    case 6: return rmsnorm_fwd_kernel<XDT, WDT, V, 6, MODE, false, NT, fwd_max_threads(6 * V, MODE, ES2), true>;
    case 8: return rmsnorm_fwd_kernel<XDT, WDT, V, 8, MODE, false, NT, fwd_max_threads(8 * V, MODE, ES2), true>;
    default: break;
    }
    return nullptr;
}

template <int MODE, bool NT>
fwd_fn mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool tp) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return mis_kernel<DT_F32, DT_F32, MODE, NT>(vpt, tp);
    case RMSN_F16:
        return wf32 ? mis_kernel<DT_F16, DT_F32, MODE, NT>(vpt, tp) : mis_kernel<DT_F16, DT_F16, MODE, NT>(vpt, tp);
    case RMSN_BF16:
        return wf32 ? mis_kernel<DT_BF16, DT_F32, MODE, NT>(vpt, tp) : mis_kernel<DT_BF16, DT_BF16, MODE, NT>(vpt, tp);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

template <int MODE>
fwd_fn mis_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool tp, bool nt) {
    return nt ? mis_lookup<MODE, true>(xdt, wdt, vpt, tp) : mis_lookup<MODE, false>(xdt, wdt, vpt, tp);
}

}  // namespace

fwd_fn fwd_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, int mode, bool nt) {
    switch (mode) {
    case MODE_PLAIN: return mis_lookup_nt<MODE_PLAIN>(xdt, wdt, vpt, two_pass, nt);
    case MODE_RESID: return mis_lookup_nt<MODE_RESID>(xdt, wdt, vpt, two_pass, nt);
    case MODE_ADALN: return mis_lookup_nt<MODE_ADALN>(xdt, wdt, vpt, two_pass, nt);
    default: break;
    }
    return nullptr;
}

}  // namespace rmsn
