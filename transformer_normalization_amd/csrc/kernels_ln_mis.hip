// kernels_ln_mis.hip -- instantiations of the LayerNorm forward (plain and
// fused residual) for rows off the 16-byte grid: 16-byte vectors read and
// written at the row's byte offset (ln_kernels.hpp, MIS), resident or, for
// long rows, in passes over the row.
#include "kernel_tables.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, bool RES, bool NT>
ln_fn mis_kernel(int vpt, bool tp) {
    // 2: x and its parameters are all 16-bit (the register budget)
    constexpr int ES2 = Fmt<XDT>::bytes == 2 && Fmt<WDT>::bytes == 2 ? 2 : 4;
    constexpr int V = 16 / Fmt<XDT>::bytes;
    if (tp) return vpt == 4 ? layernorm_fwd_kernel<XDT, WDT, V, 4, RES, true, NT, 1024, true> : nullptr;
    switch (vpt) {
    case 1: return layernorm_fwd_kernel<XDT, WDT, V, 1, RES, false, NT, ln_max_threads(1 * V, ES2), true>;
    case 2: return layernorm_fwd_kernel<XDT, WDT, V, 2, RES, false, NT, ln_max_threads(2 * V, ES2), true>;
    case 3: return layernorm_fwd_kernel<XDT, WDT, V, 3, RES, false, NT, ln_max_threads(3 * V, ES2), true>;
    case 4: return layernorm_fwd_kernel<XDT, WDT, V, 4, RES, false, NT, ln_max_threads(4 * V, ES2), true>;
    case 6: return layernorm_fwd_kernel<XDT, WDT, V, 6, RES, false, NT, ln_max_threads(6 * V, ES2), true>;
    case 8: return layernorm_fwd_kernel<XDT, WDT, V, 8, RES, false, NT, ln_max_threads(8 * V, ES2), true>;
    default: break;
    }
    return nullptr;
}

template <bool RES, bool NT>
ln_fn mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool tp) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return mis_kernel<DT_F32, DT_F32, RES, NT>(vpt, tp);
    case RMSN_F16:
        return wf32 ? mis_kernel<DT_F16, DT_F32, RES, NT>(vpt, tp) : mis_kernel<DT_F16, DT_F16, RES, NT>(vpt, tp);
    case RMSN_BF16:
        return wf32 ? mis_kernel<DT_BF16, DT_F32, RES, NT>(vpt, tp) : mis_kernel<DT_BF16, DT_BF16, RES, NT>(vpt, tp);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace

ln_fn ln_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, bool nt, bool resid) {
    if (resid)
        return nt ? mis_lookup<true, true>(xdt, wdt, vpt, two_pass) : mis_lookup<true, false>(xdt, wdt, vpt, two_pass);
    return nt ? mis_lookup<false, true>(xdt, wdt, vpt, two_pass) : mis_lookup<false, false>(xdt, wdt, vpt, two_pass);
}

}  // namespace rmsn
