// kernels_bwd_mis.hip -- instantiations of the backward (plain and residual)
// for rows off the 16-byte grid: 16-byte vectors read and written at the row's
// byte offset (bwd_kernels.hpp, MIS), in one pass or two.
#include "kernel_tables.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, bool RES, bool NT>
bwd_fn mis_kernel(int vpt, bool two_pass, bool deep) {
    constexpr int ES = Fmt<XDT>::bytes;  // x's element size, for the register budget
    constexpr int V = 16 / ES;
    if (two_pass) return vpt == 4 ? rmsnorm_bwd_kernel<XDT, WDT, V, 4, RES, true, NT, 1024, true> : nullptr;
    if (deep) {  // the one-vector tile, three rows prefetched (16-bit formats)
        constexpr int T = bwd_max_threads(V, RES, ES);
        if constexpr (ES == 2)
            return vpt == 1 ? rmsnorm_bwd_kernel<XDT, WDT, V, 1, RES, false, NT, T, true, true> : nullptr;
        return nullptr;
    }
    switch (vpt) {
    case 1: return rmsnorm_bwd_kernel<XDT, WDT, V, 1, RES, false, NT, bwd_max_threads(1 * V, RES, ES), true>;
    case 2: return rmsnorm_bwd_kernel<XDT, WDT, V, 2, RES, false, NT, bwd_max_threads(2 * V, RES, ES), true>;
    case 3: return rmsnorm_bwd_kernel<XDT, WDT, V, 3, RES, false, NT, bwd_max_threads(3 * V, RES, ES), true>;
    case 4: return rmsnorm_bwd_kernel<XDT, WDT, V, 4, RES, false, NT, bwd_max_threads(4 * V, RES, ES), true>;
    default: break;
    }
    return nullptr;
}

template <bool RES, bool NT>
bwd_fn mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool tp, bool dp) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return mis_kernel<DT_F32, DT_F32, RES, NT>(vpt, tp, dp);
    case RMSN_F16:
        return wf32 ? mis_kernel<DT_F16, DT_F32, RES, NT>(vpt, tp, dp)
                    : mis_kernel<DT_F16, DT_F16, RES, NT>(vpt, tp, dp);
    case RMSN_BF16:
        return wf32 ? mis_kernel<DT_BF16, DT_F32, RES, NT>(vpt, tp, dp)
                    : mis_kernel<DT_BF16, DT_BF16, RES, NT>(vpt, tp, dp);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace

bwd_fn bwd_mis_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vpt, bool two_pass, bool res, bool nt, bool deep) {
    if (res)
        return nt ? mis_lookup<true, true>(xdt, wdt, vpt, two_pass, deep)
                  : mis_lookup<true, false>(xdt, wdt, vpt, two_pass, deep);
    return nt ? mis_lookup<false, true>(xdt, wdt, vpt, two_pass, deep)
              : mis_lookup<false, false>(xdt, wdt, vpt, two_pass, deep);
}

}  // namespace rmsn
