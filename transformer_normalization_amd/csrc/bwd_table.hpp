// bwd_table.hpp -- maps (formats, access width, tile) to a backward kernel
// instantiation.  kernels_bwd.hip instantiates the plain backward and
// kernels_bwd_residual.hip the one that adds the residual-stream gradient, so
// the two compile in parallel.
#pragma once

#include "kernel_tables.hpp"

namespace rmsn {
namespace tables {

template <int XDT, int WDT, int VEC, bool RES, bool NT>
bwd_fn bwd_kernel_for(int vpt, bool two_pass, bool deep) {
    constexpr int ES = Fmt<XDT>::bytes;  // x's element size, for the register budget
    if (deep) {  // the plain backward's one-vector tile, three rows prefetched (16-bit formats)
        constexpr int T = bwd_max_threads(VEC, RES, ES);
        if constexpr (VEC > 1 && !RES && ES == 2)
            return vpt == 1 && !two_pass ? rmsnorm_bwd_kernel<XDT, WDT, VEC, 1, RES, false, NT, T, false, true>
                                         : nullptr;
        return nullptr;
    }
    if (two_pass) {
        constexpr int V = VEC > 1 ? 4 : 8;
        return rmsnorm_bwd_kernel<XDT, WDT, VEC, V, RES, true, NT, 1024>;
    }
    switch (vpt) {
    case 1: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 1, RES, false, NT, bwd_max_threads(1 * VEC, RES, ES)>;
    case 2: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 2, RES, false, NT, bwd_max_threads(2 * VEC, RES, ES)>;
    case 4: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 4, RES, false, NT, bwd_max_threads(4 * VEC, RES, ES)>;
    default: break;
    }
    if constexpr (VEC == 1) {
        if (vpt == 8) return rmsnorm_bwd_kernel<XDT, WDT, VEC, 8, RES, false, NT, bwd_max_threads(8 * VEC, RES, ES)>;
    }
    if constexpr (VEC > 1) {
        switch (vpt) {
        case 3: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 3, RES, false, NT, bwd_max_threads(3 * VEC, RES, ES)>;
        default: break;
        }
    }
    return nullptr;
}

template <int XDT, int WDT, bool RES, bool NT>
bwd_fn bwd_kernel_vec(int vec, int vpt, bool two_pass, bool deep) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    return vec == 1 ? bwd_kernel_for<XDT, WDT, 1, RES, NT>(vpt, two_pass, deep)
                    : bwd_kernel_for<XDT, WDT, V, RES, NT>(vpt, two_pass, deep);
}

template <bool RES, bool NT>
bwd_fn bwd_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool deep) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return bwd_kernel_vec<DT_F32, DT_F32, RES, NT>(vec, vpt, two_pass, deep);
    case RMSN_F16:
        return wf32 ? bwd_kernel_vec<DT_F16, DT_F32, RES, NT>(vec, vpt, two_pass, deep)
                    : bwd_kernel_vec<DT_F16, DT_F16, RES, NT>(vec, vpt, two_pass, deep);
    case RMSN_BF16:
        return wf32 ? bwd_kernel_vec<DT_BF16, DT_F32, RES, NT>(vec, vpt, two_pass, deep)
                    : bwd_kernel_vec<DT_BF16, DT_BF16, RES, NT>(vec, vpt, two_pass, deep);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace tables
}  // namespace rmsn
