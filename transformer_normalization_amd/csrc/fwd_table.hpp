// fwd_table.hpp -- maps (formats, access width, tile) to a forward kernel
// instantiation.  Included by the one translation unit per kernel family
// (kernels_fwd.hip, kernels_fwd_residual.hip, kernels_adaln.hip), each of
// which instantiates a single MODE, so the families compile in parallel.
#pragma once

#include "kernel_tables.hpp"

namespace rmsn {
namespace tables {

template <int XDT, int WDT, int VEC, int MODE, bool NT>
fwd_fn fwd_kernel_for(int vpt, bool two_pass) {
    // 2: x and its parameters are all 16-bit (the register budget)
    constexpr int ES2 = Fmt<XDT>::bytes == 2 && Fmt<WDT>::bytes == 2 ? 2 : 4;
    if (two_pass) {
        constexpr int V = VEC > 1 ? 4 : 8;
        return rmsnorm_fwd_kernel<XDT, WDT, VEC, V, MODE, true, NT, 1024>;
    }
    switch (vpt) {
    case 1: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 1, MODE, false, NT, fwd_max_threads(1 * VEC, MODE, ES2)>;
    case 2: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 2, MODE, false, NT, fwd_max_threads(2 * VEC, MODE, ES2)>;
    case 4: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 4, MODE, false, NT, fwd_max_threads(4 * VEC, MODE, ES2)>;
    case 8: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 8, MODE, false, NT, fwd_max_threads(8 * VEC, MODE, ES2)>;
    default: break;
    }
    if constexpr (VEC > 1) {
        switch (vpt) {
        case 3: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 3, MODE, false, NT, fwd_max_threads(3 * VEC, MODE, ES2)>;
        case 6: return rmsnorm_fwd_kernel<XDT, WDT, VEC, 6, MODE, false, NT, fwd_max_threads(6 * VEC, MODE, ES2)>;
        default: break;
        }
    }
    return nullptr;
}

template <int XDT, int WDT, int MODE, bool NT>
fwd_fn fwd_kernel_vec(int vec, int vpt, bool two_pass) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    return vec == 1 ? fwd_kernel_for<XDT, WDT, 1, MODE, NT>(vpt, two_pass)
                    : fwd_kernel_for<XDT, WDT, V, MODE, NT>(vpt, two_pass);
}

template <int MODE, bool NT>
fwd_fn fwd_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return fwd_kernel_vec<DT_F32, DT_F32, MODE, NT>(vec, vpt, two_pass);
    case RMSN_F16:
        return wf32 ? fwd_kernel_vec<DT_F16, DT_F32, MODE, NT>(vec, vpt, two_pass)
                    : fwd_kernel_vec<DT_F16, DT_F16, MODE, NT>(vec, vpt, two_pass);
    case RMSN_BF16:
        return wf32 ? fwd_kernel_vec<DT_BF16, DT_F32, MODE, NT>(vec, vpt, two_pass)
                    : fwd_kernel_vec<DT_BF16, DT_BF16, MODE, NT>(vec, vpt, two_pass);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace tables
}  // namespace rmsn
