// kernels_ln.hip -- instantiations of the LayerNorm forward kernels
// (ln_kernels.hpp), plain and fused with the residual add.
#include "kernel_tables.hpp"
#include "ln_kernels.hpp"

namespace rmsn {
namespace {

template <int XDT, int WDT, int VEC, bool RES, bool NT>
ln_fn ln_kernel_for(int vpt, bool two_pass) {
    // 2: x and its parameters are all 16-bit (the register budget)
    constexpr int ES2 = Fmt<XDT>::bytes == 2 && Fmt<WDT>::bytes == 2 ? 2 : 4;
    if (two_pass) {
        constexpr int V = VEC > 1 ? 4 : 8;
        return layernorm_fwd_kernel<XDT, WDT, VEC, V, RES, true, NT, 1024>;
    }
    switch (vpt) {
    case 1: return layernorm_fwd_kernel<XDT, WDT, VEC, 1, RES, false, NT, ln_max_threads(1 * VEC, ES2)>;
    case 2: return layernorm_fwd_kernel<XDT, WDT, VEC, 2, RES, false, NT, ln_max_threads(2 * VEC, ES2)>;
    case 4: return layernorm_fwd_kernel<XDT, WDT, VEC, 4, RES, false, NT, ln_max_threads(4 * VEC, ES2)>;
    case 8: return layernorm_fwd_kernel<XDT, WDT, VEC, 8, RES, false, NT, ln_max_threads(8 * VEC, ES2)>;
    default: break;
    }
    if constexpr (VEC > 1) {
        switch (vpt) {
        case 3: return layernorm_fwd_kernel<XDT, WDT, VEC, 3, RES, false, NT, ln_max_threads(3 * VEC, ES2)>;
        case 6: return layernorm_fwd_kernel<XDT, WDT, VEC, 6, RES, false, NT, ln_max_threads(6 * VEC, ES2)>;
        default: break;
        }
    }
    return nullptr;
}

template <int XDT, int WDT, bool RES, bool NT>
ln_fn ln_kernel_vec(int vec, int vpt, bool two_pass) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    return vec == 1 ? ln_kernel_for<XDT, WDT, 1, RES, NT>(vpt, two_pass)
                    : ln_kernel_for<XDT, WDT, V, RES, NT>(vpt, two_pass);
}

template <bool RES, bool NT>
ln_fn ln_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return ln_kernel_vec<DT_F32, DT_F32, RES, NT>(vec, vpt, two_pass);
    case RMSN_F16:
        return wf32 ? ln_kernel_vec<DT_F16, DT_F32, RES, NT>(vec, vpt, two_pass)
                    : ln_kernel_vec<DT_F16, DT_F16, RES, NT>(vec, vpt, two_pass);
    case RMSN_BF16:
        return wf32 ? ln_kernel_vec<DT_BF16, DT_F32, RES, NT>(vec, vpt, two_pass)
                    : ln_kernel_vec<DT_BF16, DT_BF16, RES, NT>(vec, vpt, two_pass);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace

ln_fn ln_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt, bool resid) {
    if (resid)
        return nt ? ln_lookup_nt<true, true>(xdt, wdt, vec, vpt, two_pass)
                  : ln_lookup_nt<true, false>(xdt, wdt, vec, vpt, two_pass);
    return nt ? ln_lookup_nt<false, true>(xdt, wdt, vec, vpt, two_pass)
              : ln_lookup_nt<false, false>(xdt, wdt, vec, vpt, two_pass);
}

}  // namespace rmsn
