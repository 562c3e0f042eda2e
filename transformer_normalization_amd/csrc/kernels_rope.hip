// kernels_rope.hip -- instantiations of the RoPE apply kernel (rope_kernels.hpp).
#include "kernel_tables.hpp"
#include "rope_kernels.hpp"

namespace rmsn {
namespace {

template <int XDT, int TDT, bool NT>
rope_fn rope_for(int vec, bool xchg) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    if (vec == 1) return xchg ? nullptr : rope_apply_kernel<XDT, TDT, 1, NT, false>;
    return xchg ? rope_apply_kernel<XDT, TDT, V, NT, true> : rope_apply_kernel<XDT, TDT, V, NT, false>;
}

template <bool NT>
rope_fn rope_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t tdt, int vec, bool xchg) {
    const bool tf32 = (tdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return rope_for<DT_F32, DT_F32, NT>(vec, xchg);
    case RMSN_F16:
        return tf32 ? rope_for<DT_F16, DT_F32, NT>(vec, xchg) : rope_for<DT_F16, DT_F16, NT>(vec, xchg);
    case RMSN_BF16:
        return tf32 ? rope_for<DT_BF16, DT_F32, NT>(vec, xchg) : rope_for<DT_BF16, DT_BF16, NT>(vec, xchg);
    default: break;  // any other value: no kernel
    }
    return nullptr;
}

}  // namespace

rope_fn rope_lookup(rmsn_dtype_t xdt, rmsn_dtype_t tdt, int vec, bool nt, bool xchg) {
    return nt ? rope_lookup_nt<true>(xdt, tdt, vec, xchg) : rope_lookup_nt<false>(xdt, tdt, vec, xchg);
}

}  // namespace rmsn
