// kernels_bwd.hip -- instantiations of the backward kernels (bwd_kernels.hpp).
#include "kernel_tables.hpp"

namespace rmsn {

__global__ void __launch_bounds__(1024) rmsnorm_dw_finalize(const float *__restrict__ partial, int P, int H,
                                                            float *__restrict__ dw) {
    __shared__ float sums[kFinSlices][kFinCols];
    const int c = threadIdx.x % kFinCols;
    const int s = threadIdx.x / kFinCols;
    const int col = blockIdx.x * kFinCols + c;
    float acc = 0.0f;
    if (col < H) {
        int q = s;
        for (; q + kFinSlices * 7 < P; q += kFinSlices * 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = partial[(int64_t)(q + kFinSlices * j) * H + col];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += v[j];
        }
        for (; q < P; q += kFinSlices) acc += partial[(int64_t)q * H + col];
    }
    sums[s][c] = acc;
    __syncthreads();
    if (s == 0 && col < H) {
        float tot = sums[0][c];
#pragma unroll
        for (int i = 1; i < kFinSlices; ++i) tot += sums[i][c];
        dw[col] = tot;
    }
}


namespace {

template <int XDT, int WDT, int VEC, bool NT>
bwd_fn bwd_kernel_for(int vpt, bool two_pass) {
    if (two_pass) {
        constexpr int V = VEC > 1 ? 4 : 8;
        return rmsnorm_bwd_kernel<XDT, WDT, VEC, V, true, NT, 1024>;
    }
    switch (vpt) {
    case 1: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 1, false, NT, bwd_max_threads(1 * VEC)>;
    case 2: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 2, false, NT, bwd_max_threads(2 * VEC)>;
    case 4: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 4, false, NT, bwd_max_threads(4 * VEC)>;
    default: break;
    }
    if constexpr (VEC == 1) {
        if (vpt == 8) return rmsnorm_bwd_kernel<XDT, WDT, VEC, 8, false, NT, bwd_max_threads(8 * VEC)>;
    }
    if constexpr (VEC > 1) {
        switch (vpt) {
        case 3: return rmsnorm_bwd_kernel<XDT, WDT, VEC, 3, false, NT, bwd_max_threads(3 * VEC)>;
        default: break;
        }
    }
    return nullptr;
}

template <int XDT, int WDT, bool NT>
bwd_fn bwd_kernel_vec(int vec, int vpt, bool two_pass) {
    constexpr int V = 16 / Fmt<XDT>::bytes;
    return vec == 1 ? bwd_kernel_for<XDT, WDT, 1, NT>(vpt, two_pass) : bwd_kernel_for<XDT, WDT, V, NT>(vpt, two_pass);
}

template <bool NT>
bwd_fn bwd_lookup_nt(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass) {
    const bool wf32 = (wdt == RMSN_F32);
    switch (xdt) {
    case RMSN_F32: return bwd_kernel_vec<DT_F32, DT_F32, NT>(vec, vpt, two_pass);
    case RMSN_F16:
        return wf32 ? bwd_kernel_vec<DT_F16, DT_F32, NT>(vec, vpt, two_pass)
                    : bwd_kernel_vec<DT_F16, DT_F16, NT>(vec, vpt, two_pass);
    case RMSN_BF16:
        return wf32 ? bwd_kernel_vec<DT_BF16, DT_F32, NT>(vec, vpt, two_pass)
                    : bwd_kernel_vec<DT_BF16, DT_BF16, NT>(vec, vpt, two_pass);
    }
    return nullptr;
}


}  // namespace

bwd_fn bwd_lookup(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt) {
    return nt ? bwd_lookup_nt<true>(xdt, wdt, vec, vpt, two_pass) : bwd_lookup_nt<false>(xdt, wdt, vec, vpt, two_pass);
}

const void *dw_finalize_kernel() { return (const void *)rmsnorm_dw_finalize; }

}  // namespace rmsn
