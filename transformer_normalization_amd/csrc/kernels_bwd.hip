// kernels_bwd.hip -- instantiations of the backward kernels (bwd_kernels.hpp)
// and the dw finalize kernel.
#include "bwd_table.hpp"

namespace rmsn {

__global__ void __launch_bounds__(kFinCols * kFinSlices) rmsnorm_dw_finalize(const float *__restrict__ partial, int P,
                                                                             int H, float *__restrict__ dw) {
    __shared__ float sums[kFinSlices][kFinCols];
    const int c = threadIdx.x % kFinCols;
    const int s = threadIdx.x / kFinCols;
    const int col = blockIdx.x * kFinCols + c;
    float acc = 0.0f;
    if (col < H) {
        int q = s;
        for (; q + kFinSlices * (kFinBatch - 1) < P; q += kFinSlices * kFinBatch) {
            float v[kFinBatch];
#pragma unroll
            for (int j = 0; j < kFinBatch; ++j) v[j] = partial[(int64_t)(q + kFinSlices * j) * H + col];
#pragma unroll
            for (int j = 0; j < kFinBatch; ++j) acc += v[j];
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

bwd_fn bwd_lookup_plain(rmsn_dtype_t xdt, rmsn_dtype_t wdt, int vec, int vpt, bool two_pass, bool nt,
                        bool deep) {
    return nt ? tables::bwd_lookup_nt<false, true>(xdt, wdt, vec, vpt, two_pass, deep)
              : tables::bwd_lookup_nt<false, false>(xdt, wdt, vec, vpt, two_pass, deep);
}

const void *dw_finalize_kernel() { return (const void *)rmsnorm_dw_finalize; }

}  // namespace rmsn
