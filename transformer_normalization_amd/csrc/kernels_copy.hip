// kernels_copy.hip -- the speed-of-light reference of rmsnorm_tuning_copy():
// a plain copy with the forward kernels' access pattern (256 threads per
// workgroup, two 16-byte vectors per thread, non-temporal loads and stores,
// one workgroup per 8 KiB), so that a step's HBM rate can be set beside that
// of moving the same bytes with no arithmetic at all -- with aligned 16-byte
// accesses, or, for buffers off the 16-byte grid, unaligned ones.
#include "host_common.hpp"
#include "kernel_tables.hpp"
#include "rmsnorm_tuning.h"

namespace rmsn {

// A: the 16-byte vector type of the accesses -- u32x4 for 16-byte aligned
// buffers, or a 2-byte-aligned vector for buffers off the 16-byte grid (one
// unaligned global_load_dwordx4 / global_store_dwordx4 each, as the kernels
// for rows off the grid make).
template <typename A>
__global__ void __launch_bounds__(256) copy_reference_kernel(const A *__restrict__ src, A *__restrict__ dst,
                                                             int64_t nvec) {
    const int64_t base = (int64_t)blockIdx.x * 512 + threadIdx.x;
    A v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int64_t i = base + k * 256;
        if (i < nvec) v[k] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int64_t i = base + k * 256;
        if (i < nvec) __builtin_nontemporal_store(v[k], dst + i);
    }
}

}  // namespace rmsn

using namespace rmsn::host;

#define RMSN_API __attribute__((visibility("default")))

extern "C" RMSN_API rmsn_status_t rmsnorm_tuning_copy(const void *src, void *dst, int64_t bytes,
                                                      hipStream_t stream) {
    if (src == nullptr || dst == nullptr) return fail(RMSN_ERR_INVALID_ARG, "src and dst must not be NULL");
    if (bytes < 0 || bytes % 16 != 0)
        return fail(RMSN_ERR_INVALID_ARG, "bytes = %lld must be a non-negative multiple of 16", (long long)bytes);
    if (!aligned_to(src, 2) || !aligned_to(dst, 2))
        return fail(RMSN_ERR_INVALID_ARG, "src and dst must be 2-byte aligned");
    const Region a = vec("src", src, bytes, 1), b = vec("dst", dst, bytes, 1);
    if (bytes > 0 && (!a.fits() || !b.fits()))
        return fail(RMSN_ERR_INVALID_ARG, "src or dst extends past the end of the address space");
    if (bytes > 0 && a.overlaps(b)) return fail(RMSN_ERR_INVALID_ARG, "src and dst overlap");
    if (bytes == 0) return ok();
    const int64_t nvec = bytes / 16;
    const int64_t grid = (nvec + 511) / 512;
    if (grid > INT32_MAX) return fail(RMSN_ERR_UNSUPPORTED, "bytes = %lld is too large", (long long)bytes);
    int cus = 0;
    rmsn_status_t st = device_info(&cus);
    if (st != RMSN_OK) return st;
    void *args[] = {(void *)&src, &dst, (void *)&nvec};
    const bool grid16 = aligned16(src) && aligned16(dst);
    const void *fn = grid16 ? (const void *)rmsn::copy_reference_kernel<rmsn::u32x4>
                            : (const void *)rmsn::copy_reference_kernel<rmsn::u32x4_elem_aligned>;
    st = launch(fn, dim3((unsigned)grid), dim3(256), args, stream, "rmsnorm_tuning_copy");
    return st == RMSN_OK ? ok() : st;
}

