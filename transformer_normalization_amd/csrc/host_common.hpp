// host_common.hpp -- host-side helpers shared by the library's entry points
// (rmsnorm_api.hip, rope_api.hip): error reporting, per-device facts,
// argument checks and kernel launch.  Nothing here allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsnorm.h"

namespace rmsn {
namespace host {

// Records a printf-style message for rmsnorm_last_error() and returns s.
rmsn_status_t fail(rmsn_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns RMSN_OK (the end of a successful call).
rmsn_status_t ok();
// The calling thread's most recent message ("" after a success).
const char *last_error();

// Compute-unit count of the current device, read once per device.  A failed
// read is RMSN_ERR_HIP and a device other than gfx950 RMSN_ERR_UNSUPPORTED;
// no value is ever guessed.
rmsn_status_t device_info(int *cus);

inline int dtype_bytes(rmsn_dtype_t t) { return t == RMSN_F32 ? 4 : 2; }
inline bool dtype_valid(int t) { return t == RMSN_F32 || t == RMSN_F16 || t == RMSN_BF16; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned_to(const void *p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

// A buffer as the byte range spanned by `rows` rows of `cols` elements,
// `stride` elements apart, plus what identifies "the same buffer".
struct Region {
    const char *name;
    uintptr_t base;
    int64_t stride;  // elements, 0 for vectors
    int64_t rows;
    int64_t cols;
    int ebytes;
    bool present;
    // Byte bounds in 128-bit arithmetic: no size the caller passes can
    // overflow them (check_overlap rejects a region whose end passes 2^64
    // before comparing any).  Regions have rows >= 1.
    unsigned __int128 lo() const { return base; }
    unsigned __int128 hi() const {
        return (unsigned __int128)base +
               (unsigned __int128)(((__int128)(rows - 1) * stride + cols) * (__int128)ebytes);
    }
    bool fits() const { return hi() <= ((unsigned __int128)1 << 64); }
    bool overlaps(const Region &o) const { return lo() < o.hi() && o.lo() < hi(); }
    bool same(const Region &o) const {
        return base == o.base && stride == o.stride && rows == o.rows && cols == o.cols && ebytes == o.ebytes;
    }
};

inline Region mat(const char *name, const void *p, int64_t stride, int64_t M, int64_t H, int eb) {
    return Region{name, (uintptr_t)p, stride, M, H, eb, p != nullptr};
}
inline Region vec(const char *name, const void *p, int64_t n, int eb) {
    return Region{name, (uintptr_t)p, 0, 1, n, eb, p != nullptr};
}

// Outputs must not overlap each other; an output may overlap an input only
// by being exactly the same buffer.
rmsn_status_t check_overlap(const Region *outs, int nout, const Region *ins, int nin);

// stride >= cols, and the last byte of `rows` rows is addressable.
rmsn_status_t check_stride(const char *name, int64_t stride, int64_t rows, int64_t cols, int eb);

// Whether a call moving `bytes_moved` bytes of streamed data should use
// non-temporal accesses (by size unless forced by set_stream_mode: -1 by
// size, 0 never, 1 always; rmsnorm_tuning_set_streaming).
bool use_streaming(int64_t bytes_moved);
void set_stream_mode(int mode);

// Launch-geometry override (include/rmsnorm_tuning.h): which = 0 forward,
// 1 backward, 2 RoPE; the meaning of a..d is the caller's.
struct Override {
    bool set = false;
    int a = 0, b = 0, c = 0;
    int64_t d = 0;
};
Override get_override(int which);
void set_override(int which, int a, int b, int c, int64_t d);

// shmem: dynamic LDS bytes per workgroup
rmsn_status_t launch(const void *fn, dim3 grid, dim3 block, void **args, hipStream_t stream, const char *what,
                     size_t shmem = 0);

}  // namespace host
}  // namespace rmsn
