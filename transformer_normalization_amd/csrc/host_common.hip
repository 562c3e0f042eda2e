// host_common.hip -- definitions of the host helpers in host_common.hpp.

#include <atomic>
#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "host_common.hpp"

namespace rmsn {
namespace host {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

rmsn_status_t fail(rmsn_status_t s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

const char *last_error() { return g_last_error; }

rmsn_status_t ok() {
    g_last_error[0] = '\0';
    return RMSN_OK;
}

// ---------------------------------------------------------------------------
// device facts (read once per device; a failed read is an error, never a guess)
// ---------------------------------------------------------------------------

namespace {
constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::once_flag once;
    rmsn_status_t status = RMSN_ERR_HIP;
    int cus = 0;
    char detail[256] = "";
};

DeviceInfo g_devices[kMaxDevices];
}  // namespace

rmsn_status_t device_info(int *cus) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RMSN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(RMSN_ERR_HIP, "device index %d out of range", dev);
    DeviceInfo &d = g_devices[dev];
    std::call_once(d.once, [&d, dev]() {
        int n = 0;
        hipError_t err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess || n <= 0) {
            snprintf(d.detail, sizeof d.detail, "reading the compute-unit count of device %d failed: %s", dev,
                     hipGetErrorString(err));
            d.status = RMSN_ERR_HIP;
            return;
        }
        hipDeviceProp_t prop;
        err = hipGetDeviceProperties(&prop, dev);
        if (err != hipSuccess) {
            snprintf(d.detail, sizeof d.detail, "reading the properties of device %d failed: %s", dev,
                     hipGetErrorString(err));
            d.status = RMSN_ERR_HIP;
            return;
        }
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            snprintf(d.detail, sizeof d.detail, "device %d is %s; this library is built for gfx950 only", dev,
                     prop.gcnArchName);
            d.status = RMSN_ERR_UNSUPPORTED;
            return;
        }
        d.cus = n;
        d.status = RMSN_OK;
    });
    if (d.status != RMSN_OK) return fail(d.status, "%s", d.detail);
    *cus = d.cus;
    return RMSN_OK;
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------

rmsn_status_t check_overlap(const Region *outs, int nout, const Region *ins, int nin) {
    for (int k = 0; k < nout + nin; ++k) {
        const Region &r = k < nout ? outs[k] : ins[k - nout];
        if (r.present && !r.fits())
            return fail(RMSN_ERR_INVALID_ARG, "%s extends past the end of the address space", r.name);
    }
    for (int i = 0; i < nout; ++i) {
        if (!outs[i].present) continue;
        for (int j = i + 1; j < nout; ++j)
            if (outs[j].present && outs[i].overlaps(outs[j]))
                return fail(RMSN_ERR_INVALID_ARG, "outputs %s and %s overlap", outs[i].name, outs[j].name);
        for (int j = 0; j < nin; ++j)
            if (ins[j].present && outs[i].overlaps(ins[j]) && !outs[i].same(ins[j]))
                return fail(RMSN_ERR_INVALID_ARG, "output %s partially overlaps input %s", outs[i].name,
                            ins[j].name);
    }
    return RMSN_OK;
}

rmsn_status_t check_stride(const char *name, int64_t stride, int64_t M, int64_t H, int eb) {
    if (stride < H)
        return fail(RMSN_ERR_INVALID_ARG, "%s = %lld is smaller than the row length %lld", name, (long long)stride,
                    (long long)H);
    // the last byte of the matrix must be addressable without overflow
    if (M > 1 && (stride > (INT64_MAX / eb) / (M - 1)))
        return fail(RMSN_ERR_INVALID_ARG, "%s * M overflows", name);
    return RMSN_OK;
}

// Streaming (non-temporal) accesses pay off when a call moves more data than
// the caches could usefully keep for the next kernel; below that, ordinary
// cached accesses leave the outputs in L2 / the last-level cache for the
// consumer.  Mode -1 = decide by size, 0 = never, 1 = always.
constexpr int64_t kStreamBytes = int64_t(64) << 20;
namespace {
std::atomic<int> g_stream_mode{-1};
}  // namespace

bool use_streaming(int64_t bytes_moved) {
    const int mode = g_stream_mode.load(std::memory_order_relaxed);
    return mode < 0 ? bytes_moved >= kStreamBytes : mode > 0;
}

void set_stream_mode(int mode) { g_stream_mode.store(mode < 0 ? -1 : mode > 0 ? 1 : 0); }

// Launch-geometry override for tuning and for tests that must reach the
// grid-stride and two-pass paths at small sizes, set only through
// rmsnorm_tuning_set_geometry() (include/rmsnorm_tuning.h): slot 0 forward,
// 1 backward, 2 RoPE.  Nothing else (no environment variable) changes it.
namespace {
std::mutex g_override_mu;
Override g_override[3];
std::atomic<bool> g_override_any{false};
}  // namespace

Override get_override(int which) {
    if (!g_override_any.load(std::memory_order_relaxed)) return Override{};
    std::lock_guard<std::mutex> lk(g_override_mu);
    return g_override[which];
}

void set_override(int which, int a, int b, int c, int64_t d) {
    std::lock_guard<std::mutex> lk(g_override_mu);
    if (which < 0 || which > 2) return;
    Override o;
    o.set = a > 0 && b > 0;
    o.a = a;
    o.b = b;
    o.c = c;
    o.d = d;
    g_override[which] = o;
    g_override_any.store(g_override[0].set || g_override[1].set || g_override[2].set);
}

rmsn_status_t launch(const void *fn, dim3 grid, dim3 block, void **args, hipStream_t stream, const char *what,
                     size_t shmem) {
    hipError_t e = hipLaunchKernel(fn, grid, block, args, shmem, stream);
    if (e != hipSuccess) return fail(RMSN_ERR_HIP, "launching %s failed: %s", what, hipGetErrorString(e));
    return RMSN_OK;
}

}  // namespace host
}  // namespace rmsn
