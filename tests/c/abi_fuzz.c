/* Random-argument driver of every C ABI entry point, for a run of the
 * library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitize_cpu.py).
 *
 * Sizes, strides and counts are drawn from values that stress the library's
 * own arithmetic (0, +-1, powers of two around 2^31, 2^62, INT64_MIN and
 * INT64_MAX, random small values); formats from valid and invalid codes; eps
 * from normal, zero, negative, NaN, infinite and tiny values; pointers from
 * NULL and fake, never dereferenced device addresses (aligned, misaligned,
 * and equal to another argument).  No call may crash or trip a sanitizer,
 * every status must be one of the five documented codes, and every failure
 * must come with an error message.
 *
 * It runs only where no device is visible: then no call can reach a kernel
 * launch (a call that passes every check fails at the device query), so the
 * fake addresses are never used.  With a device present it exits at once
 * with status 77 (skipped). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "layernorm.h"
#include "rmsnorm.h"
#include "rmsnorm_tuning.h"
#include "rope.h"

static int failures = 0;
static uint64_t state = 0x243F6A8885A308D3ull;

static uint64_t next(void) { /* SplitMix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static int64_t size_arg(void) {
    static const int64_t special[] = {0, 1, 2, 3, 7, 8, 15, 16, 63, 64, 65, 512, 4096, 6144, 65535, 65536,
                                      (1ll << 30), (1ll << 30) + 1, (1ll << 31) - 1, (1ll << 31), (1ll << 32),
                                      (1ll << 40), (1ll << 62), INT64_MAX, INT64_MAX - 1, -1, -2, -64,
                                      INT64_MIN, INT64_MIN + 1};
    const uint64_t r = next() % 3;
    if (r == 0) return special[next() % (sizeof special / sizeof special[0])];
    if (r == 1) return (int64_t)(next() % 5000);
    return (int64_t)(next() % 70) - 2;
}
static int int_arg(void) {
    static const int special[] = {0, 1, 2, 3, 4, 7, 8, 16, 64, 1024, 65536, 1 << 30, 2147483647, -1, -2,
                                  -2147483647 - 1};
    return next() % 2 ? special[next() % (sizeof special / sizeof special[0])] : (int)(next() % 40) - 3;
}
static rmsn_dtype_t dtype_arg(void) {
    static const int codes[] = {0, 1, 2, 0, 1, 2, 3, 4, -1, 7, 2147483647, -2147483647 - 1};
    return (rmsn_dtype_t)codes[next() % (sizeof codes / sizeof codes[0])];
}
static float eps_arg(void) {
    static const float v[] = {1e-5f, 1e-6f, 1.0f, 0.0f, -0.0f, -1e-5f, 1e-45f, 3.4e38f};
    const uint64_t r = next() % 10;
    if (r == 0) return NAN;
    if (r == 1) return INFINITY;
    if (r == 2) return -INFINITY;
    return v[next() % (sizeof v / sizeof v[0])];
}
/* fake device addresses: 2^44 apart, aligned or not; NULL now and then; an
 * argument may repeat an earlier one (aliasing) */
static void *pool[8];
static int npool = 0;
static void *ptr_arg(void) {
    const uint64_t r = next() % 10;
    void *p;
    if (r == 0) {
        p = NULL;
    } else if (r == 1 && npool > 0) {
        p = pool[next() % (uint64_t)npool];
    } else {
        uintptr_t a = ((uintptr_t)(next() % 16) + 1) << 44;
        if (r == 2) a += (uintptr_t)(next() % 16) * 2;
        p = (void *)a;
    }
    if (npool < 8) pool[npool++] = p;
    return p;
}
static size_t bytes_arg(void) {
    static const size_t v[] = {0, 1, 16, 4096, (size_t)1 << 20, (size_t)1 << 33, SIZE_MAX, SIZE_MAX - 15};
    return next() % 2 ? v[next() % (sizeof v / sizeof v[0])] : (size_t)(next() % (1u << 26));
}

static void check(const char *what, rmsn_status_t s) {
    if ((int)s < 0 || (int)s > 4) {
        printf("FAIL %s: status %d is not a documented code\n", what, (int)s);
        ++failures;
        return;
    }
    if (s != RMSN_OK && rmsnorm_last_error()[0] == '\0') {
        printf("FAIL %s: %s without an error message\n", what, rmsnorm_status_string(s));
        ++failures;
    }
    if (rmsnorm_status_string(s) == NULL) {
        printf("FAIL %s: no status string\n", what);
        ++failures;
    }
}

int main(int argc, char **argv) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
        printf("skipped: a device is visible\n");
        return 77;
    }
    const int iters = argc > 1 ? atoi(argv[1]) : 20000;
    if (argc > 2) state ^= strtoull(argv[2], NULL, 10) * 0x9E3779B97F4A7C15ull;  /* seed */
    for (int it = 0; it < iters; ++it) {
        npool = 0;
        /* sometimes force a launch geometry with extreme values first */
        if (next() % 8 == 0) rmsnorm_tuning_set_geometry(int_arg() % 4, int_arg(), int_arg(), int_arg(), size_arg());
        if (next() % 16 == 0) rmsnorm_tuning_set_streaming(int_arg());
        switch (next() % 13) {
        case 0:
            check("rmsnorm_fwd", rmsnorm_fwd(ptr_arg(), size_arg(), ptr_arg(), ptr_arg(), size_arg(), (float *)ptr_arg(),
                                             size_arg(), size_arg(), eps_arg(), dtype_arg(), dtype_arg(), NULL));
            break;
        case 1:
            check("rmsnorm_fwd_residual",
                  rmsnorm_fwd_residual(ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(), ptr_arg(), size_arg(),
                                       ptr_arg(), size_arg(), (float *)ptr_arg(), size_arg(), size_arg(), eps_arg(),
                                       dtype_arg(), dtype_arg(), NULL));
            break;
        case 2:
            check("rmsnorm_adaln_fwd",
                  rmsnorm_adaln_fwd(ptr_arg(), size_arg(), ptr_arg(), ptr_arg(), ptr_arg(), size_arg(), size_arg(),
                                    ptr_arg(), size_arg(), (float *)ptr_arg(), size_arg(), size_arg(), eps_arg(),
                                    dtype_arg(), dtype_arg(), NULL));
            break;
        case 3: {
            const size_t need = rmsnorm_bwd_workspace_bytes(size_arg(), size_arg());
            (void)need;
            check("rmsnorm_bwd",
                  rmsnorm_bwd(ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(), (const float *)ptr_arg(),
                              ptr_arg(), size_arg(), (float *)ptr_arg(), ptr_arg(), bytes_arg(), size_arg(),
                              size_arg(), dtype_arg(), dtype_arg(), NULL));
            break;
        }
        case 4:
            check("rmsnorm_bwd_residual",
                  rmsnorm_bwd_residual(ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(),
                                       (const float *)ptr_arg(), ptr_arg(), size_arg(), (float *)ptr_arg(), ptr_arg(),
                                       bytes_arg(), size_arg(), size_arg(), dtype_arg(), dtype_arg(), NULL));
            break;
        case 5:
            check("rope_apply", rope_apply(ptr_arg(), size_arg(), size_arg(), ptr_arg(), ptr_arg(), size_arg(),
                                           ptr_arg(), size_arg(), size_arg(), size_arg(), size_arg(), size_arg(),
                                           size_arg(), int_arg(), dtype_arg(), dtype_arg(), NULL));
            break;
        case 6:
            check("layernorm_fwd", layernorm_fwd(ptr_arg(), size_arg(), ptr_arg(), ptr_arg(), ptr_arg(), size_arg(),
                                                 (float *)ptr_arg(), (float *)ptr_arg(), size_arg(), size_arg(),
                                                 eps_arg(), dtype_arg(), dtype_arg(), NULL));
            break;
        case 7:
            check("layernorm_fwd_residual",
                  layernorm_fwd_residual(ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(), ptr_arg(),
                                         ptr_arg(), size_arg(), ptr_arg(), size_arg(), (float *)ptr_arg(),
                                         (float *)ptr_arg(), size_arg(), size_arg(), eps_arg(), dtype_arg(),
                                         dtype_arg(), NULL));
            break;
        case 8:
            check("rmsnorm_tuning_copy", rmsnorm_tuning_copy(ptr_arg(), ptr_arg(), size_arg(), NULL));
            break;
        case 9: {
            const char *s = rmsnorm_status_string((rmsn_status_t)int_arg());
            if (s == NULL || s[0] == '\0') {
                printf("FAIL rmsnorm_status_string: empty\n");
                ++failures;
            }
            break;
        }
        case 10:
            check("rmsnorm_bwd_noalloc",
                  rmsnorm_bwd_noalloc(ptr_arg(), size_arg(), ptr_arg(), size_arg(), ptr_arg(), (const float *)ptr_arg(),
                                      ptr_arg(), size_arg(), (float *)ptr_arg(), size_arg(), size_arg(), dtype_arg(),
                                      dtype_arg(), NULL));
            break;
        case 11: {
            int32_t tile[6];
            check("rmsnorm_tuning_tile", rmsnorm_tuning_tile(int_arg(), size_arg(), dtype_arg(), int_arg(),
                                                             next() % 8 ? tile : NULL));
            break;
        }
        default:
            (void)rmsnorm_bwd_workspace_bytes(size_arg(), size_arg());
            break;
        }
    }
    rmsnorm_tuning_set_geometry(0, 0, 0, 0, 0);
    rmsnorm_tuning_set_geometry(1, 0, 0, 0, 0);
    rmsnorm_tuning_set_geometry(2, 0, 0, 0, 0);
    rmsnorm_tuning_set_streaming(-1);
    printf("%s (%d failures in %d calls)\n", failures ? "FAILED" : "ok", failures, iters);
    return failures ? 1 : 0;
}
