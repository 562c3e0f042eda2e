/* Plain C client of librmsnorm.so on the GPU: device buffers from hipMalloc,
 * no Python, no torch.  Every expected value is exact and follows from the
 * definitions alone:
 *   - bfloat16 rows of +-1 with eps = 1e-5 normalise to rrms = 0.999995,
 *     and +-0.999995 * w rounds back to +-w for w = 1.5;
 *   - the fused residual with x = 1, r = -0.5 writes h = 0.5 exactly and
 *     normalises it to +-w the same way;
 *   - RoPE with quarter-turn tables (cos, sin in {0, +-1}) copies or negates
 *     elements exactly.
 * Exit status 0 = all checks passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rmsnorm.h"
#include "rope.h"

static int failures = 0;

#define CHECK_HIP(call)                                                                 \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) {                                                         \
            printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

static uint16_t bf16(float f) {  /* exact for the values used here */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void expect_ok(const char *what, rmsn_status_t s) {
    if (s != RMSN_OK) {
        printf("FAIL %s: %s (%s)\n", what, rmsnorm_status_string(s), rmsnorm_last_error());
        ++failures;
    }
}

static void expect_bits(const char *what, const uint16_t *got, const uint16_t *want, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (got[i] != want[i]) {
            printf("FAIL %s: element %zu is 0x%04x, expected 0x%04x\n", what, i, got[i], want[i]);
            ++failures;
            return;
        }
}

int main(void) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
        printf("no GPU\n");
        return 2;
    }
    enum { M = 300, H = 4096 };
    const size_t n = (size_t)M * H;
    uint16_t *hx = malloc(n * 2), *hr = malloc(n * 2), *hy = malloc(n * 2), *want = malloc(n * 2);
    uint16_t hw[H];
    for (size_t i = 0; i < n; ++i) {
        const int neg = (int)((i / H + i % H) % 3 == 0);
        hx[i] = bf16(neg ? -1.0f : 1.0f);
        want[i] = bf16(neg ? -1.5f : 1.5f);
    }
    for (int j = 0; j < H; ++j) hw[j] = bf16(1.5f);

    void *dx, *dr, *dy, *dro, *dw;
    float *drrms;
    CHECK_HIP(hipMalloc(&dx, n * 2));
    CHECK_HIP(hipMalloc(&dr, n * 2));
    CHECK_HIP(hipMalloc(&dy, n * 2));
    CHECK_HIP(hipMalloc(&dro, n * 2));
    CHECK_HIP(hipMalloc(&dw, H * 2));
    CHECK_HIP(hipMalloc((void **)&drrms, M * 4));
    CHECK_HIP(hipMemcpy(dx, hx, n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dw, hw, H * 2, hipMemcpyHostToDevice));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));

    /* forward: rows of +-1 -> +-w */
    expect_ok("rmsnorm_fwd", rmsnorm_fwd(dx, H, dw, dy, H, drrms, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(hy, dy, n * 2, hipMemcpyDeviceToHost));
    expect_bits("rmsnorm_fwd y", hy, want, n);
    float hrr[M];
    CHECK_HIP(hipMemcpy(hrr, drrms, M * 4, hipMemcpyDeviceToHost));
    for (int i = 0; i < M; ++i)
        if (fabs(hrr[i] - 1.0 / sqrt(1.0 + (double)1e-5f)) > 1e-6) {
            printf("FAIL rrms[%d] = %.9g\n", i, hrr[i]);
            ++failures;
            break;
        }

    /* fused residual: x = +-1 everywhere ... with r = -0.5 * x gives h = +-0.5 */
    for (size_t i = 0; i < n; ++i) {
        const int neg = (int)((i / H + i % H) % 3 == 0);
        hr[i] = bf16(neg ? 0.5f : -0.5f);
    }
    CHECK_HIP(hipMemcpy(dr, hr, n * 2, hipMemcpyHostToDevice));
    expect_ok("rmsnorm_fwd_residual", rmsnorm_fwd_residual(dx, H, dr, H, dw, dy, H, dro, H, NULL, M, H, 1e-5f,
                                                           RMSN_BF16, RMSN_BF16, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(hy, dy, n * 2, hipMemcpyDeviceToHost));
    expect_bits("rmsnorm_fwd_residual y", hy, want, n);
    CHECK_HIP(hipMemcpy(hy, dro, n * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; ++i) {
        const int neg = (int)((i / H + i % H) % 3 == 0);
        want[i] = bf16(neg ? -0.5f : 0.5f);
    }
    expect_bits("rmsnorm_fwd_residual residual_out", hy, want, n);

    /* RoPE [2, 8, 4, 64] in place, quarter turns: position s turns by s * 90 degrees */
    enum { B = 2, S = 8, NH = 4, D = 64 };
    const size_t nq = (size_t)B * S * NH * D;
    uint16_t *hq = malloc(nq * 2), *hq2 = malloc(nq * 2), hc[S * D], hs[S * D];
    for (size_t i = 0; i < nq; ++i) hq[i] = bf16((float)((int)(i % 97) - 48) / 16.0f);
    for (int s = 0; s < S; ++s)
        for (int j = 0; j < D; ++j) {
            const int q = s % 4;
            hc[s * D + j] = bf16(q == 0 ? 1.0f : q == 2 ? -1.0f : 0.0f);
            hs[s * D + j] = bf16(q == 1 ? 1.0f : q == 3 ? -1.0f : 0.0f);
        }
    void *dq, *dc, *ds;
    CHECK_HIP(hipMalloc(&dq, nq * 2));
    CHECK_HIP(hipMalloc(&dc, S * D * 2));
    CHECK_HIP(hipMalloc(&ds, S * D * 2));
    CHECK_HIP(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dc, hc, S * D * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ds, hs, S * D * 2, hipMemcpyHostToDevice));
    expect_ok("rope_apply", rope_apply(dq, NH * D, D, dc, ds, D, dq, NH * D, D, B, S, NH, D, 0, RMSN_BF16, RMSN_BF16,
                                       stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(hq2, dq, nq * 2, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < S; ++s)
            for (int h = 0; h < NH; ++h)
                for (int j = 0; j < D / 2; ++j) {
                    const size_t base = (((size_t)b * S + s) * NH + h) * D;
                    const uint16_t x0 = hq[base + j], x1 = hq[base + j + D / 2];
                    const int q = s % 4;
                    /* out0 = x0 c - x1 s, out1 = x1 c + x0 s with (c, s) = (1,0), (0,1), (-1,0), (0,-1) */
                    const uint16_t w0 = q == 0 ? x0 : q == 1 ? (uint16_t)(x1 ^ 0x8000) : q == 2 ? (uint16_t)(x0 ^ 0x8000) : x1;
                    const uint16_t w1 = q == 0 ? x1 : q == 1 ? x0 : q == 2 ? (uint16_t)(x1 ^ 0x8000) : (uint16_t)(x0 ^ 0x8000);
                    const uint16_t g0 = hq2[base + j], g1 = hq2[base + j + D / 2];
                    /* +0 and -0 are the same value */
                    if ((g0 != w0 && ((g0 | w0) & 0x7fff)) || (g1 != w1 && ((g1 | w1) & 0x7fff))) {
                        printf("FAIL rope b=%d s=%d h=%d j=%d: 0x%04x 0x%04x, expected 0x%04x 0x%04x\n", b, s, h, j,
                               g0, g1, w0, w1);
                        ++failures;
                        b = B;
                        s = S;
                        h = NH;
                        break;
                    }
                }

    printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    hipFree(dx); hipFree(dr); hipFree(dy); hipFree(dro); hipFree(dw); hipFree(drrms);
    hipFree(dq); hipFree(dc); hipFree(ds);
    hipStreamDestroy(stream);
    free(hx); free(hr); free(hy); free(want); free(hq); free(hq2);
    return failures ? 1 : 0;
}
