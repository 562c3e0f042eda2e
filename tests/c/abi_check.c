/* Plain C client of librmsnorm.so: checks that include/rmsnorm.h compiles as
 * C and that argument errors are reported before any device work.  Pointers
 * are never dereferenced: every call below fails validation on the host.
 * Exit status 0 = all checks passed. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "layernorm.h"
#include "rmsnorm.h"
#include "rmsnorm_tuning.h"
#include "rope.h"

static int failures = 0;

static void expect(const char *what, rmsn_status_t got, rmsn_status_t want) {
    if (got != want) {
        printf("FAIL %s: got %s want %s (%s)\n", what, rmsnorm_status_string(got), rmsnorm_status_string(want),
               rmsnorm_last_error());
        ++failures;
    } else if (want != RMSN_OK && rmsnorm_last_error()[0] == '\0') {
        printf("FAIL %s: no error detail\n", what);
        ++failures;
    }
}

int main(void) {
    /* fake, 256-byte aligned device addresses far apart; never dereferenced */
    void *x = (void *)(uintptr_t)0x100000000ull;
    void *y = (void *)(uintptr_t)0x200000000ull;
    void *w = (void *)(uintptr_t)0x300000000ull;
    void *r = (void *)(uintptr_t)0x400000000ull;
    float *rr = (float *)(uintptr_t)0x500000000ull;
    void *ws = (void *)(uintptr_t)0x600000000ull;
    float *dw = (float *)(uintptr_t)0x700000000ull;
    const int64_t M = 64, H = 4096;

    expect("M == 0 is a no-op", rmsnorm_fwd(NULL, H, NULL, NULL, H, NULL, 0, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_OK);
    if (rmsnorm_last_error()[0] != '\0') { printf("FAIL error detail not cleared\n"); ++failures; }
    expect("x NULL", rmsnorm_fwd(NULL, H, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("y NULL", rmsnorm_fwd(x, H, w, NULL, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("H 0", rmsnorm_fwd(x, H, w, y, H, rr, M, 0, 1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("M < 0", rmsnorm_fwd(x, H, w, y, H, rr, -1, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("stride < H", rmsnorm_fwd(x, H - 1, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("eps 0", rmsnorm_fwd(x, H, w, y, H, rr, M, H, 0.0f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("eps < 0", rmsnorm_fwd(x, H, w, y, H, rr, M, H, -1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("eps NaN", rmsnorm_fwd(x, H, w, y, H, rr, M, H, NAN, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("eps inf", rmsnorm_fwd(x, H, w, y, H, rr, M, H, INFINITY, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("bad dtype", rmsnorm_fwd(x, H, w, y, H, rr, M, H, 1e-5f, (rmsn_dtype_t)7, RMSN_BF16, 0),
           RMSN_ERR_UNSUPPORTED);
    expect("w f16 with x bf16", rmsnorm_fwd(x, H, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_F16, 0),
           RMSN_ERR_UNSUPPORTED);
    expect("H > 2^30", rmsnorm_fwd(x, (int64_t)1 << 31, w, y, (int64_t)1 << 31, rr, 1, (int64_t)1 << 31, 1e-5f,
                                   RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_UNSUPPORTED);
    expect("y partially overlaps x",
           rmsnorm_fwd(x, H, w, (char *)x + 2 * H, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("y same start as x but other stride",
           rmsnorm_fwd(x, H, w, x, 2 * H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("rrms inside x", rmsnorm_fwd(x, H, w, y, H, (float *)x, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("rrms inside y", rmsnorm_fwd(x, H, w, y, H, (float *)((char *)y + 64), M, H, 1e-5f, RMSN_BF16,
                                        RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("stride overflow", rmsnorm_fwd(x, INT64_MAX / 2, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);

    expect("residual NULL", rmsnorm_fwd_residual(x, H, NULL, H, w, y, H, r, H, rr, M, H, 1e-5f, RMSN_BF16,
                                                 RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("residual_out overlaps y", rmsnorm_fwd_residual(x, H, r, H, w, y, H, (char *)y + 16, H, rr, M, H, 1e-5f,
                                                           RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("residual_out == y", rmsnorm_fwd_residual(x, H, r, H, w, y, H, y, H, rr, M, H, 1e-5f, RMSN_BF16,
                                                     RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("r_stride < H", rmsnorm_fwd_residual(x, H, r, 8, w, y, H, NULL, 0, rr, M, H, 1e-5f, RMSN_BF16,
                                                RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("residual M == 0", rmsnorm_fwd_residual(NULL, H, NULL, H, NULL, NULL, H, NULL, H, NULL, 0, H, 1e-5f,
                                                   RMSN_F16, RMSN_F32, 0), RMSN_OK);

    void *sc = (void *)(uintptr_t)0x800000000ull, *sh = (void *)(uintptr_t)0x900000000ull;
    expect("adaln scale NULL", rmsnorm_adaln_fwd(x, H, w, NULL, sh, H, 1, y, H, rr, M, H, 1e-5f, RMSN_BF16,
                                                 RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("adaln rows_per_cond 0", rmsnorm_adaln_fwd(x, H, w, sc, sh, H, 0, y, H, rr, M, H, 1e-5f, RMSN_BF16,
                                                      RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("adaln cond_stride < H", rmsnorm_adaln_fwd(x, H, w, sc, sh, H - 8, 1, y, H, rr, M, H, 1e-5f, RMSN_BF16,
                                                      RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("adaln param f16 with x bf16", rmsnorm_adaln_fwd(x, H, NULL, sc, sh, H, 1, y, H, rr, M, H, 1e-5f,
                                                            RMSN_BF16, RMSN_F16, 0), RMSN_ERR_UNSUPPORTED);
    expect("adaln y overlaps shift", rmsnorm_adaln_fwd(x, H, w, sc, sh, H, 1, (char *)sh + 32, H, rr, M, H, 1e-5f,
                                                       RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("adaln M == 0", rmsnorm_adaln_fwd(NULL, H, NULL, NULL, NULL, H, 1, NULL, H, NULL, 0, H, 1e-5f, RMSN_BF16,
                                             RMSN_F32, 0), RMSN_OK);

    size_t need = rmsnorm_bwd_workspace_bytes(M, H);
    if (need != (size_t)M * H * 4) { printf("FAIL workspace size %zu\n", need); ++failures; }
    if (rmsnorm_bwd_workspace_bytes(1 << 20, 6144) != (size_t)1024 * 6144 * 4) {
        printf("FAIL workspace cap\n"); ++failures;
    }
    if (rmsnorm_bwd_workspace_bytes(0, H) != 0 || rmsnorm_bwd_workspace_bytes(M, 0) != 0) {
        printf("FAIL empty workspace\n"); ++failures;
    }
    expect("dw without w", rmsnorm_bwd(r, H, x, H, NULL, rr, y, H, dw, ws, need, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("workspace NULL", rmsnorm_bwd(r, H, x, H, w, rr, y, H, dw, NULL, need, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_WORKSPACE);
    expect("workspace small", rmsnorm_bwd(r, H, x, H, w, rr, y, H, dw, ws, need - 1, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_WORKSPACE);
    expect("workspace misaligned", rmsnorm_bwd(r, H, x, H, w, rr, y, H, dw, (char *)ws + 4, need, M, H, RMSN_BF16,
                                               RMSN_BF16, 0), RMSN_ERR_WORKSPACE);
    expect("rrms NULL", rmsnorm_bwd(r, H, x, H, w, NULL, y, H, dw, ws, need, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("dw overlaps workspace", rmsnorm_bwd(r, H, x, H, w, rr, y, H, (float *)ws, ws, need, M, H, RMSN_BF16,
                                                RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("dx overlaps rrms", rmsnorm_bwd(r, H, x, H, w, (float *)y, y, H, dw, ws, need, M, H, RMSN_BF16,
                                           RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("workspace overlaps x", rmsnorm_bwd(r, H, x, H, w, rr, y, H, dw, x, need, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("bwd M == 0 without dw", rmsnorm_bwd(NULL, H, NULL, H, NULL, NULL, NULL, H, NULL, NULL, 0, 0, H,
                                                RMSN_BF16, RMSN_BF16, 0), RMSN_OK);

    /* the no-allocation backward validates as rmsnorm_bwd, with no workspace */
    expect("noalloc dw without w", rmsnorm_bwd_noalloc(r, H, x, H, NULL, rr, y, H, dw, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("noalloc rrms NULL", rmsnorm_bwd_noalloc(r, H, x, H, w, NULL, y, H, dw, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("noalloc dx overlaps rrms", rmsnorm_bwd_noalloc(r, H, x, H, w, (float *)y, y, H, dw, M, H, RMSN_BF16,
                                                           RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("noalloc stride < H", rmsnorm_bwd_noalloc(r, H - 1, x, H, w, rr, y, H, dw, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("noalloc bad dtype", rmsnorm_bwd_noalloc(r, H, x, H, w, rr, y, H, dw, M, H, (rmsn_dtype_t)7, RMSN_BF16, 0),
           RMSN_ERR_UNSUPPORTED);
    expect("noalloc M == 0 without dw", rmsnorm_bwd_noalloc(NULL, H, NULL, H, NULL, NULL, NULL, H, NULL, 0, H,
                                                            RMSN_BF16, RMSN_BF16, 0), RMSN_OK);
    /* with valid arguments the call needs the device (the partial-row count
       depends on its compute units): no device here, so a HIP error */
    expect("noalloc needs the device", rmsnorm_bwd_noalloc(r, H, x, H, w, rr, y, H, dw, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_HIP);

    /* the tile query is host only */
    {
        int32_t t[6];
        expect("tile query", rmsnorm_tuning_tile(0, 4096, RMSN_BF16, 0, t), RMSN_OK);
        if (t[0] != 8 || t[1] * t[2] * 64 < 512 || t[4] != 0 || t[5] != 0) {
            printf("FAIL tile query: vec %d vpt %d wpr %d mis %d multi %d\n", t[0], t[1], t[2], t[4], t[5]);
            ++failures;
        }
        expect("tile query off grid", rmsnorm_tuning_tile(1, 4097, RMSN_BF16, 1, t), RMSN_OK);
        if (t[4] != 1) { printf("FAIL tile query off grid: mis %d\n", t[4]); ++failures; }
        expect("tile query NULL", rmsnorm_tuning_tile(0, 4096, RMSN_BF16, 0, NULL), RMSN_ERR_INVALID_ARG);
        expect("tile query bad op", rmsnorm_tuning_tile(7, 4096, RMSN_BF16, 0, t), RMSN_ERR_INVALID_ARG);
        expect("tile query H 0", rmsnorm_tuning_tile(0, 0, RMSN_BF16, 0, t), RMSN_ERR_INVALID_ARG);
        expect("tile query bad dtype", rmsnorm_tuning_tile(0, 64, (rmsn_dtype_t)9, 0, t), RMSN_ERR_UNSUPPORTED);
    }

    void *g = (void *)(uintptr_t)0xa00000000ull;
    expect("bwd_residual dres_stride < H", rmsnorm_bwd_residual(r, H, x, H, g, H - 8, w, rr, y, H, dw, ws, need, M,
                                                                H, RMSN_BF16, RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("bwd_residual dh partially overlaps dres",
           rmsnorm_bwd_residual(r, H, x, H, g, H, w, rr, (char *)g + 16, H, dw, ws, need, M, H, RMSN_BF16,
                                RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("bwd_residual workspace overlaps dres",
           rmsnorm_bwd_residual(r, H, x, H, g, H, w, rr, y, H, dw, g, need, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("bwd_residual workspace small",
           rmsnorm_bwd_residual(r, H, x, H, g, H, w, rr, y, H, dw, ws, need - 16, M, H, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_WORKSPACE);
    expect("bwd_residual M == 0", rmsnorm_bwd_residual(NULL, H, NULL, H, NULL, H, NULL, NULL, NULL, H, NULL, NULL, 0,
                                                       0, H, RMSN_BF16, RMSN_BF16, 0), RMSN_OK);

    /* LayerNorm */
    expect("ln eps 0", layernorm_fwd(x, H, w, r, y, H, NULL, NULL, M, H, 0.0f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    expect("ln bias f16 with x bf16", layernorm_fwd(x, H, NULL, r, y, H, NULL, NULL, M, H, 1e-5f, RMSN_BF16,
                                                    RMSN_F16, 0), RMSN_ERR_UNSUPPORTED);
    expect("ln mean overlaps x", layernorm_fwd(x, H, w, NULL, y, H, (float *)x, NULL, M, H, 1e-5f, RMSN_BF16,
                                               RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("ln y overlaps bias", layernorm_fwd(x, H, w, (char *)y + 64, y, H, NULL, NULL, M, H, 1e-5f, RMSN_BF16,
                                               RMSN_BF16, 0), RMSN_ERR_INVALID_ARG);
    expect("ln residual NULL", layernorm_fwd_residual(x, H, NULL, H, w, NULL, y, H, NULL, 0, NULL, NULL, M, H, 1e-5f,
                                                      RMSN_F32, RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("ln M == 0", layernorm_fwd_residual(NULL, H, NULL, H, NULL, NULL, NULL, H, NULL, H, NULL, NULL, 0, H,
                                               1e-5f, RMSN_F32, RMSN_F32, 0), RMSN_OK);

    /* RoPE: x [2, 8, 4, 64] */
    const int64_t rs = 4 * 64;
    expect("rope odd head_dim", rope_apply(x, rs, 64, w, r, 64, y, rs, 64, 2, 8, 4, 63, 0, RMSN_BF16, RMSN_F32, 0),
           RMSN_ERR_INVALID_ARG);
    expect("rope head stride < head_dim", rope_apply(x, rs, 32, w, r, 64, y, rs, 64, 2, 8, 4, 64, 0, RMSN_BF16,
                                                     RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("rope row stride too small", rope_apply(x, 3 * 64, 64, w, r, 64, y, rs, 64, 2, 8, 4, 64, 0, RMSN_BF16,
                                                   RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("rope table stride < head_dim/2", rope_apply(x, rs, 64, w, r, 16, y, rs, 64, 2, 8, 4, 64, 0, RMSN_BF16,
                                                        RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("rope f16 tables for bf16 x", rope_apply(x, rs, 64, w, r, 64, y, rs, 64, 2, 8, 4, 64, 0, RMSN_BF16,
                                                    RMSN_F16, 0), RMSN_ERR_UNSUPPORTED);
    expect("rope out over the cos table", rope_apply(x, rs, 64, w, r, 64, (char *)w + 16, rs, 64, 2, 8, 4, 64, 0,
                                                     RMSN_BF16, RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("rope out partially over x", rope_apply(x, rs, 64, w, r, 64, (char *)x + 32, rs, 64, 2, 8, 4, 64, 0,
                                                   RMSN_BF16, RMSN_F32, 0), RMSN_ERR_INVALID_ARG);
    expect("rope seq_len 0", rope_apply(x, rs, 64, w, r, 64, y, rs, 64, 2, 0, 4, 64, 0, RMSN_BF16, RMSN_F32, 0),
           RMSN_ERR_INVALID_ARG);
    expect("rope batch 0", rope_apply(NULL, rs, 64, NULL, NULL, 64, NULL, rs, 64, 0, 8, 4, 64, 0, RMSN_BF16,
                                      RMSN_F32, 0), RMSN_OK);

    expect("copy odd address", rmsnorm_tuning_copy((char *)x + 1, y, 4096, 0), RMSN_ERR_INVALID_ARG);
    expect("copy odd size", rmsnorm_tuning_copy(x, y, 4100, 0), RMSN_ERR_INVALID_ARG);
    expect("copy overlap", rmsnorm_tuning_copy(x, (char *)x + 4096, 8192, 0), RMSN_ERR_INVALID_ARG);
    expect("copy nothing", rmsnorm_tuning_copy(x, y, 0, 0), RMSN_OK);

    /* a geometry that cannot cover the row is rejected before the device */
    rmsnorm_tuning_set_geometry(0, 3, 1, 1, 0);
    expect("override too small", rmsnorm_fwd(x, H, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    rmsnorm_tuning_set_geometry(0, 2, 32, 1, 0);
    expect("override too many threads", rmsnorm_fwd(x, H, w, y, H, rr, M, H, 1e-5f, RMSN_BF16, RMSN_BF16, 0),
           RMSN_ERR_INVALID_ARG);
    rmsnorm_tuning_set_geometry(0, 0, 0, 0, 0);

    if (strcmp(rmsnorm_status_string(RMSN_ERR_WORKSPACE), "RMSN_ERR_WORKSPACE") != 0) {
        printf("FAIL status string\n"); ++failures;
    }
    printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
