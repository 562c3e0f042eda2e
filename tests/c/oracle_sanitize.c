/* Driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_sanitize_cpu.py together with oracle/rmsnorm_oracle.c).
 *
 * Every input buffer is allocated with exactly the bytes its shape and
 * strides reach (the last row ends at its H-th element; padding only between
 * rows), so a read past a row or a table by any oracle routine is a heap
 * overflow that ASan reports; outputs are allocated at their documented
 * dense sizes.  Inputs are random bit patterns: NaN, infinities, subnormals
 * and extremes included.  Every 16-bit pattern is decoded and encoded back,
 * and special doubles are encoded to every format.
 * Exit status 0 = every call returned as documented and no sanitizer fired. */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_decode(const void *src, int dt, int64_t n, double *out);
int orc_encode(const double *v, int64_t n, int dt, void *out);
int orc_fwd(const void *x, int64_t x_stride, const void *w, int x_dt, int w_dt, int64_t M, int64_t H, double eps,
            double *y, double *rrms);
int orc_fwd_residual(const void *x, int64_t x_stride, const void *res, int64_t r_stride, const void *w, int x_dt,
                     int w_dt, int64_t M, int64_t H, double eps, double *y, double *h, double *rrms);
int orc_bwd(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride, const void *w, const double *rrms,
            int x_dt, int w_dt, int64_t M, int64_t H, double *dx, double *dw, double *dx_terms);
int orc_adaln_fwd(const void *x, int64_t x_stride, const void *w, const void *scale, const void *shift,
                  int64_t cond_stride, int64_t rows_per_cond, int x_dt, int w_dt, int c_dt, int64_t M, int64_t H,
                  double eps, double *y, double *rrms);
int orc_bwd_residual(const void *dy, int64_t dy_stride, const void *h, int64_t h_stride, const void *dres,
                     int64_t dres_stride, const void *w, const double *rrms, int x_dt, int w_dt, int64_t M,
                     int64_t H, double *dh, double *dw, double *dh_terms);
int orc_rope(const void *x, int64_t x_row_stride, int64_t x_head_stride, const void *cos_t, const void *sin_t,
             int64_t table_stride, int x_dt, int t_dt, int64_t batch, int64_t seq_len, int64_t heads,
             int64_t head_dim, int transpose, double *out);
int orc_layernorm(const void *x, int64_t x_stride, const void *res, int64_t r_stride, const void *w, const void *b,
                  int x_dt, int w_dt, int64_t M, int64_t H, double eps, double *y, double *h_out, double *mean_out,
                  double *rstd_out);

static int failures = 0;
static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint64_t next(void) { /* SplitMix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }

static size_t esize(int dt) { return dt == 0 ? 4 : dt == 3 ? 8 : 2; }

/* n elements of format dt: exactly n * size bytes (at least one byte, so the
 * pointer is never NULL), filled with random bits */
static void *random_buf(int64_t n, int dt) {
    const size_t bytes = (size_t)n * esize(dt);
    unsigned char *p = malloc(bytes ? bytes : 1);
    for (size_t i = 0; i < bytes; ++i) p[i] = (unsigned char)next();
    return p;
}
/* elements reached by `rows` rows of `width` elements, `stride` apart */
static int64_t span(int64_t rows, int64_t stride, int64_t width) { return rows > 0 ? (rows - 1) * stride + width : 0; }
static double *dbuf(int64_t n) { return malloc(sizeof(double) * (size_t)(n > 0 ? n : 1)); }

static void expect_rc(const char *what, int rc, int want) {
    if (rc != want) {
        printf("FAIL %s: returned %d, expected %d\n", what, rc, want);
        ++failures;
    }
}

static void check_codecs(void) {
    uint16_t *all = malloc(65536 * 2), *back = malloc(65536 * 2);
    double *dec = dbuf(65536);
    for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
    for (int dt = 1; dt <= 2; ++dt) {
        expect_rc("decode every 16-bit pattern", orc_decode(all, dt, 65536, dec), 0);
        expect_rc("encode every decoded pattern", orc_encode(dec, 65536, dt, back), 0);
        for (int i = 0; i < 65536; ++i)
            if (!isnan(dec[i]) && back[i] != all[i]) {
                printf("FAIL format %d: pattern 0x%04x decodes and encodes to 0x%04x\n", dt, i, back[i]);
                ++failures;
                break;
            }
    }
    const double special[] = {0.0, -0.0, NAN, -NAN, INFINITY, -INFINITY, DBL_MAX, -DBL_MAX, DBL_MIN, 5e-324,
                              -5e-324, FLT_MAX, (double)FLT_MAX * 1.0000001, 65504.0, 65520.0, 65519.99, 1e-8,
                              5.960464477539063e-08, 2.9802322387695312e-08, 3.0e-08, 1.0, -1.0, 0.1};
    const int n = (int)(sizeof special / sizeof special[0]);
    unsigned char out[8 * 32];
    for (int dt = 0; dt <= 3; ++dt) expect_rc("encode special doubles", orc_encode(special, n, dt, out), 0);
    /* random doubles of every exponent */
    double r[4096];
    for (int i = 0; i < 4096; ++i) {
        uint64_t u = next();
        memcpy(&r[i], &u, sizeof u);
    }
    for (int dt = 0; dt <= 3; ++dt) {
        void *o = malloc(4096 * esize(dt));
        expect_rc("encode random doubles", orc_encode(r, 4096, dt, o), 0);
        free(o);
    }
    free(all);
    free(back);
    free(dec);
}

static void check_norms(int iters) {
    for (int it = 0; it < iters; ++it) {
        const int64_t M = pick(0, 5), H = pick(1, 70);
        const int xdt = (int)pick(0, 3), wdt = (int)pick(0, 3);
        const int64_t xs = H + pick(0, 5), rs = H + pick(0, 5), cs = H + pick(0, 3);
        const int weighted = (int)pick(0, 1);
        const double eps = pick(0, 1) ? 1e-5 : 1e-30;
        void *x = random_buf(span(M, xs, H), xdt), *r = random_buf(span(M, rs, H), xdt);
        void *w = weighted ? random_buf(H, wdt) : NULL;
        double *y = dbuf(M * H), *h = dbuf(M * H), *rr = dbuf(M), *terms = dbuf(M * H), *dw = dbuf(H);
        expect_rc("orc_fwd", orc_fwd(x, xs, w, xdt, wdt, M, H, eps, y, rr), 0);
        expect_rc("orc_fwd_residual", orc_fwd_residual(x, xs, r, rs, w, xdt, wdt, M, H, eps, y, h, rr), 0);
        /* backward from positive rrms values (any finite value is legal) */
        for (int64_t i = 0; i < M; ++i) rr[i] = 0.5 + (double)(next() % 1000) / 500.0;
        expect_rc("orc_bwd", orc_bwd(r, rs, x, xs, w, rr, xdt, wdt, M, H, y, weighted ? dw : NULL, terms), 0);
        expect_rc("orc_bwd_residual",
                  orc_bwd_residual(r, rs, x, xs, x, xs, w, rr, xdt, wdt, M, H, y, weighted ? dw : NULL, terms), 0);
        /* AdaLN: one conditioning row per row, or per block of rows */
        const int64_t rpc = pick(1, 4), ncond = M > 0 ? (M - 1) / rpc + 1 : 0;
        const int cdt = (int)pick(0, 3);
        void *sc = random_buf(span(ncond, cs, H), cdt), *sh = random_buf(span(ncond, cs, H), cdt);
        expect_rc("orc_adaln_fwd", orc_adaln_fwd(x, xs, w, sc, sh, cs, rpc, xdt, wdt, cdt, M, H, eps, y, rr), 0);
        /* LayerNorm, with and without the residual, weight and bias */
        void *b = pick(0, 1) ? random_buf(H, wdt) : NULL;
        expect_rc("orc_layernorm", orc_layernorm(x, xs, pick(0, 1) ? r : NULL, rs, w, b, xdt, wdt, M, H, eps, y, h,
                                                 rr, terms),
                  0);
        free(x), free(r), free(w), free(sc), free(sh), free(b);
        free(y), free(h), free(rr), free(terms), free(dw);
    }
}

static void check_rope(int iters) {
    for (int it = 0; it < iters; ++it) {
        const int64_t B = pick(0, 3), S = pick(1, 9), NH = pick(1, 5), D = 2 * pick(1, 20);
        const int64_t hs = D + pick(0, 4), rs = NH * hs + pick(0, 6), ts = D / 2 + pick(0, 5);  /* the oracle reads rows of NH * hs */
        const int xdt = (int)pick(0, 3), tdt = (int)pick(0, 3);
        void *x = random_buf(span(B * S, rs, (NH - 1) * hs + D), xdt);
        void *c = random_buf(span(S, ts, D / 2), tdt), *s = random_buf(span(S, ts, D / 2), tdt);
        double *out = dbuf(B * S * NH * D);
        expect_rc("orc_rope", orc_rope(x, rs, hs, c, s, ts, xdt, tdt, B, S, NH, D, (int)pick(0, 1), out), 0);
        free(x), free(c), free(s), free(out);
    }
}

static void check_rejections(void) {
    double y[4], rr[2];
    float x[8] = {0};
    expect_rc("fwd: H < 1", orc_fwd(x, 1, NULL, 0, 0, 1, 0, 1e-5, y, rr), -1);
    expect_rc("fwd: stride < H", orc_fwd(x, 1, NULL, 0, 0, 1, 2, 1e-5, y, rr), -1);
    expect_rc("fwd: eps <= 0", orc_fwd(x, 2, NULL, 0, 0, 1, 2, 0.0, y, rr), -1);
    expect_rc("fwd: eps NaN", orc_fwd(x, 2, NULL, 0, 0, 1, 2, NAN, y, rr), -1);
    expect_rc("fwd: bad format", orc_fwd(x, 2, NULL, 9, 0, 1, 2, 1e-5, y, rr), -1);
    expect_rc("bwd: dw without w", orc_bwd(x, 2, x, 2, NULL, rr, 0, 0, 1, 2, y, y, NULL), -1);
    expect_rc("rope: odd head_dim", orc_rope(x, 3, 3, x, x, 2, 0, 0, 1, 1, 1, 3, 0, y), -1);
    expect_rc("rope: table too narrow", orc_rope(x, 4, 4, x, x, 1, 0, 0, 1, 1, 1, 4, 0, y), -1);
    expect_rc("layernorm: negative eps", orc_layernorm(x, 2, NULL, 2, NULL, NULL, 0, 0, 1, 2, -1.0, y, NULL, NULL,
                                                       NULL),
              -1);
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 400;
    check_codecs();
    check_norms(iters);
    check_rope(iters);
    check_rejections();
    printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
    return failures ? 1 : 0;
}
