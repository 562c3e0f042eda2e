/*
 * rmsnorm_oracle.c -- slow, plain float64 CPU definition of RMSNorm, its fused
 * residual pre-norm form and its backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources (the page "Skill: Write a Triton RMSNorm Kernel", ahel.ai):
 *   - "Purpose": y = x * rsqrt(mean(x^2 over the last axis) + eps) * weight.
 *   - "Required reasoning process", steps 5-8: the mean divides by H, the
 *     full row length; eps sits inside the square root; the weight has shape
 *     (H,) and is indexed by column only; there is no bias and no mean
 *     subtraction ("Correctness requirements").
 *   - "Use this when" and "Kernel design rules": the fused pre-norm adds the
 *     residual before squaring and may write the sum back as the next
 *     residual stream.
 *   - "Required reasoning process", step 12: with xn = x * rrms and the saved
 *     per-row rrms, dx = rrms*(dy*w) - (xn*rrms/H) * sum_h(dy*w*xn), and
 *     dweight = sum over rows of dy*xn, shape (H,).
 *   - The weightless form (no weight, LTX-Video's elementwise_affine=False)
 *     is the page "rocm-kernels" (skillselion.com), "Core Kernel
 *     Implementations", RMSNorm: out = x * rms_inv when there is no weight.
 *   - Backward of the fused residual pre-norm (h = x + r, y = RMSNorm(h), and
 *     h written back as the next residual stream): both x and r receive
 *     dh = d(norm)/dh . dy + d(residual_out), the gradient of y through the
 *     norm plus the gradient arriving on the residual stream (the chain rule
 *     through the sum; the page only states the forward fusion).
 *   - AdaLN: the same page, "Core Kernel Implementations", 4. AdaLN, and its
 *     "Template 4": norm(x) * weight * (1 + scale) + shift, with scale and
 *     shift one row per token ([B, S, H]) or one row per batch ([B, 1, H]).
 *   - RoPE apply (the same page, "Core Kernel Implementations", 2. RoPE 3D,
 *     and "Triton kernel templates", Template 2): q or k of shape
 *     [batch, seq_len, heads, head_dim] is rotated pairwise in the
 *     rotate-half layout, element j with element j + head_dim/2, by the angle
 *     whose cos and sin sit at column j of the token's row of [seq_len,
 *     head_dim] tables; with the batch folded into the rows, the table row is
 *     the flat row index modulo seq_len.  Only the first head_dim/2 columns of
 *     a table row are read.  The transposed rotation (sin negated) is the
 *     gradient of the rotation with respect to its input, and its inverse.
 *   - Residual + LayerNorm (the page "SpeedROCm: shape-aware Triton
 *     acceleration for Transformer inference", "How the solution addresses
 *     the problem", item 4: each residual add fused with the LayerNorm that
 *     consumes it, in a pre-LayerNorm transformer).  LayerNorm is the one the
 *     page names among its runtime interfaces (torch.nn's): over the last
 *     axis, mean and population (biased) variance, eps inside the square
 *     root, then the optional elementwise weight and bias:
 *       h = x + r,  y = (h - mean(h)) / sqrt(var(h) + eps) * w + b.
 *
 * Everything is computed in IEEE float64 from exactly decoded inputs, one row
 * at a time, in the plain left-to-right order of the definition.  Rounding to
 * a storage format is round-to-nearest-even (a reading: the pages only say the
 * result is converted to the output dtype).
 *
 * Storage codes used by this file: 0 = float32, 1 = float16, 2 = bfloat16,
 * 3 = float64 (float64 is for finite-difference checks only).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_F64 = 3 };

static int orc_valid_code(int dt) { return dt >= ORC_F32 && dt <= ORC_F64; }

/* ---- exact decoding ---------------------------------------------------- */

static double decode_f16_bits(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 10) & 0x1f;
    int f = b & 0x3ff;
    double v;
    if (e == 0x1f) {
        v = f ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    } else {
        v = ldexp((double)(f | 0x400), e - 25); /* (1024+f) * 2^(e-15-10) */
    }
    return sign ? -v : v;
}

static double decode_bf16_bits(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dt, int64_t i) {
    switch (dt) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_F16: return decode_f16_bits(((const uint16_t *)base)[i]);
    case ORC_BF16: return decode_bf16_bits(((const uint16_t *)base)[i]);
    default: return ((const double *)base)[i];
    }
}

/* ---- round-to-nearest-even encoding -------------------------------------- */

/* Round |a| (finite, > 0) to a binary format with p significand bits and
 * smallest normal exponent emin; returns the rounded magnitude (may be +inf
 * when it exceeds the largest finite value maxf). */
static double round_magnitude(double a, int p, int emin, double maxf) {
    int e;
    frexp(a, &e);          /* a = m * 2^e with m in [0.5, 1) */
    int lead = e - 1;      /* exponent of the leading bit */
    if (lead < emin) lead = emin; /* subnormal range keeps a fixed quantum */
    double quantum = ldexp(1.0, lead - (p - 1));
    double q = rint(a / quantum); /* rint: round half to even (default mode) */
    double r = q * quantum;
    return r > maxf ? INFINITY : r;
}

static uint16_t encode_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7e00);
    double a = fabs(v);
    if (a == 0.0) return sign;
    double r = isinf(a) ? INFINITY : round_magnitude(a, 11, -14, 65504.0);
    if (isinf(r)) return (uint16_t)(sign | 0x7c00);
    if (r < ldexp(1.0, -14)) { /* subnormal: r = f * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    }
    int e;
    double m = frexp(r, &e); /* r = m * 2^e, m in [0.5,1) */
    int biased = (e - 1) + 15;
    uint16_t frac = (uint16_t)(ldexp(m, 11) - 1024.0);
    return (uint16_t)(sign | (uint16_t)(biased << 10) | frac);
}

static uint16_t encode_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7fc0);
    double a = fabs(v);
    if (a == 0.0) return sign;
    const double maxf = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    double r = isinf(a) ? INFINITY : round_magnitude(a, 8, -126, maxf);
    if (isinf(r)) return (uint16_t)(sign | 0x7f80);
    /* r has at most 8 significant bits, so it is exact in float32 and its low
     * 16 bits there are zero */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

static float encode_f32(double v) {
    if (isnan(v)) return (float)v;
    double a = fabs(v);
    if (a == 0.0 || isinf(a)) return (float)v;
    const double maxf = ldexp(16777215.0, 104); /* (2 - 2^-23) * 2^127 */
    double r = round_magnitude(a, 24, -126, maxf);
    float f = (float)r; /* exact: r already has float32 precision */
    return signbit(v) ? -f : f;
}

/* ---- exported helpers ---------------------------------------------------- */

int orc_decode(const void *src, int dt, int64_t n, double *out) {
    if (!orc_valid_code(dt) || n < 0 || (n > 0 && (!src || !out))) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(src, dt, i);
    return 0;
}

int orc_encode(const double *v, int64_t n, int dt, void *out) {
    if (!orc_valid_code(dt) || n < 0 || (n > 0 && (!v || !out))) return -1;
    for (int64_t i = 0; i < n; ++i) {
        switch (dt) {
        case ORC_F32: ((float *)out)[i] = encode_f32(v[i]); break;
        case ORC_F16: ((uint16_t *)out)[i] = encode_f16(v[i]); break;
        case ORC_BF16: ((uint16_t *)out)[i] = encode_bf16(v[i]); break;
        default: ((double *)out)[i] = v[i]; break;
        }
    }
    return 0;
}

/* ---- forward --------------------------------------------------------------
 * For each row i: ss = sum_j x_ij^2; ms = ss / H; rrms_i = 1 / sqrt(ms + eps);
 * y_ij = x_ij * rrms_i * w_j, with w_j = 1 when w is NULL (weightless).
 * x rows are x_stride elements apart; y is dense float64 (M, H); rrms (M,)
 * may be NULL.  Returns 0, or -1 on a bad argument.
 */
int orc_fwd(const void *x, int64_t x_stride, const void *w, int x_dt, int w_dt,
            int64_t M, int64_t H, double eps, double *y, double *rrms) {
    if (!orc_valid_code(x_dt) || (w && !orc_valid_code(w_dt))) return -1;
    if (M < 0 || H < 1 || x_stride < H || !(eps > 0.0)) return -1;
    if (M > 0 && (!x || !y)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        const int64_t row = i * x_stride;
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, row + j);
            ss += v * v;
        }
        double ms = ss / (double)H;
        double r = 1.0 / sqrt(ms + eps);
        if (rrms) rrms[i] = r;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, row + j);
            double wj = w ? load_elem(w, w_dt, j) : 1.0;
            y[i * H + j] = v * r * wj;
        }
    }
    return 0;
}

/* ---- fused residual pre-norm ----------------------------------------------
 * h_ij = x_ij + res_ij (float64; exact for the 16- and 32-bit formats);
 * h (dense (M, H) float64) is the post-add residual stream before rounding;
 * y is orc_fwd applied to the unrounded h.
 */
int orc_fwd_residual(const void *x, int64_t x_stride, const void *res, int64_t r_stride,
                     const void *w, int x_dt, int w_dt, int64_t M, int64_t H, double eps,
                     double *y, double *h, double *rrms) {
    if (!orc_valid_code(x_dt) || (w && !orc_valid_code(w_dt))) return -1;
    if (M < 0 || H < 1 || x_stride < H || r_stride < H || !(eps > 0.0)) return -1;
    if (M > 0 && (!x || !res || !y || !h)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, i * x_stride + j) + load_elem(res, x_dt, i * r_stride + j);
            h[i * H + j] = v;
            ss += v * v;
        }
        double ms = ss / (double)H;
        double r = 1.0 / sqrt(ms + eps);
        if (rrms) rrms[i] = r;
        for (int64_t j = 0; j < H; ++j) {
            double wj = w ? load_elem(w, w_dt, j) : 1.0;
            y[i * H + j] = h[i * H + j] * r * wj;
        }
    }
    return 0;
}

/* ---- backward -------------------------------------------------------------
 * Given the saved per-row rrms r_i (passed in, never recomputed):
 *   xn_ij = x_ij * r_i,  g_ij = dy_ij * w_j  (w_j = 1 when weightless)
 *   c_i   = sum_j g_ij * xn_ij
 *   dx_ij = r_i * g_ij - xn_ij * r_i * c_i / H
 *   dw_j  = sum_i dy_ij * xn_ij        (only when w is given; dw may be NULL)
 * dx is dense float64 (M, H).  dx_terms, when not NULL, receives
 * |r_i*g_ij| + |xn_ij*r_i*c_i/H| per element: the size of the two terms whose
 * difference dx is, used to judge cancellation.
 */
int orc_bwd(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride,
            const void *w, const double *rrms, int x_dt, int w_dt, int64_t M, int64_t H,
            double *dx, double *dw, double *dx_terms) {
    if (!orc_valid_code(x_dt) || (w && !orc_valid_code(w_dt))) return -1;
    if (M < 0 || H < 1 || x_stride < H || dy_stride < H) return -1;
    if (M > 0 && (!x || !dy || !rrms || !dx)) return -1;
    if (dw && !w) return -1;
    if (dw)
        for (int64_t j = 0; j < H; ++j) dw[j] = 0.0;
    for (int64_t i = 0; i < M; ++i) {
        const double r = rrms[i];
        double c = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double xn = load_elem(x, x_dt, i * x_stride + j) * r;
            double g = load_elem(dy, x_dt, i * dy_stride + j) * (w ? load_elem(w, w_dt, j) : 1.0);
            c += g * xn;
        }
        for (int64_t j = 0; j < H; ++j) {
            double xv = load_elem(x, x_dt, i * x_stride + j);
            double dyv = load_elem(dy, x_dt, i * dy_stride + j);
            double xn = xv * r;
            double g = dyv * (w ? load_elem(w, w_dt, j) : 1.0);
            double t1 = r * g;
            double t2 = xn * r * c / (double)H;
            dx[i * H + j] = t1 - t2;
            if (dx_terms) dx_terms[i * H + j] = fabs(t1) + fabs(t2);
            if (dw) dw[j] += dyv * xn;
        }
    }
    return 0;
}

/* ---- AdaLN-RMSNorm --------------------------------------------------------
 * y_ij = x_ij * rrms_i * w_j * (1 + scale_cj) + shift_cj, with c = i / rows_per_cond
 * (rows_per_cond = 1: one conditioning row per row; = S: one per batch of S
 * rows).  scale and shift rows are cond_stride elements apart, in c_dt.
 */
int orc_adaln_fwd(const void *x, int64_t x_stride, const void *w, const void *scale, const void *shift,
                  int64_t cond_stride, int64_t rows_per_cond, int x_dt, int w_dt, int c_dt, int64_t M, int64_t H,
                  double eps, double *y, double *rrms) {
    if (!orc_valid_code(x_dt) || !orc_valid_code(c_dt) || (w && !orc_valid_code(w_dt))) return -1;
    if (M < 0 || H < 1 || x_stride < H || cond_stride < H || rows_per_cond < 1 || !(eps > 0.0)) return -1;
    if (M > 0 && (!x || !y || !scale || !shift)) return -1;
    for (int64_t i = 0; i < M; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, i * x_stride + j);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        if (rrms) rrms[i] = r;
        const int64_t c = i / rows_per_cond;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, i * x_stride + j);
            double wj = w ? load_elem(w, w_dt, j) : 1.0;
            double sc = load_elem(scale, c_dt, c * cond_stride + j);
            double sh = load_elem(shift, c_dt, c * cond_stride + j);
            y[i * H + j] = v * r * wj * (1.0 + sc) + sh;
        }
    }
    return 0;
}

/* ---- backward of the fused residual pre-norm -------------------------------
 * dh_ij = (orc_bwd dx of dy through the norm of h)_ij + dres_ij, where h is
 * the post-add stream (as stored, h_stride apart) and dres the gradient that
 * arrives on the residual-stream output (NULL = 0).  dw as orc_bwd.
 */
int orc_bwd_residual(const void *dy, int64_t dy_stride, const void *h, int64_t h_stride, const void *dres,
                     int64_t dres_stride, const void *w, const double *rrms, int x_dt, int w_dt, int64_t M,
                     int64_t H, double *dh, double *dw, double *dh_terms) {
    int rc = orc_bwd(dy, dy_stride, h, h_stride, w, rrms, x_dt, w_dt, M, H, dh, dw, dh_terms);
    if (rc != 0) return rc;
    if (dres) {
        if (dres_stride < H) return -1;
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < H; ++j) {
                double d = load_elem(dres, x_dt, i * dres_stride + j);
                dh[i * H + j] += d;
                if (dh_terms) dh_terms[i * H + j] += fabs(d);
            }
    }
    return 0;
}

/* ---- RoPE apply (rotate-half) ------------------------------------------------
 * x: rows = batch * seq_len token rows, row r at r * x_row_stride, head h at
 * + h * x_head_stride, head_dim contiguous elements.  cos and sin: seq_len
 * rows table_stride apart (>= head_dim / 2 columns read).  out: float64,
 * contiguous (rows, heads, head_dim).  For each token row r, head h and
 * j < head_dim / 2, with s = r mod seq_len:
 *   out[r][h][j]            = x0 * c - x1 * sn
 *   out[r][h][j + half]     = x0 * sn + x1 * c
 * where x0 = x[r][h][j], x1 = x[r][h][j + half], c = cos[s][j], sn = sin[s][j]
 * (sn = -sin[s][j] when transpose != 0).
 */
int orc_rope(const void *x, int64_t x_row_stride, int64_t x_head_stride, const void *cos_t, const void *sin_t,
             int64_t table_stride, int x_dt, int t_dt, int64_t batch, int64_t seq_len, int64_t heads,
             int64_t head_dim, int transpose, double *out) {
    if (!orc_valid_code(x_dt) || !orc_valid_code(t_dt) || batch < 0 || seq_len < 1 || heads < 1 ||
        head_dim < 2 || head_dim % 2 != 0)
        return -1;
    const int64_t half = head_dim / 2;
    if (table_stride < half || x_head_stride < head_dim || x_row_stride < heads * x_head_stride) return -1;
    const int64_t rows = batch * seq_len;
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t srow = r % seq_len;
        for (int64_t h = 0; h < heads; ++h) {
            const int64_t base = r * x_row_stride + h * x_head_stride;
            double *o = out + (r * heads + h) * head_dim;
            for (int64_t j = 0; j < half; ++j) {
                double x0 = load_elem(x, x_dt, base + j);
                double x1 = load_elem(x, x_dt, base + j + half);
                double c = load_elem(cos_t, t_dt, srow * table_stride + j);
                double sn = load_elem(sin_t, t_dt, srow * table_stride + j);
                if (transpose) sn = -sn;
                o[j] = x0 * c - x1 * sn;
                o[j + half] = x0 * sn + x1 * c;
            }
        }
    }
    return 0;
}

/* ---- residual + LayerNorm --------------------------------------------------
 * res may be NULL (plain LayerNorm: h = x); w and b may each be NULL (1 and
 * 0).  Outputs: y (M, H) and, when non-NULL, h (M, H) (the exact sum, before
 * any rounding to a storage format), mean (M,) and rstd (M,).
 */
int orc_layernorm(const void *x, int64_t x_stride, const void *res, int64_t r_stride, const void *w, const void *b,
                  int x_dt, int w_dt, int64_t M, int64_t H, double eps, double *y, double *h_out, double *mean_out,
                  double *rstd_out) {
    if (!orc_valid_code(x_dt) || !orc_valid_code(w_dt) || M < 0 || H < 1 || x_stride < H ||
        (res && r_stride < H) || !(eps >= 0.0))
        return -1;
    double *h = (double *)malloc(sizeof(double) * (size_t)H);
    if (!h) return -2;
    for (int64_t i = 0; i < M; ++i) {
        double sum = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dt, i * x_stride + j);
            if (res) v += load_elem(res, x_dt, i * r_stride + j);
            h[j] = v;
            sum += v;
        }
        const double mean = sum / (double)H;
        double sq = 0.0;
        for (int64_t j = 0; j < H; ++j) sq += (h[j] - mean) * (h[j] - mean);
        const double var = sq / (double)H;
        const double rstd = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < H; ++j) {
            double wj = w ? load_elem(w, w_dt, j) : 1.0;
            double bj = b ? load_elem(b, w_dt, j) : 0.0;
            y[i * H + j] = (h[j] - mean) * rstd * wj + bj;
            if (h_out) h_out[i * H + j] = h[j];
        }
        if (mean_out) mean_out[i] = mean;
        if (rstd_out) rstd_out[i] = rstd;
    }
    free(h);
    return 0;
}
