// rmsnorm_api.hip -- host side of the gfx950 RMSNorm library: argument
// validation, launch geometry and the extern "C" entry points declared in
// include/rmsnorm.h and include/layernorm.h (shared helpers: host_common.hpp).
//
// Nothing here allocates, frees or synchronises.  Argument errors are found
// before the first HIP call.  The only HIP calls are hipGetDevice,
// hipDeviceGetAttribute / hipGetDeviceProperties (once per device, cached)
// and hipLaunchKernel.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "host_common.hpp"
#include "kernel_tables.hpp"
#include "layernorm.h"
#include "rmsnorm.h"
#include "rmsnorm_tuning.h"

namespace {

using namespace rmsn;
using namespace rmsn::host;

// ---------------------------------------------------------------------------
// argument checks of the norm entry points
// ---------------------------------------------------------------------------

constexpr int64_t kMaxH = int64_t(1) << 30;

rmsn_status_t check_common(int64_t M, int64_t H, rmsn_dtype_t xdt, const void *w, rmsn_dtype_t wdt) {
    if (!dtype_valid(xdt)) return fail(RMSN_ERR_UNSUPPORTED, "x_dtype %d is not RMSN_F32/F16/BF16", (int)xdt);
    if (w != nullptr && !(wdt == xdt || wdt == RMSN_F32))
        return fail(RMSN_ERR_UNSUPPORTED, "w_dtype %d must equal x_dtype %d or be RMSN_F32", (int)wdt, (int)xdt);
    if (M < 0) return fail(RMSN_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (H < 1) return fail(RMSN_ERR_INVALID_ARG, "H = %lld must be >= 1", (long long)H);
    if (H > kMaxH) return fail(RMSN_ERR_UNSUPPORTED, "H = %lld exceeds 2^30", (long long)H);
    return RMSN_OK;
}

rmsn_status_t check_eps(float eps) {
    if (!(eps > 0.0f) || !std::isfinite(eps))
        return fail(RMSN_ERR_INVALID_ARG, "eps = %g must be positive and finite", (double)eps);
    return RMSN_OK;
}

// ---------------------------------------------------------------------------
// geometry
// ---------------------------------------------------------------------------


// vectors per thread available as kernel instantiations
enum class Kind { Fwd, FwdResid, FwdAdaln, Ln, Bwd, BwdRes };
constexpr int kFwdVecVpt[] = {1, 2, 3, 4, 6, 8};
constexpr int kBwdVecVpt[] = {1, 2, 3, 4};
constexpr int kScalarVpt[] = {1, 2, 4, 8};
// largest workgroup each register tile may use (the kernels' launch bounds);
// pb: bytes per element of the forward family's parameters (weight, AdaLN's
// rows, LayerNorm's bias; x's format when there are none)
int max_threads_for(Kind kind, int vpt, int vec, int pb = 4) {
    const int es2 = vec == 8 && pb == 2 ? 2 : 4;  // x and its parameters all 16-bit
    return kind == Kind::Bwd        ? bwd_max_threads(vpt * vec)
           : kind == Kind::BwdRes   ? bwd_max_threads(vpt * vec, true, vec == 8 ? 2 : 4)
           : kind == Kind::FwdResid ? fwd_max_threads(vpt * vec, MODE_RESID, es2)
           : kind == Kind::FwdAdaln ? fwd_max_threads(vpt * vec, MODE_ADALN, es2)
           : kind == Kind::Ln       ? ln_max_threads(vpt * vec, es2)
                                    : fwd_max_threads(vpt * vec, MODE_PLAIN, es2);
}

struct Geom {
    int vec;      // elements per access (16 bytes / element, or 1)
    int vpt;      // accesses per thread per chunk
    int wpr;      // waves per row group
    int rpw;      // row groups per workgroup
    int nvec;     // accesses per row
    int nchunks;  // 1 = resident
    bool two_pass;
};

// Pick (vpt, wpr) so that 64*wpr*vpt covers nvec with the least idle slots,
// preferring `pref` elements per thread; rows longer than the largest tile
// use two passes.
Geom pick_row_geom(Kind kind, int H, int vec, int pref_elems, int pb = 4) {
    Geom g{};
    g.vec = vec;
    g.nvec = (H + vec - 1) / vec;
    const bool bwd = kind == Kind::Bwd || kind == Kind::BwdRes;
    const int *set = vec == 1 ? kScalarVpt : bwd ? kBwdVecVpt : kFwdVecVpt;
    const int nset = vec == 1 ? 4 : bwd ? 4 : 6;
    // Rows spread over more waves than `wcap` are avoided when a tile with
    // more vectors per thread fits (measured on gfx950, bf16, 64 Mi-element
    // calls: the forward and fused residual at H = 16384 ran 72 % of peak on
    // 16-wave rows and 74.5-75 % on 8-11-wave rows; LayerNorm, with two
    // reductions per row, 64 % on 16- and 8-wave rows and 73 % on 4-wave rows
    // at H = 16384, while at H <= 8192 its tiles were within 1 %).  A
    // penalty, not a limit: with no tile under the cap the row stays
    // resident on the best tile over it.
    // AdaLN tiles count as over the cap beyond 8 waves: 16-bit ones always,
    // float32 ones of more than 16 elements per thread.  Tiles of more than
    // 16 elements per thread take 104-124 VGPRs (four waves per SIMD), and
    // one such workgroup per CU leaves SIMDs idle (bf16, 2048 rows:
    // H = 16384 on 3 x 11 waves 74.5 % against 82.8 % on 4 x 8, H = 12296 on
    // 3 x 9 66.1 % against 76.9 % on 4 x 7).  16-bit rows of 2 vectors per
    // thread on more than 8 waves ran slow too (bf16 8192 rows, per token:
    // H = 10240 on 2 x 10 waves 65.7 % against 79.0 % on 3 x 7, H = 12288 on
    // 2 x 12 67.5 % against 81.0 % on 3 x 8; per batch 51.0 % and 54.5 %
    // against 62.0 % and 68.6 %); float32 rows on 12 waves lost nothing
    // (float32 8192 x 6144 80.7 % against 79.4 % on 3 x 8).
    const int wcap = kind == Kind::Ln ? (g.nvec > 1024 ? 4 : 16) : bwd ? 16 : 12;
    double best = 1e30;
    for (int i = 0; i < nset; ++i) {
        const int vpt = set[i];
        const int maxw = max_threads_for(kind, vpt, vec, pb) / 64;
        const int wpr = (g.nvec + 64 * vpt - 1) / (64 * vpt);
        if (wpr > maxw) continue;
        const double slots = 64.0 * wpr * vpt;
        const double idle = (slots - g.nvec) / slots;
        const double pref = std::fabs(std::log2((double)(vpt * vec) / pref_elems));
        const int cap = kind == Kind::FwdAdaln && (vpt * vec > 16 || vec == 8) ? 8 : wcap;
        const double cost = 8.0 * idle + pref + (wpr > cap ? 4.0 : 0.0);
        if (cost < best) {
            best = cost;
            g.vpt = vpt;
            g.wpr = wpr;
        }
    }
    if (best < 1e30) {
        g.nchunks = 1;
        g.two_pass = false;
    } else {
        g.vpt = vec > 1 ? 4 : 8;
        g.wpr = 16;
        const int chunk = 64 * g.wpr * g.vpt;
        g.nchunks = (g.nvec + chunk - 1) / chunk;
        g.two_pass = true;
    }
    g.rpw = 1;
    while (g.rpw * g.wpr < 4 && 64 * g.wpr * g.rpw * 2 <= max_threads_for(kind, g.vpt, g.vec, pb)) g.rpw *= 2;
    return g;
}

// Tile of the RMSNorm forward (and 16-bit LayerNorm) on rows off the 16-byte
// grid from 1 KiB (16-byte vectors at the row's byte offset).  A lane without
// a vector costs no memory traffic, and the fewer waves a row takes, the more
// rows a CU holds in flight, so the cost is the row's waves plus 8 x the idle
// share of its slots, over vpt <= 6; rows of at most three waves share a
// workgroup in pairs.
// Measured on gfx950 (bf16, 2^25 elements) against the vector tile rule and
// against the LDS staging this replaced: H = 2049 64.8 % (48.2 % on the vector
// rule, 58.5 % staged), H = 4097 63.7 % (61.3 % staged; one row per
// workgroup: 60.1 %), H = 6143 64.5 % (58.7 % staged), fused residual
// H = 6143 68.7 % (58.4 % staged).
Geom pick_offgrid_geom(Kind kind, int H, int vec, int pb) {
    static const int kOffgridVpt[] = {1, 2, 3, 4, 6};
    Geom g{};
    g.vec = vec;
    g.nvec = (H + vec - 1) / vec;
    double best = 1e30;
    for (int vpt : kOffgridVpt) {
        const int wpr = (g.nvec + 64 * vpt - 1) / (64 * vpt);
        if (wpr > max_threads_for(kind, vpt, vec, pb) / 64) continue;
        const double slots = 64.0 * wpr * vpt;
        const double cost = wpr + 8.0 * (slots - g.nvec) / slots;
        if (cost < best) {
            best = cost;
            g.vpt = vpt;
            g.wpr = wpr;
        }
    }
    g.two_pass = best >= 1e30;
    g.nchunks = 1;
    g.rpw = g.wpr <= 3 && 64 * g.wpr * 2 <= max_threads_for(kind, g.vpt, vec, pb) ? 2 : 1;
    return g;
}

// 16-bit rows off the grid of 193 to 768 vectors, every forward kind: two
// waves per row, with the fewest idle vector slots over vpt in {1, 2, 3, 4, 6};
// vpt = 0 for other rows.  Measured on gfx950 (bf16, HIP events, previous rule
// in brackets):
//   AdaLN, 2 x 4096 rows, against the aligned rule: per-batch conditioning
//   H = 2049 45.1 % (37.3 %), 3073 50.1 % (44.9 %), 4097 48.5 % (41.2 %),
//   6143 54.0 % (46.4 %); per-token H = 2049 66.8 % (53.1 %), 4097 71.2 %
//   (63.1 %), 6143 73.8 % (60.7 %); 1537 and 7169 within 0.3 %.  The plain
//   forward's off-grid rule, which takes fewer waves per row, lost to the
//   aligned rule there at H = 1537, 7169 and 8191 with per-batch
//   conditioning (-3 to -4 points).
//   Plain forward and fused residual, 2^25 elements, against the off-grid
//   rule: H = 1537 61.7 % (59.3 %), 2049 66.4 % (63.4 %), 4097 63.6 %
//   (62.2 %), fused residual 2049 67.1 % (65.5 %); LayerNorm 2049 58.4 %
//   (53.6 %), 4097 54.6 % (53.9 %); 3073, 5121 and 6143 the same tile.
//   float32 rows lost 0.5 points at H = 2049 and keep their rules.  Rows of
//   up to 192 vectors keep them too: at H = 1023 and 1025 the plain forward
//   lost 3.6 and 4.4 points and LayerNorm 7.9 to one-wave rows (the fused
//   residual, AdaLN and residual LayerNorm gained 1.6 to 2.7).
Geom pick_two_wave_geom(Kind kind, int H, int vec, int pb) {
    static const int kVpt[] = {1, 2, 3, 4, 6};
    Geom g{};
    g.vec = vec;
    g.nvec = (H + vec - 1) / vec;
    if (g.nvec <= 192) return g;
    int best = 0;
    for (int vpt : kVpt) {
        if (128 * vpt < g.nvec || max_threads_for(kind, vpt, vec, pb) < 128) continue;
        if (best == 0) best = vpt;  // the smallest vpt that holds the row idles the fewest slots
    }
    if (best == 0) return g;
    g.vpt = best;
    g.wpr = 2;
    g.nchunks = 1;
    g.two_pass = false;
    g.rpw = 64 * 2 * 2 <= max_threads_for(kind, best, vec, pb) ? 2 : 1;
    return g;
}

// The forward family's tile with no forced geometry (vec_ok, mis_ok as for
// bwd_tile; mis_ok also needs the bias and AdaLN's conditioning rows
// aligned).  Rows off the 16-byte grid take 16-byte vectors at each row's
// byte offset when the row holds at least 512 bytes.  16-bit rows of 193 to
// 768 vectors, every forward kind, take two waves per row; other RMSNorm and
// 16-bit LayerNorm rows from 1 KiB take the off-grid tile rule; shorter rows,
// other AdaLN rows and float32 LayerNorm the aligned rule; rows longer than
// any resident tile passes over the row.
// Measured on gfx950 against the element-wise tile (bf16, 2^25 elements):
// H = 257 49.5 % against 37.4 % of peak, H = 511 68.9 % and 56.3 %, but
// H = 127 27.8 % and 31.3 % (16 vectors leave most of a wave idle);
// LayerNorm against the LDS staging it replaced: float32 fused residual
// H = 1023 70.5 % against 63.7 %, bf16 H = 4097 55.5 % and 51.9 %.
// LayerNorm on the off-grid rule against the aligned one (2^25 elements or
// more): bf16 H = 2049 57.3 % against 40.5 %, H = 6143 62.0 % against
// 53.0 % (fused residual 64.8 % against 58.5 %), H = 4097 and 1025 within
// 0.1 %; float32 H = 4097 the same, fused residual H = 1025 66.1 % against
// 68.3 %, so float32 keeps the aligned rule.  Otherwise the element-wise
// tile.
Geom fwd_tile(Kind kind, int H, int eb, int pb, bool vec_ok, bool mis_ok, bool *mis, bool ln_resid = false) {
    const int vecw = 16 / eb;
    const bool offrule = kind == Kind::Fwd || kind == Kind::FwdResid || (kind == Kind::Ln && eb == 2);
    *mis = false;
    if (!vec_ok && mis_ok && (int64_t)H * eb >= 512) {
        Geom m{};
        if (eb == 2 && (offrule || kind == Kind::FwdAdaln) && (int64_t)H * eb >= 1024)
            m = pick_two_wave_geom(kind, H, vecw, pb);
        if (m.vpt == 0 && offrule && (int64_t)H * eb >= 1024) m = pick_offgrid_geom(kind, H, vecw, pb);
        if (m.vpt == 0 || m.two_pass) m = pick_row_geom(kind, H, vecw, eb == 4 ? 8 : 16, pb);
        *mis = true;
        return m;
    }
    Geom g = pick_row_geom(kind, H, vec_ok ? vecw : 1, eb == 4 ? 8 : 16, pb);
    // 16-bit rows on the grid of 193 to 768 vectors: two waves per row too,
    // for LayerNorm and AdaLN always, for the plain forward unless the rule's
    // tile is a whole tile of 2 or more vectors per thread; the fused
    // residual keeps the rule's tile.
    if (vec_ok && eb == 2 && kind != Kind::FwdResid && !g.two_pass) {
        const Geom t = pick_two_wave_geom(kind, H, vecw, pb);
        const bool whole = g.vpt >= 2 && 64 * g.wpr * g.vpt == g.nvec;
        if (t.vpt != 0 && (kind != Kind::Fwd || !whole)) g = t;
    }
    // 16-bit LayerNorm rows on the grid of 769 to 1024 vectors: two waves of
    // 8 vectors per thread, two rows per workgroup.  Measured on gfx950,
    // bf16 8192 x 8192: 46.6 us against 47.6 us on 2 x 8 waves walking two
    // rows (50.0 us without the walk), 16384 x 8192 88.1 against 90.4 us,
    // 8192 x 7168 41.2 against 43.8 us; the fused residual LayerNorm (90.1
    // against 88.7 us), the plain forward and AdaLN lost on that tile (45.5
    // against 44.8 us, 86.8 against 85.0 us).
    if (vec_ok && eb == 2 && kind == Kind::Ln && !ln_resid && !g.two_pass && g.nvec > 768 && g.nvec <= 1024 &&
        max_threads_for(kind, 8, vecw, pb) >= 256) {
        g.vpt = 8;
        g.wpr = 2;
        g.rpw = 2;
        g.nchunks = 1;
    }
    return g;
}

// ---------------------------------------------------------------------------
// kernel tables
// ---------------------------------------------------------------------------



// ---------------------------------------------------------------------------
// forward (plain and fused residual)
// ---------------------------------------------------------------------------

// Conditioning rows of an AdaLN call (scale and shift share the layout).
struct Cond {
    const void *scale = nullptr;
    const void *shift = nullptr;
    int64_t cs = 0;             // row stride, elements
    int64_t rows_per_cond = 1;  // x rows per conditioning row
};

// LayerNorm calls (modes kLn, kLnResid): the bias and the per-row mean
// output; the rrms argument of fwd_impl then receives rstd.
struct LnExtra {
    const void *bias = nullptr;
    float *mean = nullptr;
};
constexpr int kLn = 3, kLnResid = 4;  // host-side modes beside MODE_PLAIN/RESID/ADALN

// mode: MODE_PLAIN, MODE_RESID, MODE_ADALN, kLn or kLnResid.  For AdaLN, wdt
// is the format of the weight, scale and shift; for LayerNorm, of the weight
// and bias.
rmsn_status_t fwd_impl(int mode, const void *x, int64_t xs, const void *r, int64_t rs, const void *w, void *y,
                       int64_t ys, void *ro, int64_t ros, float *rrms, int64_t M, int64_t H, float eps,
                       rmsn_dtype_t xdt, rmsn_dtype_t wdt, const Cond &cond, const LnExtra &lnx,
                       hipStream_t stream) {
    const bool ln = mode == kLn || mode == kLnResid;
    const bool resid = mode == MODE_RESID || mode == kLnResid, adaln = mode == MODE_ADALN;
    const void *bias = ln ? lnx.bias : nullptr;
    float *mean = ln ? lnx.mean : nullptr;
    rmsn_status_t st = check_common(M, H, xdt, (w || adaln || bias) ? (const void *)1 : nullptr, wdt);
    if (st != RMSN_OK) return st;
    if ((st = check_eps(eps)) != RMSN_OK) return st;
    const int eb = dtype_bytes(xdt);
    if ((st = check_stride("x_stride", xs, M, H, eb)) != RMSN_OK) return st;
    if ((st = check_stride("y_stride", ys, M, H, eb)) != RMSN_OK) return st;
    if (resid) {
        if ((st = check_stride("r_stride", rs, M, H, eb)) != RMSN_OK) return st;
        if (ro != nullptr && (st = check_stride("ro_stride", ros, M, H, eb)) != RMSN_OK) return st;
    }
    int64_t crows = 0;
    const int pb = dtype_bytes(wdt);
    if (adaln) {
        if (cond.rows_per_cond < 1)
            return fail(RMSN_ERR_INVALID_ARG, "rows_per_cond = %lld must be >= 1", (long long)cond.rows_per_cond);
        crows = M / cond.rows_per_cond + (M % cond.rows_per_cond != 0);  // ceil, without overflow
        if ((st = check_stride("cond_stride", cond.cs, crows, H, pb)) != RMSN_OK) return st;
    }
    if (M == 0) return RMSN_OK;
    if (x == nullptr) return fail(RMSN_ERR_INVALID_ARG, "x is NULL");
    if (y == nullptr) return fail(RMSN_ERR_INVALID_ARG, "y is NULL");
    if (resid && r == nullptr) return fail(RMSN_ERR_INVALID_ARG, "residual is NULL");
    if (adaln && (cond.scale == nullptr || cond.shift == nullptr))
        return fail(RMSN_ERR_INVALID_ARG, "scale and shift must not be NULL");

    const int wb = w ? dtype_bytes(wdt) : 1;
    Region ins[6] = {mat("x", x, xs, M, H, eb), mat("residual", resid ? r : nullptr, rs, M, H, eb),
                     vec("w", w, H, wb), mat("scale", adaln ? cond.scale : nullptr, cond.cs, crows, H, pb),
                     mat("shift", adaln ? cond.shift : nullptr, cond.cs, crows, H, pb), vec("bias", bias, H, pb)};
    Region outs[4] = {mat("y", y, ys, M, H, eb), mat("residual_out", resid ? ro : nullptr, ros, M, H, eb),
                      vec(ln ? "rstd" : "rrms", rrms, M, 4), vec("mean", mean, M, 4)};
    if ((st = check_overlap(outs, 4, ins, 6)) != RMSN_OK) return st;
    // the per-row statistics are never "the same buffer" as an input: compare
    // ranges only
    for (int i = 2; i < 4; ++i) {
        if (!outs[i].present) continue;
        for (const Region &in : ins)
            if (in.present && outs[i].overlaps(in))
                return fail(RMSN_ERR_INVALID_ARG, "%s overlaps input %s", outs[i].name, in.name);
    }

    // vector path: every row start 16-byte aligned and H a whole number of vectors
    const int vecw = 16 / eb;
    bool vec_ok = (H % vecw) == 0 && aligned16(x) && aligned16(y) && xs % (16 / eb) == 0 && ys % (16 / eb) == 0 &&
                  (w == nullptr || aligned16(w));
    if (resid)
        vec_ok = vec_ok && aligned16(r) && rs % (16 / eb) == 0 &&
                 (ro == nullptr || (aligned16(ro) && ros % (16 / eb) == 0));
    if (adaln)
        vec_ok = vec_ok && aligned16(cond.scale) && aligned16(cond.shift) && cond.cs % (16 / pb) == 0;
    if (bias != nullptr) vec_ok = vec_ok && aligned16(bias);

    const Kind kind = ln ? Kind::Ln : resid ? Kind::FwdResid : adaln ? Kind::FwdAdaln : Kind::Fwd;
    const Override ov = get_override(0);
    // rows off the grid: every row start element-aligned, the weight (and
    // bias) 16-byte aligned; a forced geometry keeps the element-wise tile
    const bool mis_ok = !vec_ok && !ov.set && (w == nullptr || aligned16(w)) &&
                        (bias == nullptr || aligned16(bias)) && aligned_to(x, eb) && aligned_to(y, eb) &&
                        (!resid || (aligned_to(r, eb) && (ro == nullptr || aligned_to(ro, eb)))) &&
                        (!adaln || (aligned_to(cond.scale, pb) && aligned_to(cond.shift, pb)));
    bool mis = false;
    // the parameters' format as the kernels see it (x's when there are none)
    const int kpb = dtype_bytes((w || adaln || bias) ? wdt : xdt);
    Geom g = fwd_tile(kind, (int)H, eb, kpb, vec_ok, mis_ok, &mis, ln && resid);
    int64_t grid = (M + g.rpw - 1) / g.rpw;
    if (ov.set) {
        // bounds first: the products below are then small
        if (ov.a < 1 || ov.a > 64 || ov.b < 1 || ov.b > 16 || ov.c < 0 || ov.c > 16)
            return fail(RMSN_ERR_INVALID_ARG, "forced forward geometry: tile vpt %d wpr %d rpw %d out of range",
                        ov.a, ov.b, ov.c);
        Geom o = g;
        o.vpt = ov.a;
        o.wpr = ov.b;
        o.rpw = ov.c > 0 ? ov.c : 1;
        const int maxt = max_threads_for(kind, o.vpt, o.vec, kpb);
        if (o.vpt < 1 || o.wpr < 1 || o.wpr * o.rpw * 64 > maxt || o.wpr * o.rpw > 16)
            return fail(RMSN_ERR_INVALID_ARG,
                        "forced forward geometry: bad tile vpt %d wpr %d rpw %d (max %d threads)", o.vpt, o.wpr,
                        o.rpw, maxt);
        const int chunk = 64 * o.wpr * o.vpt;
        o.nchunks = (o.nvec + chunk - 1) / chunk;
        o.two_pass = o.nchunks > 1;
        if (o.two_pass && o.vpt != (o.vec > 1 ? 4 : 8))
            return fail(RMSN_ERR_INVALID_ARG, "forced forward geometry: two-pass tiles need vpt %d",
                        o.vec > 1 ? 4 : 8);
        g = o;
        grid = (M + g.rpw - 1) / g.rpw;
        if (ov.d > 0 && ov.d < grid) grid = ov.d;
    }
    const int64_t groups = (M + g.rpw - 1) / g.rpw;
    if (grid > INT32_MAX) grid = INT32_MAX;
    int64_t iters = (groups + grid - 1) / grid;

    const int64_t streamed = (resid ? (ro ? 4 : 3) : 2) * M * H * eb;
    const bool nt = use_streaming(streamed);
    const rmsn_dtype_t kwdt = (w || adaln || bias) ? wdt : xdt;
    int cus = 0;  // the device must be a readable gfx950 before anything is enqueued
    if (ln) {
        ln_fn fn = mis ? ln_mis_lookup(xdt, kwdt, g.vpt, g.two_pass, nt, resid)
                       : ln_lookup(xdt, kwdt, g.vec, g.vpt, g.two_pass, nt, resid);
        if (fn == nullptr) return fail(RMSN_ERR_INVALID_ARG, "no kernel for vec %d vpt %d", g.vec, g.vpt);
        if ((st = device_info(&cus)) != RMSN_OK) return st;
        // LayerNorm (no residual) whose weight and bias take 16 KiB or more
        // between them: each row group walks 2 rows, so that the parameters
        // it holds in registers serve both.  Every row's workgroup otherwise
        // fetches them from L2 again (they miss the CU's L1).  Measured on
        // gfx950, the same tiles and bits (one row per row group in
        // brackets): bf16 8192 x 4096 64.5 % (62.5 %), 8192 x 6144 66.2 %
        // (60.2 %), 8192 x 8192 70.0 % (66.0 %), 16384 x 4096 72.0 % (68.1 %),
        // off the grid 8192 x 4097 55.3 % (53.6 %); float32 8192 x 4096
        // 71.4 % (65.5 %), 16384 x 2048 72.6 % (69.3 %).  Only from 32 row
        // groups per CU: with half the workgroups, smaller calls pay a
        // partial last round of resident workgroups (bf16 4096 x 4096 53.6 %
        // against 56.6 %).  The residual form, with twice the row streams,
        // and RMSNorm's one weight row lost or gained nothing.  Rows of one or
        // two waves do not walk: on the two-wave tiles the walk measured level
        // or slower (bf16 8192 x 4096 24.5-24.7 us either way, 8192 x 6144
        // 40.7 us walking against 38.7 us).
        if (!resid && w != nullptr && bias != nullptr && !ov.set && !g.two_pass && g.wpr > 2 &&
            2 * H * kpb >= 16384 && groups >= 32LL * cus) {
            grid = (groups + 1) / 2;
            iters = (groups + grid - 1) / grid;
        }
        LnParams p;
        p.x = x;
        p.r = r;
        p.w = w;
        p.b = bias;
        p.y = y;
        p.ro = ro;
        p.mean = mean;
        p.rstd = rrms;
        p.xs = xs;
        p.rs = rs;
        p.ys = ys;
        p.ros = ros;
        p.M = M;
        p.iters = iters;
        p.H = (int)H;
        p.nvec = g.nvec;
        p.wpr = g.wpr;
        p.rpw = g.rpw;
        p.nchunks = g.nchunks;
        p.eps = eps;
        p.inv_h = (float)(1.0 / (double)H);
        void *args[] = {&p};
        return launch((const void *)fn, dim3((unsigned)grid), dim3(64 * g.wpr * g.rpw), args, stream,
                      resid ? "layernorm_fwd_residual" : "layernorm_fwd");
    }
    fwd_fn fn = mis     ? fwd_mis_lookup(xdt, kwdt, g.vpt, g.two_pass, mode, nt)
                : resid ? fwd_lookup_resid(xdt, kwdt, g.vec, g.vpt, g.two_pass, nt)
                : adaln ? fwd_lookup_adaln(xdt, kwdt, g.vec, g.vpt, g.two_pass, nt)
                        : fwd_lookup_plain(xdt, kwdt, g.vec, g.vpt, g.two_pass, nt);
    if (fn == nullptr) return fail(RMSN_ERR_INVALID_ARG, "no kernel for vec %d vpt %d", g.vec, g.vpt);
    if ((st = device_info(&cus)) != RMSN_OK) return st;
    // AdaLN with conditioning rows shared by many rows (per-batch scale and
    // shift): each row group walks 4 (or 8) rows, so that the weight and the
    // conditioning rows it holds in registers serve all of them.  Measured on
    // gfx950, bf16 2 x 4096 x 2048 with one conditioning row per batch:
    // 14.30 us against 15.25 us with one row per row group (same tile, same
    // bits); per-token conditioning gained nothing.  Only where the grid of
    // one row per row group has at least 16 workgroups per CU.  16-bit rows
    // walk only when the
    // call has at most two conditioning rows: with more, a row group's rows
    // (a quarter of the call apart) mostly fall in different batches and
    // reload theirs, and the smaller grid lost (bf16, one row per row group
    // first: 4 x 4096 x 2048 26.5 against 27.5 us, 16 x 1024 x 2048 25.8
    // against 27.4 us, 3 x 4096 x 2048 22.3 against 22.7 us, 8 x 1024 x 2048
    // level).  float32 rows, with twice the weight bytes, still gained from
    // the walk at three batches (3 x 4096 x 2048 38.4 against 40.5 us).
    // Rows of 8 KiB or more walk 8 rows when the call has at most two
    // conditioning rows (walk of 4 first): bf16 2 x 4096 x 8192 51.7 against
    // 48.7 us, 2 x 4096 x 6144 37.3 against 36.8 us, float32 2 x 4096 x 2048
    // 26.1 against 24.9 us, 2 x 4096 x 4096 47.8 against 46.8 us; 4 KiB rows
    // lost on 8 (bf16 2 x 4096 x 2048 14.3 against 16.3 us, float32
    // 2 x 4096 x 1024 14.0 against 14.8 us).
    int64_t run_iters = iters;
    const bool few_cond = M <= 2 * cond.rows_per_cond;
    const bool walk_rows = eb == 4 || few_cond;
    const int64_t walk = H * eb >= 8192 && few_cond ? 8 : 4;
    if (adaln && !ov.set && !g.two_pass && cond.rows_per_cond >= 4 && walk_rows && groups >= 16LL * cus) {
        grid = (groups + walk - 1) / walk;
        if (grid > INT32_MAX) grid = INT32_MAX;
        run_iters = (groups + grid - 1) / grid;
    }

    FwdParams p;
    p.x = x;
    p.r = r;
    p.w = w;
    p.y = y;
    p.ro = ro;
    p.rrms = rrms;
    p.xs = xs;
    p.rs = rs;
    p.ys = ys;
    p.ros = ros;
    p.M = M;
    p.iters = run_iters;
    p.H = (int)H;
    p.nvec = g.nvec;
    p.wpr = g.wpr;
    p.rpw = g.rpw;
    p.nchunks = g.nchunks;
    p.eps = eps;
    p.inv_h = (float)(1.0 / (double)H);
    p.scale = cond.scale;
    p.shift = cond.shift;
    p.cs = cond.cs;
    p.rows_per_cond = cond.rows_per_cond;
    void *args[] = {&p};
    return launch((const void *)fn, dim3((unsigned)grid), dim3(64 * g.wpr * g.rpw), args, stream,
                  resid ? "rmsnorm_fwd_residual" : adaln ? "rmsnorm_adaln_fwd" : "rmsnorm_fwd");
}

// Most dw partial rows a backward call may use: 1024, or more for short rows
// (up to 8 MiB of partial sums, at most 8192 rows).  Depends on H only, so
// the workspace size is known without a device.
int64_t max_partials(int64_t H) {
    int64_t p = (int64_t(8) << 20) / (4 * H);
    if (p < 1024) p = 1024;
    if (p > 8192) p = 8192;
    return p;
}

// Row groups (workgroups) of the backward resident per CU.  Measured on
// gfx950 over H = 256 .. 8192 and M = 4096 .. 131072 (bf16): the plain
// backward is fastest with about 8 waves per CU when a row spans several
// waves, and about 4 when a row is one wave (its reduction has no barrier)
// -- more when that wave is partly idle; the residual form, whose rows carry
// a third stream, with about 4.  More groups than that slow both kernels:
// each adds a partial row for the finalize to sum and shortens the rows a
// group streams between its prologue and its partial store.
int bwd_groups_per_cu(bool res, int wpr, int nvec) {
    if (res) return wpr >= 4 ? 1 : 4 / wpr;
    if (wpr >= 2) return wpr >= 8 ? 1 : 8 / wpr;
    const int active = nvec < 64 ? nvec : 64;  // busy lanes of the row's wave
    return 4 * 64 / active;
}

// The backward on rows off the 16-byte grid (single elements), H >= 512:
// 4 elements per thread when the row fits 16 waves, else 8, and more
// workgroups than the vector tile takes -- ceil(16 / wpr) per CU at 4
// elements per thread, one at 8.  Measured on gfx950 over H = 513 ... 8191
// (bf16, 2^25-element calls, plain and residual): plain H = 1025 ran
// 39.6 % of peak against 24.5 % on the vector tile's rule, H = 2050
// 44.6 % against 32.3 %, H = 513 35.2 % against 16.3 %; residual 43-49 %
// against 28-37 %; at H >= 4097 both rules take 8 x wpr on one workgroup per
// CU.  two_pass is set when no tile holds the row.
Geom pick_bwd_elem_geom(Kind kind, int H, int *groups_per_cu) {
    Geom g{};
    g.vec = 1;
    g.nvec = H;
    g.rpw = 1;
    g.nchunks = 1;
    g.two_pass = false;
    for (int vpt : {4, 8}) {
        const int wpr = (H + 64 * vpt - 1) / (64 * vpt);
        if (wpr <= max_threads_for(kind, vpt, 1) / 64 && wpr <= 16) {
            g.vpt = vpt;
            g.wpr = wpr;
            *groups_per_cu = vpt == 4 ? (16 + wpr - 1) / wpr : 1;
            return g;
        }
    }
    g.two_pass = true;
    return g;
}

// The backward's tile with no forced geometry.  vec_ok: every row start is
// 16-byte aligned and H a whole number of vectors.  mis_ok: otherwise, every
// row start element-aligned and w 16-byte aligned.  Rows off the grid take
// 16-byte vectors at their byte offset when mis_ok and the row holds at least
// 16 bytes, in one pass or, for rows longer than a tile, two; otherwise rows
// from 512 elements take the single-element rule (*elem_groups = its
// workgroups per CU), shorter ones the vector rule's single-element tile.
Geom bwd_tile(Kind kind, int H, int eb, bool vec_ok, bool mis_ok, bool *mis, int *elem_groups) {
    const int vecw = 16 / eb;
    Geom g = pick_row_geom(kind, H, vec_ok ? vecw : 1, 8);
    *mis = false;
    *elem_groups = 0;
    if (!vec_ok && mis_ok && (int64_t)H * eb >= 16) {
        g = pick_row_geom(kind, H, vecw, 8);
        *mis = true;
    }
    if (!vec_ok && !*mis && H >= 512) {
        const Geom e = pick_bwd_elem_geom(kind, H, elem_groups);
        if (e.two_pass)
            *elem_groups = 0;
        else
            g = e;
    }
    return g;
}

// The tile of a backward on rows off the grid whose vectors sit on memory's
// 16-byte grid (`frame`): a row of H elements at offset a within its first
// chunk spans up to ceil((H * eb + 16 - eb) / 16) chunks, one more vector than
// at the row's offset when H * eb mod 16 is 0 or above eb.  The vector tile
// rule for that many vectors; false when it takes two passes (the frame is
// for one pass only) or single elements.
bool bwd_frame_tile(Kind kind, int H, int eb, Geom *out) {
    bool mis = false;
    int elem_groups = 0;
    const Geom g = bwd_tile(kind, H + (16 - eb) / eb, eb, false, true, &mis, &elem_groups);
    if (!mis || g.two_pass) return false;
    *out = g;
    return true;
}

size_t bwd_workspace(int64_t M, int64_t H) {
    if (M <= 0 || H <= 0 || H > kMaxH) return 0;
    const int64_t cap = max_partials(H);
    const int64_t P = M < cap ? M : cap;
    return (size_t)P * (size_t)H * sizeof(float);
}

// ---------------------------------------------------------------------------
// static scratch of rmsnorm_bwd_noalloc
// ---------------------------------------------------------------------------

// The dw partial rows of rmsnorm_bwd_noalloc live here instead of a caller's
// workspace: every device the library runs on holds one copy until the
// process ends.  Each call writes every partial row it reads before reading
// it, so nothing has to start at zero; calls that overlap on one device
// share the array and race.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    hipError_t err = hipErrorUnknown;
    void *ptr = nullptr;
};
constexpr int kScratchDevices = 64;  // device indices with a slot
ScratchSlot g_scratch[kScratchDevices];

// Device address of this device's copy of `scratch`, looked up once per
// device with that device current.  In host code the array's name is only a
// host-side stand-in; kernels receive this address.
rmsn_status_t scratch_partials(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RMSN_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchDevices) return fail(RMSN_ERR_HIP, "device index %d out of range", dev);
    ScratchSlot &s = g_scratch[dev];
    std::call_once(s.once, [&s]() {
        void *p = nullptr;
        s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (s.err == hipSuccess && p == nullptr) s.err = hipErrorInvalidSymbol;
        if (s.err == hipSuccess) s.ptr = p;
    });
    if (s.err != hipSuccess)
        return fail(RMSN_ERR_HIP, "looking up the scratch array on device %d failed: %s", dev,
                    hipGetErrorString(s.err));
    *out = s.ptr;
    return RMSN_OK;
}

// dres == nullptr: the plain backward; otherwise the backward of the fused
// residual pre-norm, which adds dres (rows drs apart) to dx.
// use_scratch: the dw partial rows go to this library's static device array
// (scratch_partials) instead of the caller's workspace, which is then ignored.
rmsn_status_t bwd_impl(const void *dy, int64_t dys, const void *x, int64_t xs, const void *dres, int64_t drs,
                       const void *w, const float *rrms, void *dx, int64_t dxs, float *dw, void *ws, size_t ws_bytes,
                       int64_t M, int64_t H, rmsn_dtype_t xdt, rmsn_dtype_t wdt, hipStream_t stream,
                       bool use_scratch = false) {
    rmsn_status_t st = check_common(M, H, xdt, w, wdt);
    if (st != RMSN_OK) return st;
    const int eb = dtype_bytes(xdt);
    const bool res = dres != nullptr;
    if ((st = check_stride("dy_stride", dys, M, H, eb)) != RMSN_OK) return st;
    if ((st = check_stride("x_stride", xs, M, H, eb)) != RMSN_OK) return st;
    if ((st = check_stride("dx_stride", dxs, M, H, eb)) != RMSN_OK) return st;
    if (res && (st = check_stride("dres_stride", drs, M, H, eb)) != RMSN_OK) return st;
    if (dw != nullptr && w == nullptr)
        return fail(RMSN_ERR_INVALID_ARG, "dw requested for a weightless norm (w is NULL)");
    if (M > 0) {
        if (dy == nullptr) return fail(RMSN_ERR_INVALID_ARG, "dy is NULL");
        if (x == nullptr) return fail(RMSN_ERR_INVALID_ARG, "x is NULL");
        if (rrms == nullptr) return fail(RMSN_ERR_INVALID_ARG, "rrms is NULL");
        if (dx == nullptr) return fail(RMSN_ERR_INVALID_ARG, "dx is NULL");
    }
    if (use_scratch) ws = nullptr;
    const size_t need = bwd_workspace(M, H);
    if (dw != nullptr && M > 0 && !use_scratch) {
        if (ws == nullptr || ws_bytes < need)
            return fail(RMSN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : (size_t)0,
                        need);
        if (!aligned16(ws)) return fail(RMSN_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    }
    const int wb = w ? dtype_bytes(wdt) : 1;
    if (M > 0) {
        Region ins[5] = {mat("dy", dy, dys, M, H, eb), mat("x", x, xs, M, H, eb), vec("w", w, H, wb),
                         vec("rrms", rrms, M, 4), mat("dres", dres, drs, M, H, eb)};
        Region outs[3] = {mat("dx", dx, dxs, M, H, eb), vec("dw", dw, H, 4),
                          vec("workspace", dw ? ws : nullptr, (int64_t)need, 1)};
        if ((st = check_overlap(outs, 3, ins, 5)) != RMSN_OK) return st;
        for (int i = 1; i < 3; ++i)
            for (const Region &in : ins)
                if (outs[i].present && in.present && outs[i].overlaps(in))
                    return fail(RMSN_ERR_INVALID_ARG, "%s overlaps input %s", outs[i].name, in.name);
        // dx may be the same buffer as dy, x or dres, but never w or rrms
        if (outs[0].overlaps(ins[2]) && ins[2].present) return fail(RMSN_ERR_INVALID_ARG, "dx overlaps w");
        if (outs[0].overlaps(ins[3])) return fail(RMSN_ERR_INVALID_ARG, "dx overlaps rrms");
    } else if (dw == nullptr) {
        return RMSN_OK;
    }

    if (M == 0) {  // dw of zero rows is zero
        int cus = 0;
        if ((st = device_info(&cus)) != RMSN_OK) return st;
        const float *none = nullptr;
        int P = 0, Hi = (int)H;
        void *args[] = {(void *)&none, &P, &Hi, &dw};
        return launch(dw_finalize_kernel(), dim3((unsigned)((H + kFinCols - 1) / kFinCols)),
                      dim3(kFinCols * kFinSlices), args, stream, "rmsnorm_dw_finalize");
    }

    const int vecw = 16 / eb;
    const bool vec_ok = (H % vecw) == 0 && aligned16(dy) && aligned16(x) && aligned16(dx) &&
                        dys % (16 / eb) == 0 && xs % (16 / eb) == 0 && dxs % (16 / eb) == 0 &&
                        (w == nullptr || aligned16(w)) && (!res || (aligned16(dres) && drs % (16 / eb) == 0));
    const Kind kind = res ? Kind::BwdRes : Kind::Bwd;
    const Override ov = get_override(1);
    const bool mis_ok = !vec_ok && !ov.set && aligned_to(dy, eb) && aligned_to(x, eb) && aligned_to(dx, eb) &&
                        (!res || aligned_to(dres, eb)) && (w == nullptr || aligned16(w));
    int elem_groups = 0;  // workgroups per CU of the single-element rule, 0: the vector tile's rule
    bool mis = false;
    Geom g = bwd_tile(kind, (int)H, eb, vec_ok, mis_ok, &mis, &elem_groups);
    int64_t P = 0;  // 0: chosen from the device below
    // rows interleaved across workgroups: the rows in flight at any moment are
    // neighbours in memory, as in the forward's one-row-per-workgroup grid
    bool interleave = true;
    if (ov.set) {
        if (ov.a < 1 || ov.a > 64 || ov.b < 1 || ov.b > 16)
            return fail(RMSN_ERR_INVALID_ARG, "forced backward geometry: tile vpt %d wpr %d out of range", ov.a, ov.b);
        Geom o = g;
        o.vpt = ov.a;
        o.wpr = ov.b;
        const int maxt = max_threads_for(kind, o.vpt, o.vec);
        if (o.vpt < 1 || o.wpr < 1 || o.wpr * 64 > maxt)
            return fail(RMSN_ERR_INVALID_ARG, "forced backward geometry: bad tile vpt %d wpr %d", o.vpt, o.wpr);
        const int chunk = 64 * o.wpr * o.vpt;
        o.nchunks = (o.nvec + chunk - 1) / chunk;
        o.two_pass = o.nchunks > 1;
        if (o.two_pass && o.vpt != (o.vec > 1 ? 4 : 8))
            return fail(RMSN_ERR_INVALID_ARG, "forced backward geometry: two-pass tiles need vpt %d",
                        o.vec > 1 ? 4 : 8);
        g = o;
        elem_groups = 0;
        if (ov.c > 0) P = ov.c;
        if (ov.d == 1) interleave = true;
        if (ov.d == 2) interleave = false;
    }
    const bool nt = use_streaming((res ? 4 : 3) * M * H * eb);
    // Rows off the grid whose x, dy, dres and dx rows all sit at the same
    // offset within their 16-byte chunks take their vectors on memory's
    // 16-byte grid instead (`frame` in rmsnorm_bwd_kernel), on the tile that
    // covers the one extra vector a row may then take.  Measured on gfx950,
    // bf16 8192 x 4097: 16-byte vectors at the row offset took 48.5 us, the
    // same tile on rows on the grid (H = 4104) 39.6 us.
    bool af = false;
    const Geom g_off = g;  // the row-offset tile
    if (mis && !g.two_pass && interleave) {
        const uintptr_t bx = reinterpret_cast<uintptr_t>(x);
        auto same_offsets = [&](const void *q, int64_t s) {
            return ((reinterpret_cast<uintptr_t>(q) - bx) & 15u) == 0 && (((uint64_t)(s - xs) * eb) & 15u) == 0;
        };
        if (same_offsets(dy, dys) && same_offsets(dx, dxs) && (!res || same_offsets(dres, drs)))
            af = bwd_frame_tile(kind, (int)H, eb, &g);
    }
    int cus = 0;
    if ((st = device_info(&cus)) != RMSN_OK) return st;
    int gpc = 0;
    bool deep = false;
    int64_t rows_per = 0;
    const int64_t P_set = P;
    for (int attempt = 0; attempt < 2; ++attempt) {
        // Whole row groups per CU, rows interleaved (see bwd_groups_per_cu).
        gpc = elem_groups > 0 ? elem_groups : bwd_groups_per_cu(res, g.wpr, g.nvec);
        // A one-vector tile whose rule leaves at most 6 waves per CU keeps three
        // rows in flight per wave instead of two.  Measured on gfx950 (bf16,
        // 2^25-element calls, two rows in brackets): plain aligned H = 512 (4
        // waves) 67.4 % (61.2 %), 3072 (6) 62.5 % (60.0 %), off the grid
        // H = 1025 (6) 52.9 % (48.7 %), 2049 (5) 50.0 % (44.7 %), residual off the
        // grid H = 1025 (3) 44.3 % (39.2 %), 2049 (5) 56.7 % (52.8 %).  With more
        // waves it lost: plain aligned H = 2048 and 1024 (8 waves) -1.1 and -0.6
        // points, 6144 (12) -1.0; and so did the aligned residual H = 512 (4
        // waves, -3.3), which keeps two.  Same bits either way.  16-bit formats
        // only (as measured).
        deep = !ov.set && eb == 2 && !g.two_pass && g.vec > 1 && g.vpt == 1 && (mis || !res) && gpc * g.wpr <= 6;
        // The dw partial sums are P x H x 4 bytes, written and read once.  A
        // grid that is not a multiple of the CU count leaves a tail of CUs
        // with an extra block.
        P = P_set > 0 ? P_set : (int64_t)cus * gpc;
        if (P > max_partials(H)) P = max_partials(H);
        if (P > M) P = M;
        rows_per = (M + P - 1) / P;
        P = (M + rows_per - 1) / rows_per;
        if (!af || P >= M) break;
        // AF: the rows b, b + P, ... of a workgroup share one offset when P
        // rows span a whole number of 16-byte chunks
        const uint64_t rb = ((uint64_t)xs * eb) & 15u;
        const int64_t q = rb == 0 ? 1 : rb % 8 == 0 ? 2 : rb % 4 == 0 ? 4 : rb % 2 == 0 ? 8 : 16;
        if (P >= q) {
            P = P / q * q;
            rows_per = (M + P - 1) / P;
            break;
        }
        af = false;  // too few workgroups for that: the row-offset tile
        g = g_off;
    }
    bwd_fn fn = mis   ? bwd_mis_lookup(xdt, w ? wdt : xdt, g.vpt, g.two_pass, res, nt, deep)
                : res ? bwd_lookup_res(xdt, w ? wdt : xdt, g.vec, g.vpt, g.two_pass, nt)
                      : bwd_lookup_plain(xdt, w ? wdt : xdt, g.vec, g.vpt, g.two_pass, nt, deep);
    if (fn == nullptr) return fail(RMSN_ERR_INVALID_ARG, "no kernel for vec %d vpt %d", g.vec, g.vpt);
    if (use_scratch && dw != nullptr) {
        if ((uint64_t)P * (uint64_t)H * sizeof(float) > kScratchBytes)
            return fail(RMSN_ERR_WORKSPACE,
                        "the dw partial rows of this call (%lld x %lld float32) exceed the %zu-byte static scratch "
                        "of rmsnorm_bwd_noalloc; call rmsnorm_bwd with a workspace",
                        (long long)P, (long long)H, kScratchBytes);
        if ((st = scratch_partials(&ws)) != RMSN_OK) return st;
    }

    BwdParams p;
    p.dy = dy;
    p.x = x;
    p.w = w;
    p.rrms = rrms;
    p.dres = dres;
    p.dx = dx;
    p.partial = dw != nullptr ? static_cast<float *>(ws) : nullptr;
    p.dys = dys;
    p.xs = xs;
    p.dxs = dxs;
    p.drs = drs;
    p.M = M;
    p.rows_per_wg = rows_per;
    p.interleave = interleave ? 1 : 0;
    p.frame = af ? 1 : 0;
    p.H = (int)H;
    p.nvec = g.nvec;
    p.wpr = g.wpr;
    p.nchunks = g.nchunks;
    p.inv_h = (float)(1.0 / (double)H);
    void *args[] = {&p};
    if ((st = launch((const void *)fn, dim3((unsigned)P), dim3(64 * g.wpr), args, stream,
                     res ? "rmsnorm_bwd_residual" : "rmsnorm_bwd")) != RMSN_OK)
        return st;
    if (dw != nullptr) {
        const float *part = p.partial;
        int Pi = (int)P, Hi = (int)H;
        void *fargs[] = {(void *)&part, &Pi, &Hi, &dw};
        if ((st = launch(dw_finalize_kernel(), dim3((unsigned)((H + kFinCols - 1) / kFinCols)),
                         dim3(kFinCols * kFinSlices), fargs, stream, "rmsnorm_dw_finalize")) != RMSN_OK)
            return st;
    }
    return RMSN_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

#define RMSN_API __attribute__((visibility("default")))

extern "C" {

RMSN_API rmsn_status_t rmsnorm_fwd(const void *x, int64_t x_stride, const void *w, void *y, int64_t y_stride,
                                   float *rrms, int64_t M, int64_t H, float eps, rmsn_dtype_t x_dtype,
                                   rmsn_dtype_t w_dtype, hipStream_t stream) {
    rmsn_status_t s = fwd_impl(MODE_PLAIN, x, x_stride, nullptr, 0, w, y, y_stride, nullptr, 0, rrms, M, H, eps,
                               x_dtype, w_dtype, Cond{}, LnExtra{}, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t rmsnorm_fwd_residual(const void *x, int64_t x_stride, const void *residual, int64_t r_stride,
                                   const void *w, void *y, int64_t y_stride, void *residual_out,
                                   int64_t ro_stride, float *rrms, int64_t M, int64_t H, float eps,
                                   rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream) {
    rmsn_status_t s = fwd_impl(MODE_RESID, x, x_stride, residual, r_stride, w, y, y_stride, residual_out, ro_stride,
                               rrms, M, H, eps, x_dtype, w_dtype, Cond{}, LnExtra{}, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t rmsnorm_adaln_fwd(const void *x, int64_t x_stride, const void *w, const void *scale,
                                         const void *shift, int64_t cond_stride, int64_t rows_per_cond, void *y,
                                         int64_t y_stride, float *rrms, int64_t M, int64_t H, float eps,
                                         rmsn_dtype_t x_dtype, rmsn_dtype_t param_dtype, hipStream_t stream) {
    Cond c;
    c.scale = scale;
    c.shift = shift;
    c.cs = cond_stride;
    c.rows_per_cond = rows_per_cond;
    rmsn_status_t s = fwd_impl(MODE_ADALN, x, x_stride, nullptr, 0, w, y, y_stride, nullptr, 0, rrms, M, H, eps,
                               x_dtype, param_dtype, c, LnExtra{}, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t layernorm_fwd(const void *x, int64_t x_stride, const void *w, const void *b, void *y,
                                     int64_t y_stride, float *mean, float *rstd, int64_t M, int64_t H, float eps,
                                     rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype, hipStream_t stream) {
    LnExtra e;
    e.bias = b;
    e.mean = mean;
    rmsn_status_t s = fwd_impl(kLn, x, x_stride, nullptr, 0, w, y, y_stride, nullptr, 0, rstd, M, H, eps, x_dtype,
                               w_dtype, Cond{}, e, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t layernorm_fwd_residual(const void *x, int64_t x_stride, const void *residual, int64_t r_stride,
                                              const void *w, const void *b, void *y, int64_t y_stride,
                                              void *residual_out, int64_t ro_stride, float *mean, float *rstd,
                                              int64_t M, int64_t H, float eps, rmsn_dtype_t x_dtype,
                                              rmsn_dtype_t w_dtype, hipStream_t stream) {
    LnExtra e;
    e.bias = b;
    e.mean = mean;
    rmsn_status_t s = fwd_impl(kLnResid, x, x_stride, residual, r_stride, w, y, y_stride, residual_out, ro_stride,
                               rstd, M, H, eps, x_dtype, w_dtype, Cond{}, e, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t H) { return bwd_workspace(M, H); }

RMSN_API rmsn_status_t rmsnorm_bwd(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride, const void *w,
                          const float *rrms, void *dx, int64_t dx_stride, float *dw, void *workspace,
                          size_t workspace_bytes, int64_t M, int64_t H, rmsn_dtype_t x_dtype,
                          rmsn_dtype_t w_dtype, hipStream_t stream) {
    rmsn_status_t s = bwd_impl(dy, dy_stride, x, x_stride, nullptr, 0, w, rrms, dx, dx_stride, dw, workspace,
                               workspace_bytes, M, H, x_dtype, w_dtype, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t rmsnorm_bwd_noalloc(const void *dy, int64_t dy_stride, const void *x, int64_t x_stride,
                                           const void *w, const float *rrms, void *dx, int64_t dx_stride, float *dw,
                                           int64_t M, int64_t H, rmsn_dtype_t x_dtype, rmsn_dtype_t w_dtype,
                                           hipStream_t stream) {
    rmsn_status_t s = bwd_impl(dy, dy_stride, x, x_stride, nullptr, 0, w, rrms, dx, dx_stride, dw, nullptr, 0, M,
                               H, x_dtype, w_dtype, stream, true);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API rmsn_status_t rmsnorm_bwd_residual(const void *dy, int64_t dy_stride, const void *h, int64_t h_stride,
                                            const void *dres, int64_t dres_stride, const void *w, const float *rrms,
                                            void *dh, int64_t dh_stride, float *dw, void *workspace,
                                            size_t workspace_bytes, int64_t M, int64_t H, rmsn_dtype_t x_dtype,
                                            rmsn_dtype_t w_dtype, hipStream_t stream) {
    rmsn_status_t s = bwd_impl(dy, dy_stride, h, h_stride, dres, dres_stride, w, rrms, dh, dh_stride, dw, workspace,
                               workspace_bytes, M, H, x_dtype, w_dtype, stream);
    return s == RMSN_OK ? ok() : s;
}

RMSN_API const char *rmsnorm_status_string(rmsn_status_t s) {
    switch (s) {
    case RMSN_OK: return "RMSN_OK";
    case RMSN_ERR_INVALID_ARG: return "RMSN_ERR_INVALID_ARG";
    case RMSN_ERR_UNSUPPORTED: return "RMSN_ERR_UNSUPPORTED";
    case RMSN_ERR_WORKSPACE: return "RMSN_ERR_WORKSPACE";
    case RMSN_ERR_HIP: return "RMSN_ERR_HIP";
    default: break;
    }
    return "RMSN_UNKNOWN_STATUS";
}

RMSN_API const char *rmsnorm_last_error(void) { return last_error(); }

RMSN_API void rmsnorm_tuning_set_streaming(int mode) { set_stream_mode(mode); }

RMSN_API void rmsnorm_tuning_set_geometry(int which, int vpt, int wpr, int third, int64_t grid) {
    set_override(which, vpt, wpr, third, grid);
}

RMSN_API rmsn_status_t rmsnorm_tuning_tile(int op, int64_t H, rmsn_dtype_t x_dtype, int layout, int32_t out[6]) {
    if (out == nullptr) return fail(RMSN_ERR_INVALID_ARG, "out is NULL");
    if (op < 0 || op > 6) return fail(RMSN_ERR_INVALID_ARG, "op = %d must be 0 .. 6", op);
    if (layout < 0 || layout > 2) return fail(RMSN_ERR_INVALID_ARG, "layout = %d must be 0, 1 or 2", layout);
    rmsn_status_t st = check_common(0, H, x_dtype, nullptr, x_dtype);
    if (st != RMSN_OK) return st;
    static const Kind kinds[7] = {Kind::Fwd, Kind::FwdResid, Kind::FwdAdaln, Kind::Ln,
                                  Kind::Bwd, Kind::BwdRes, Kind::Ln};
    const Kind kind = kinds[op];
    const int eb = dtype_bytes(x_dtype);
    const bool vec_ok = layout == 0 && H % (16 / eb) == 0;
    bool mis = false;
    int elem_groups = 0;
    const bool bwd = op == 4 || op == 5;
    Geom g = bwd ? bwd_tile(kind, (int)H, eb, vec_ok, !vec_ok, &mis, &elem_groups)
                 : fwd_tile(kind, (int)H, eb, eb, vec_ok, !vec_ok, &mis, op == 6);
    const bool frame = layout == 2 && bwd && mis && !g.two_pass && bwd_frame_tile(kind, (int)H, eb, &g);
    out[0] = g.vec;
    out[1] = g.two_pass ? 0 : g.vpt;
    out[2] = g.two_pass ? 0 : g.wpr;
    out[3] = bwd ? 1 : g.rpw;
    out[4] = frame ? 2 : mis ? 1 : 0;
    out[5] = g.two_pass ? 1 : 0;
    return ok();
}

}  // extern "C"
