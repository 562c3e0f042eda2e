// rope_api.hip -- host side of the RoPE apply step: argument validation,
// launch geometry and the extern "C" entry point declared in include/rope.h.
// Nothing here allocates, frees or synchronises; argument errors are found
// before the first HIP call.

#include <hip/hip_runtime.h>

#include "host_common.hpp"
#include "kernel_tables.hpp"
#include "rope.h"

namespace {

using namespace rmsn;
using namespace rmsn::host;

constexpr int64_t kMaxHeadDim = 65536;
constexpr int64_t kMaxRowElems = int64_t(1) << 24;  // num_heads * head_dim

// The byte range of an (rows, heads, head_dim) view as a Region: `rows`
// rows of (heads - 1) * head_stride + head_dim elements.
Region view3(const char *name, const void *p, int64_t rs, int64_t hs, int64_t rows, int64_t heads, int64_t hd,
             int eb) {
    return mat(name, p, rs, rows, (heads - 1) * hs + hd, eb);
}

rmsn_status_t check_view(const char *rname, const char *hname, int64_t rs, int64_t hs, int64_t rows, int64_t heads,
                         int64_t hd, int eb) {
    if (hs < hd)
        return fail(RMSN_ERR_INVALID_ARG, "%s = %lld is smaller than head_dim = %lld", hname, (long long)hs,
                    (long long)hd);
    if (hs > (INT64_MAX / eb) / heads) return fail(RMSN_ERR_INVALID_ARG, "%s * num_heads overflows", hname);
    return check_stride(rname, rs, rows, (heads - 1) * hs + hd, eb);
}

rmsn_status_t rope_impl(const void *x, int64_t xrs, int64_t xhs, const void *cos_t, const void *sin_t, int64_t ts,
                        void *out, int64_t ors, int64_t ohs, int64_t B, int64_t S, int64_t NH, int64_t D,
                        int transpose, rmsn_dtype_t xdt, rmsn_dtype_t tdt, hipStream_t stream) {
    if (!dtype_valid(xdt)) return fail(RMSN_ERR_UNSUPPORTED, "x_dtype %d is not RMSN_F32/F16/BF16", (int)xdt);
    if (!(tdt == xdt || tdt == RMSN_F32))
        return fail(RMSN_ERR_UNSUPPORTED, "table_dtype %d must equal x_dtype %d or be RMSN_F32", (int)tdt, (int)xdt);
    if (B < 0) return fail(RMSN_ERR_INVALID_ARG, "batch = %lld is negative", (long long)B);
    if (S < 1) return fail(RMSN_ERR_INVALID_ARG, "seq_len = %lld must be >= 1", (long long)S);
    if (NH < 1) return fail(RMSN_ERR_INVALID_ARG, "num_heads = %lld must be >= 1", (long long)NH);
    if (D < 2 || D % 2 != 0)
        return fail(RMSN_ERR_INVALID_ARG, "head_dim = %lld must be even and >= 2", (long long)D);
    if (D > kMaxHeadDim) return fail(RMSN_ERR_UNSUPPORTED, "head_dim = %lld exceeds 65536", (long long)D);
    if (NH > kMaxRowElems / D)
        return fail(RMSN_ERR_UNSUPPORTED, "num_heads * head_dim = %lld * %lld exceeds 2^24", (long long)NH,
                    (long long)D);
    if (B > INT64_MAX / S) return fail(RMSN_ERR_INVALID_ARG, "batch * seq_len overflows");
    const int64_t rows = B * S;
    const int64_t half = D / 2;
    const int eb = dtype_bytes(xdt), tb = dtype_bytes(tdt);
    rmsn_status_t st;
    if ((st = check_view("x_row_stride", "x_head_stride", xrs, xhs, rows, NH, D, eb)) != RMSN_OK) return st;
    if ((st = check_view("out_row_stride", "out_head_stride", ors, ohs, rows, NH, D, eb)) != RMSN_OK) return st;
    if ((st = check_stride("table_stride", ts, S, half, tb)) != RMSN_OK) return st;
    if (rows == 0) return RMSN_OK;
    if (x == nullptr) return fail(RMSN_ERR_INVALID_ARG, "x is NULL");
    if (out == nullptr) return fail(RMSN_ERR_INVALID_ARG, "out is NULL");
    if (cos_t == nullptr || sin_t == nullptr) return fail(RMSN_ERR_INVALID_ARG, "cos and sin must not be NULL");

    Region ins[3] = {view3("x", x, xrs, xhs, rows, NH, D, eb), mat("cos", cos_t, ts, S, half, tb),
                     mat("sin", sin_t, ts, S, half, tb)};
    Region outs[1] = {view3("out", out, ors, ohs, rows, NH, D, eb)};
    if ((st = check_overlap(outs, 1, ins, 3)) != RMSN_OK) return st;
    // out may be x itself, never a table
    for (int i = 1; i < 3; ++i)
        if (outs[0].overlaps(ins[i])) return fail(RMSN_ERR_INVALID_ARG, "out overlaps %s", ins[i].name);

    // 16-byte accesses when every half-head starts on a 16-byte boundary
    const int vecw = 16 / eb;
    const bool vec_ok = half % vecw == 0 && aligned16(x) && aligned16(out) && xrs % vecw == 0 && xhs % vecw == 0 &&
                        ors % vecw == 0 && ohs % vecw == 0 && aligned16(cos_t) && aligned16(sin_t) &&
                        ts % (16 / tb) == 0;
    const int vec = vec_ok ? vecw : 1;
    const int64_t nvec = half / vec;
    // lane exchange when a head's 2*nvec lanes fit a wave: each head takes a
    // power-of-two group of lanes (padding lanes idle), so heads never
    // straddle waves
    bool xchg = vec > 1 && nvec <= 32;
    // One batch, half-heads of whole 128-byte lines, and a position's vectors
    // filling 256-thread workgroups exactly: the split layout, whose threads
    // then read two whole lines each, none idle.  Measured on gfx950 (split
    // against exchange, same bits): [1, 8192, 32, 128] bf16 68.9 % (63.9 %),
    // float32 78.2 % (71.1 %), f16 with float32 tables 68.3 % (66.0 %);
    // [1, 8192, 64, 128] bf16 74.8 % (69.4 %); [1, 8192, 32, 256] 75.0 %
    // (70.1 %); [1, 8192, 32, 64] float32 72.4 % (67.3 %); 8 and 16 heads
    // level or +1.3.  Not taken: two or more batches (split -3 to -12),
    // 64-byte half-heads ([1, 8192, 32, 64] bf16 -4.3), 40 heads of 128
    // (320 vectors a position, -7).
    const int64_t pos_vecs = NH * nvec;
    if (xchg && B == 1 && half * eb >= 128 && (pos_vecs % kRopeThreads == 0 || kRopeThreads % pos_vecs == 0))
        xchg = false;
    int group = 1;
    while (group < 2 * nvec) group *= 2;
    const Override ov = get_override(2);
    if (ov.set && ov.c == 1) xchg = false;
    const bool nt = use_streaming(2 * rows * NH * D * eb);
    rope_fn fn = rope_lookup(xdt, tdt, vec, nt, xchg);
    if (fn == nullptr) return fail(RMSN_ERR_INVALID_ARG, "no RoPE kernel for vec %d", vec);
    RopeParams p;
    p.x = x;
    p.cos = cos_t;
    p.sin = sin_t;
    p.out = out;
    p.xrs = xrs;
    p.xhs = xhs;
    p.ors = ors;
    p.ohs = ohs;
    p.ts = ts;
    p.S = S;
    p.B = B;
    p.half = (int)half;
    p.nvec = (int)nvec;
    p.group = group;
    const int64_t items = NH * (xchg ? group : nvec);
    if (items > INT32_MAX - kRopeThreads)
        return fail(RMSN_ERR_UNSUPPORTED, "num_heads * head_dim = %lld is too large", (long long)(NH * D));
    p.items = (int)items;
    p.sign = transpose ? -1.0f : 1.0f;
    if (S > (INT64_MAX - kRopeThreads) / items)
        return fail(RMSN_ERR_UNSUPPORTED, "seq_len = %lld is too large", (long long)S);
    if (xchg) {
        p.nwork = (S * items + kRopeThreads - 1) / kRopeThreads;
        p.ipw = p.tpw = p.iblocks = 0;  // unused
    } else {
        p.ipw = p.items < kRopeThreads ? p.items : kRopeThreads;
        p.tpw = kRopeThreads / p.ipw;
        p.iblocks = (p.items + p.ipw - 1) / p.ipw;
        p.nwork = ((S + p.tpw - 1) / p.tpw) * p.iblocks;  // no overflow: <= S * items + 255
    }
    int64_t grid = p.nwork;
    if (ov.set && ov.d > 0 && ov.d < grid) grid = ov.d;
    if (grid > INT32_MAX) grid = INT32_MAX;  // the work is walked grid-stride
    int cus = 0;  // the device must be a readable gfx950 before anything is enqueued
    if ((st = device_info(&cus)) != RMSN_OK) return st;
    void *args[] = {&p};
    return launch((const void *)fn, dim3((unsigned)grid), dim3(kRopeThreads), args, stream, "rope_apply");
}

}  // namespace

#define RMSN_API __attribute__((visibility("default")))

extern "C" {

RMSN_API rmsn_status_t rope_apply(const void *x, int64_t x_row_stride, int64_t x_head_stride, const void *cos,
                                  const void *sin, int64_t table_stride, void *out, int64_t out_row_stride,
                                  int64_t out_head_stride, int64_t batch, int64_t seq_len, int64_t num_heads,
                                  int64_t head_dim, int transpose, rmsn_dtype_t x_dtype, rmsn_dtype_t table_dtype,
                                  hipStream_t stream) {
    rmsn_status_t s = rope_impl(x, x_row_stride, x_head_stride, cos, sin, table_stride, out, out_row_stride,
                                out_head_stride, batch, seq_len, num_heads, head_dim, transpose, x_dtype,
                                table_dtype, stream);
    return s == RMSN_OK ? ok() : s;
}

}  // extern "C"
