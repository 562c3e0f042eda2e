// rope_kernels.hpp -- gfx950 RoPE apply (rotate-half rotation by tabulated
// angles; "rocm-kernels", "Core Kernel Implementations", 2. RoPE 3D, and
// Template 2).
//
// An elementwise, HBM-bound step: every element of x is read once and its
// rotated value written once; the cos/sin tables (seq_len rows) are read by
// every head and every batch of a position, so they come from the caches.
//
// Work item = (position s, head h, vector v): a thread holds the VEC
// elements j = v*VEC .. v*VEC+VEC-1 of the first half of head h and the
// matching elements of the second half (two 16-byte accesses head_dim/2
// apart), and the VEC table entries of those columns, which it loads once and
// applies to every batch b of position s (rows b * seq_len + s).  Consecutive
// lanes take consecutive vectors of one head, then the next head, so a wave's
// two loads together cover a contiguous stretch of the token row.
//
// Mapping: a workgroup of 256 threads covers `tpw` positions x `ipw` items;
// blockIdx.y selects the block of items when one position has more than 256.
#pragma once

#include "numerics.hpp"

namespace rmsn {

struct RopeParams {
    const void *x;
    const void *cos;
    const void *sin;
    void *out;
    int64_t xrs, xhs;  // x row and head strides, elements
    int64_t ors, ohs;  // out row and head strides
    int64_t ts;        // table row stride
    int64_t S;         // seq_len
    int64_t B;         // batch
    int half;          // head_dim / 2
    int nvec;          // vectors per half head (half / VEC)
    int items;         // num_heads * nvec
    int ipw;           // items per workgroup row (<= 256)
    int tpw;           // positions per workgroup
    float sign;        // +1, or -1 for the transposed rotation
};

constexpr int kRopeThreads = 256;

template <int XDT, int TDT, int VEC, bool NT>
__global__ void __launch_bounds__(kRopeThreads) rope_apply_kernel(const RopeParams p) {
    const int t = threadIdx.x;
    const int lt = t / p.ipw;
    const int item = blockIdx.y * p.ipw + (t - lt * p.ipw);
    const int64_t s = (int64_t)blockIdx.x * p.tpw + lt;
    if (lt >= p.tpw || item >= p.items || s >= p.S) return;
    const int h = item / p.nvec;
    const int col = (item - h * p.nvec) * VEC;

    float c[VEC], sn[VEC];
    load_elems<TDT, VEC>(p.cos, s * p.ts + col, c);
    load_elems<TDT, VEC>(p.sin, s * p.ts + col, sn);
#pragma unroll
    for (int e = 0; e < VEC; ++e) sn[e] *= p.sign;  // exact

    const int64_t xoff = s * p.xrs + (int64_t)h * p.xhs + col;
    const int64_t ooff = s * p.ors + (int64_t)h * p.ohs + col;
    const int64_t xstep = p.S * p.xrs;  // one batch further
    const int64_t ostep = p.S * p.ors;
    // two batches per iteration: both rows' loads are issued before either
    // row is stored (an output may be the input itself, but each thread
    // reads its own elements of a row before writing them)
    int64_t b = 0;
    for (; b + 1 < p.B; b += 2) {
        float x0[2][VEC], x1[2][VEC];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            load_elems<XDT, VEC, NT>(p.x, xoff + (b + u) * xstep, x0[u]);
            load_elems<XDT, VEC, NT>(p.x, xoff + (b + u) * xstep + p.half, x1[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float o0[VEC], o1[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                o0[e] = __builtin_fmaf(x0[u][e], c[e], -(x1[u][e] * sn[e]));
                o1[e] = __builtin_fmaf(x0[u][e], sn[e], x1[u][e] * c[e]);
            }
            store_elems<XDT, VEC, NT>(p.out, ooff + (b + u) * ostep, o0);
            store_elems<XDT, VEC, NT>(p.out, ooff + (b + u) * ostep + p.half, o1);
        }
    }
    if (b < p.B) {
        float x0[VEC], x1[VEC], o0[VEC], o1[VEC];
        load_elems<XDT, VEC, NT>(p.x, xoff + b * xstep, x0);
        load_elems<XDT, VEC, NT>(p.x, xoff + b * xstep + p.half, x1);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            o0[e] = __builtin_fmaf(x0[e], c[e], -(x1[e] * sn[e]));
            o1[e] = __builtin_fmaf(x0[e], sn[e], x1[e] * c[e]);
        }
        store_elems<XDT, VEC, NT>(p.out, ooff + b * ostep, o0);
        store_elems<XDT, VEC, NT>(p.out, ooff + b * ostep + p.half, o1);
    }
}

}  // namespace rmsn
