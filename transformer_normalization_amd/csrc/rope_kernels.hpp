// rope_kernels.hpp -- gfx950 RoPE apply (rotate-half rotation by tabulated
// angles; "rocm-kernels", "Core Kernel Implementations", 2. RoPE 3D, and
// Template 2).
//
// An elementwise, HBM-bound step: every element of x is read once and its
// rotated value written once; the cos/sin tables (seq_len rows) are read by
// every head and every batch of a position, so they come from the caches.
//
// Two layouts of the work, both applying a position's table entries (loaded
// once per thread) to every batch b of that position (rows b * seq_len + s):
//
//  - lane exchange (XCHG, the default when a half head is at most 32 16-byte
//    vectors): a head takes a group of `group` lanes, 2*nvec rounded up to a
//    power of two; lane k < 2*nvec of the group holds vector k of the head
//    (lanes above stay idle), so every load and store instruction of a wave
//    covers whole contiguous runs of a head; the partner element j + D/2 (or
//    j - D/2) is fetched from lane k + nvec (or k - nvec) with ds_bpermute.
//  - split (single elements, and longer heads): a thread holds the VEC
//    elements j.. of the first half and the matching elements of the second
//    half (two accesses head_dim/2 apart).
//
// Mapping of the exchange layout: the (position, item) pairs are numbered
// position-major, item fastest, and work unit u is the 256 pairs u*256 ..
// u*256+255; thread t of a workgroup takes pair u*256 + t.  No thread idles
// whatever the number of items per position (a position may span several
// units, a unit several positions), neighbouring threads and workgroups
// cover neighbouring bytes of a token row, and a head's lanes stay whole and
// aligned inside one wave (the items of a position are a multiple of the
// group, which divides 64).
//
// Mapping of the split layout: a workgroup covers `tpw` positions x `ipw`
// items; a position with more than 256 items takes `iblocks` consecutive
// workgroups.  (The flat numbering measured slower here, by 2-11 %, even
// though this mapping leaves threads idle when the items of a position are
// not a divisor or multiple of 256.)
//
// Units are walked grid-stride in both, so a capped grid also works.
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
    int group;         // exchange: lanes per head, 2 * nvec rounded up to a power of two (<= 64)
    int items;         // work items per position: num_heads * nvec (split), * group (exchange)
    int64_t nwork;     // work units: ceil(S * items / 256) (exchange), nblocks * iblocks (split)
    int ipw;           // split: items per workgroup row (<= 256)
    int tpw;           // split: positions per workgroup
    int iblocks;       // split: item blocks per position block, ceil(items / ipw)
    float sign;        // +1, or -1 for the transposed rotation
};

constexpr int kRopeThreads = 256;

// out0 = x0 c - x1 s and out1 = x1 c + x0 s: each output is
// fma(own, c, partner * s') with s' = -s for the first half and +s for the
// second, so both halves (and both layouts) evaluate the same expression
__device__ __forceinline__ float rot_lo(float x0, float x1, float c, float sn) {
    return __builtin_fmaf(x0, c, x1 * -sn);
}
__device__ __forceinline__ float rot_hi(float x0, float x1, float c, float sn) {
    return __builtin_fmaf(x1, c, x0 * sn);
}

template <int DT, int N>
__device__ __forceinline__ Raw<DT, N> from_lane(const Raw<DT, N> &r, int byte_addr) {
    Raw<DT, N> o;
#pragma unroll
    for (int c = 0; c < Raw<DT, N>::CHUNKS; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            o.v[c][w] = (uint32_t)__builtin_amdgcn_ds_bpermute(byte_addr, (int)r.v[c][w]);
    return o;
}

template <int XDT, int TDT, int VEC, bool NT, bool XCHG>
__global__ void __launch_bounds__(kRopeThreads) rope_apply_kernel(const RopeParams p) {
    const int t = threadIdx.x;
    const int64_t xstep = p.S * p.xrs;  // one batch further
    const int64_t ostep = p.S * p.ors;
    // pair u*256 + t as (position s, item); the division of the unit's first
    // pair is uniform, the thread's offset from it is below items + 256
    auto pair_of = [&](int64_t wk, int64_t &s, int &item) {
        const int64_t first = wk * kRopeThreads;
        const int64_t s0 = first / p.items;
        const int idx = (int)(first - s0 * p.items) + t;
        const int q = (int)((unsigned)idx / (unsigned)p.items);
        s = s0 + q;
        item = idx - q * p.items;
    };

    // Batches are taken two at a time.  The rows of a pair are requested
    // before the table entries of the position, so the latency of the table
    // loads overlaps that of the rows instead of adding to it (the tables are
    // needed first, but a wait for them would otherwise hold back every row
    // load behind it).  `two` depends only on the batch count: uniform.
    if constexpr (XCHG) {
        static_assert(VEC > 1, "the exchange layout moves 16-byte vectors");
        const int per_head = p.group;
        // lane k of a group (the same for every unit: units start on group
        // boundaries) and its partner, k + nvec or k - nvec
        const int k = t & (per_head - 1);
        const bool upper = k >= p.nvec;
        const int partner = ((t & 63) + (upper ? -p.nvec : p.nvec)) << 2;  // ds_bpermute byte address
        if (k >= 2 * p.nvec) return;  // padding lane of the group: no element
        for (int64_t wk = blockIdx.x; wk < p.nwork; wk += gridDim.x) {
            int64_t s;
            int item;
            pair_of(wk, s, item);
            // partners share the position: both go on or both skip (items is
            // a multiple of per_head)
            if (s >= p.S) continue;
            const int h = item / per_head;
            const int col = (upper ? k - p.nvec : k) * VEC;  // table column
            const int64_t xoff = s * p.xrs + (int64_t)h * p.xhs + k * VEC;
            const int64_t ooff = s * p.ors + (int64_t)h * p.ohs + k * VEC;
            Raw<XDT, VEC> r[2];
            auto load_pair = [&](int64_t b, bool two) {
                r[0].template load<NT>(p.x, xoff + b * xstep);
                if (two)
                    r[1].template load<NT>(p.x, xoff + (b + 1) * xstep);
                else
                    r[1].zero();
            };
            load_pair(0, p.B > 1);
            float c[VEC], sn[VEC];
            load_elems<TDT, VEC>(p.cos, s * p.ts + col, c);
            load_elems<TDT, VEC>(p.sin, s * p.ts + col, sn);
            // s' = +-s: the transposed rotation negates s, the first half
            // of a head negates it again (exact)
            const float sg = upper ? p.sign : -p.sign;
#pragma unroll
            for (int e = 0; e < VEC; ++e) sn[e] *= sg;
            // one packed 32-bit word at a time keeps few values live
            // (the kernel stays within 64 VGPRs: 8 waves per SIMD)
            auto finish = [&](const Raw<XDT, VEC> &mine, int64_t o) {
                const Raw<XDT, VEC> theirs = from_lane(mine, partner);
                constexpr int PW = 4 / Fmt<XDT>::bytes;  // elements per word
                u32x4 res;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float a[PW], b[PW], out[PW];
                    unpack_word<XDT>(mine.v[0][w], a);
                    unpack_word<XDT>(theirs.v[0][w], b);
#pragma unroll
                    for (int e = 0; e < PW; ++e) {
                        const int j = w * PW + e;
                        out[e] = __builtin_fmaf(a[e], c[j], b[e] * sn[j]);  // rot_lo / rot_hi of this half
                    }
                    res[w] = pack_word<XDT>(out);
                }
                u32x4 *dst = reinterpret_cast<u32x4 *>(static_cast<char *>(p.out) + o * Fmt<XDT>::bytes);
                if constexpr (NT)
                    __builtin_nontemporal_store(res, dst);
                else
                    *dst = res;
            };
            for (int64_t b = 0;;) {
                const bool two = b + 1 < p.B;
                finish(r[0], ooff + b * ostep);
                if (two) finish(r[1], ooff + (b + 1) * ostep);
                b += 2;
                if (b >= p.B) break;
                load_pair(b, b + 1 < p.B);
            }
        }
    } else {
        const int lt = t / p.ipw;
        const int it = t - lt * p.ipw;
        if (lt >= p.tpw) return;
        for (int64_t wk = blockIdx.x; wk < p.nwork; wk += gridDim.x) {
            const int64_t pb = wk / p.iblocks;
            const int item = (int)(wk - pb * p.iblocks) * p.ipw + it;
            const int64_t s = pb * p.tpw + lt;
            if (s >= p.S || item >= p.items) continue;
            const int h = item / p.nvec;
            const int col = (item - h * p.nvec) * VEC;
            const int64_t xoff = s * p.xrs + (int64_t)h * p.xhs + col;
            const int64_t ooff = s * p.ors + (int64_t)h * p.ohs + col;
            // each thread reads its own elements of a row before writing
            // them, so an output may be the input itself
            float x0[2][VEC], x1[2][VEC];
            auto load_pair = [&](int64_t b, bool two) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u == 0 || two) {
                        load_elems<XDT, VEC, NT>(p.x, xoff + (b + u) * xstep, x0[u]);
                        load_elems<XDT, VEC, NT>(p.x, xoff + (b + u) * xstep + p.half, x1[u]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) x0[u][e] = x1[u][e] = 0.0f;
                    }
                }
            };
            load_pair(0, p.B > 1);
            float c[VEC], sn[VEC];
            load_elems<TDT, VEC>(p.cos, s * p.ts + col, c);
            load_elems<TDT, VEC>(p.sin, s * p.ts + col, sn);
#pragma unroll
            for (int e = 0; e < VEC; ++e) sn[e] *= p.sign;  // exact
            for (int64_t b = 0;;) {
                const bool two = b + 1 < p.B;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (u == 0 || two) {
                        float o0[VEC], o1[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            o0[e] = rot_lo(x0[u][e], x1[u][e], c[e], sn[e]);
                            o1[e] = rot_hi(x0[u][e], x1[u][e], c[e], sn[e]);
                        }
                        store_elems<XDT, VEC, NT>(p.out, ooff + (b + u) * ostep, o0);
                        store_elems<XDT, VEC, NT>(p.out, ooff + (b + u) * ostep + p.half, o1);
                    }
                }
                b += 2;
                if (b >= p.B) break;
                load_pair(b, b + 1 < p.B);
            }
        }
    }
}

}  // namespace rmsn
