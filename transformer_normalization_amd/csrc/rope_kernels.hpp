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
//  - lane exchange (XCHG, the default when a half head is a power-of-two
//    number <= 32 of 16-byte vectors): lane k of a head's 2*nvec lanes holds
//    vector k of the head, so every load and store instruction of a wave
//    covers whole contiguous 128-byte lines; the partner element j + D/2 (or
//    j - D/2) is fetched from lane k ^ nvec with ds_bpermute.
//  - split (any other shape, and single elements): a thread holds the VEC
//    elements j.. of the first half and the matching elements of the second
//    half (two accesses head_dim/2 apart).
//
// Mapping: a workgroup of 256 threads covers `tpw` positions x `ipw` items.
// When one position has more than 256 items it takes `iblocks` consecutive
// workgroups, so neighbouring workgroups cover neighbouring bytes of a token
// row (a position-major order would leave strided holes in each row).  The
// (position block, item block) pairs are walked grid-stride, so a capped
// grid also works.
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
    int items;         // work items per position: num_heads * nvec (split), * 2 nvec (exchange)
    int ipw;           // items per workgroup row (<= 256)
    int tpw;           // positions per workgroup
    int64_t nblocks;   // position blocks: ceil(S / tpw)
    int iblocks;       // item blocks per position block: ceil(items / ipw)
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
    const int lt = t / p.ipw;
    const int it = t - lt * p.ipw;
    if (lt >= p.tpw) return;
    const int64_t xstep = p.S * p.xrs;  // one batch further
    const int64_t ostep = p.S * p.ors;
    const int64_t nwork = p.nblocks * p.iblocks;

    // Batches are taken two at a time.  The rows of a pair are requested
    // before the table entries of the position, so the latency of the table
    // loads overlaps that of the rows instead of adding to it (the tables are
    // needed first, but a wait for them would otherwise hold back every row
    // load behind it).  `two` depends only on the batch count: uniform.
    if constexpr (XCHG) {
        static_assert(VEC > 1, "the exchange layout moves 16-byte vectors");
        const int per_head = 2 * p.nvec;
        const int partner = ((t & 63) ^ p.nvec) << 2;  // ds_bpermute byte address
        for (int64_t wk = blockIdx.x; wk < nwork; wk += gridDim.x) {
            const int64_t pb = wk / p.iblocks;
            const int item = (int)(wk - pb * p.iblocks) * p.ipw + it;
            const int64_t s = pb * p.tpw + lt;
            // partners share the position and the item block: both go on or
            // both skip (items is a multiple of per_head)
            if (s >= p.S || item >= p.items) continue;
            const int h = item / per_head;
            const int k = item - h * per_head;  // == t % per_head: heads are aligned to per_head lanes
            const bool upper = k >= p.nvec;
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
        for (int64_t wk = blockIdx.x; wk < nwork; wk += gridDim.x) {
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
