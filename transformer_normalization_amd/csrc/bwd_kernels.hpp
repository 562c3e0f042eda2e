// bwd_kernels.hpp -- gfx950 RMSNorm backward: dx per row, dw per column.
//
// What is computed ("Skill: Write a Triton RMSNorm Kernel", "Required
// reasoning process" step 12 and "Correctness requirements"), from the saved
// per-row rrms (read, never recomputed), all in float32:
//   xn = x * rrms,  g = dy * w   (w = 1 when weightless)
//   c  = sum over the row of g * xn
//   dx = rrms * g - xn * ((c * (1/H)) * rrms)
//   dw[j] = sum over rows of dy * xn
//
// Kernel 1 (rmsnorm_bwd_kernel): workgroup b owns the contiguous block of
// rows [b*rows_per_wg, (b+1)*rows_per_wg) and walks it one row at a time with
// all 64*wpr threads.  The columns a thread owns are fixed (vector v = t +
// k*64*wpr), so it keeps the weight and its dw partial sums in registers for
// the whole block and, at the end, writes its float32 partials to row b of the
// workspace `partial` (P x H).  Longer rows use two passes: pass 1 forms c,
// pass 2 reloads x and dy, writes dx and adds dy*xn into the workgroup's own
// workspace row (no other workgroup touches it, so no atomics).
//
// NT kernels stream x, dy and dx past the caches (non-temporal accesses);
// weight, rrms and the partial sums use ordinary cached accesses.
//
// Kernel 2 (rmsnorm_dw_finalize): dw[j] = sum_p partial[p][j] in a fixed
// order (16 interleaved slices of p, then the 16 slice sums in slice order),
// so dw has the same bits on every run ("dweight ... is a separate kernel
// because it is a cross-row reduction", step 12).
#pragma once

#include "numerics.hpp"

namespace rmsn {

struct BwdParams {
    const void *dy;
    const void *x;
    const void *w;       // may be null (weightless)
    const float *rrms;
    void *dx;
    float *partial;      // P x H float32, or null when dw is not wanted
    int64_t dys, xs, dxs;  // row strides, elements
    int64_t M;
    int64_t rows_per_wg;
    int H;
    int nvec;
    int wpr;
    int nchunks;
    float inv_h;
};

template <int XDT, int WDT, int VEC, int VPT, bool TWO_PASS, bool NT, int MAXT>
__global__ void __launch_bounds__(MAXT) rmsnorm_bwd_kernel(const BwdParams p) {
    __shared__ float red[2][16];
    const int row_threads = 64 * p.wpr;  // == blockDim.x
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * p.rows_per_wg;
    const int64_t row1 = row0 + p.rows_per_wg < p.M ? row0 + p.rows_per_wg : p.M;
    float *part = p.partial != nullptr ? p.partial + (int64_t)blockIdx.x * p.H : nullptr;

    if constexpr (!TWO_PASS) {
        // x, dy and w stay packed in registers and are widened at each use;
        // only the dw partial sums are float32 registers.
        Raw<WDT, VEC> wr[VPT];
        float dwa[VPT][VEC];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = t + k * row_threads;
            if (p.w != nullptr && v < p.nvec)
                wr[k].load(p.w, (int64_t)v * VEC);
            else
                wr[k].fill_one();
#pragma unroll
            for (int e = 0; e < VEC; ++e) dwa[k][e] = 0.0f;
        }
        int parity = 0;
        for (int64_t row = row0; row < row1; ++row, parity ^= 1) {
            Raw<XDT, VEC> xr[VPT], dr[VPT];
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if (v < p.nvec) {
                    xr[k].template load<NT>(p.x, row * p.xs + (int64_t)v * VEC);
                    dr[k].template load<NT>(p.dy, row * p.dys + (int64_t)v * VEC);
                } else {
                    xr[k].zero();
                    dr[k].zero();
                }
            }
            const float rs = p.rrms[row];
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float xv[VEC], dv[VEC], wv[VEC];
                xr[k].widen_to(xv);
                dr[k].widen_to(dv);
                wr[k].widen_to(wv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(dv[e] * wv[e], xv[e] * rs, acc);
            }
            const float c = row_sum(acc, p.wpr, wave, &red[parity][0]);
            const float s = (c * p.inv_h) * rs;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                xr[k].opaque();
                dr[k].opaque();
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                float xv[VEC], dv[VEC], wv[VEC], o[VEC];
                xr[k].widen_to(xv);
                dr[k].widen_to(dv);
                wr[k].widen_to(wv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float xn = xv[e] * rs;
                    o[e] = rs * (dv[e] * wv[e]) - xn * s;
                    dwa[k][e] = __builtin_fmaf(dv[e], xn, dwa[k][e]);
                }
                if (v < p.nvec) store_elems<XDT, VEC, NT>(p.dx, row * p.dxs + (int64_t)v * VEC, o);
            }
        }
        if (part != nullptr) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if (v < p.nvec) store_elems<DT_F32, VEC>(part, (int64_t)v * VEC, dwa[k]);
            }
        }
    } else {
        const int chunk = row_threads * VPT;
        if (part != nullptr) {
            const float z[VEC] = {};
            for (int v = t; v < p.nvec; v += row_threads) store_elems<DT_F32, VEC>(part, (int64_t)v * VEC, z);
        }
        int parity = 0;
        for (int64_t row = row0; row < row1; ++row, parity ^= 1) {
            const float rs = p.rrms[row];
            float acc = 0.0f;
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (v < p.nvec) {
                        float xv[VEC], dv[VEC], wv[VEC];
                        // cached: pass 2 reads the same chunk again
                        load_elems<XDT, VEC>(p.x, row * p.xs + (int64_t)v * VEC, xv);
                        load_elems<XDT, VEC>(p.dy, row * p.dys + (int64_t)v * VEC, dv);
                        if (p.w != nullptr) {
                            load_elems<WDT, VEC>(p.w, (int64_t)v * VEC, wv);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) wv[e] = 1.0f;
                        }
#pragma unroll
                        for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(dv[e] * wv[e], xv[e] * rs, acc);
                    }
                }
            }
            const float cs = row_sum(acc, p.wpr, wave, &red[parity][0]);
            const float s = (cs * p.inv_h) * rs;
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (v < p.nvec) {
                        float xv[VEC], dv[VEC], wv[VEC], o[VEC];
                        load_elems<XDT, VEC, NT>(p.x, row * p.xs + (int64_t)v * VEC, xv);
                        load_elems<XDT, VEC, NT>(p.dy, row * p.dys + (int64_t)v * VEC, dv);
                        if (p.w != nullptr) {
                            load_elems<WDT, VEC>(p.w, (int64_t)v * VEC, wv);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) wv[e] = 1.0f;
                        }
                        float xn[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            xn[e] = xv[e] * rs;
                            o[e] = rs * (dv[e] * wv[e]) - xn[e] * s;
                        }
                        store_elems<XDT, VEC, NT>(p.dx, row * p.dxs + (int64_t)v * VEC, o);
                        if (part != nullptr) {
                            float pa[VEC];
                            load_elems<DT_F32, VEC>(part, (int64_t)v * VEC, pa);
#pragma unroll
                            for (int e = 0; e < VEC; ++e) pa[e] = __builtin_fmaf(dv[e], xn[e], pa[e]);
                            store_elems<DT_F32, VEC>(part, (int64_t)v * VEC, pa);
                        }
                    }
                }
            }
        }
    }
}

// dw[j] = sum over p of partial[p][j]: 64 columns x 16 slices per workgroup
// of 1024 threads.  Thread (col, s) sums p = s, s+16, ... in increasing p;
// the 16 slice sums are then added in slice order.
__global__ void __launch_bounds__(1024) rmsnorm_dw_finalize(const float *__restrict__ partial, int P, int H,
                                                            float *__restrict__ dw) {
    __shared__ float sums[16][64];
    const int lane = threadIdx.x & 63;
    const int s = threadIdx.x >> 6;
    const int col = blockIdx.x * 64 + lane;
    float acc = 0.0f;
    if (col < H) {
        for (int q = s; q < P; q += 16) acc += partial[(int64_t)q * H + col];
    }
    sums[s][lane] = acc;
    __syncthreads();
    if (s == 0 && col < H) {
        float tot = sums[0][lane];
#pragma unroll
        for (int i = 1; i < 16; ++i) tot += sums[i][lane];
        dw[col] = tot;
    }
}

}  // namespace rmsn
