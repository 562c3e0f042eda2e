// fwd_kernels.hpp -- gfx950 forward RMSNorm and fused residual pre-norm.
//
// What is computed ("Skill: Write a Triton RMSNorm Kernel", "Required
// reasoning process" steps 1-11 and "Kernel design rules"):
//   h      = x                     (plain form)
//   h      = float32(x) + float32(r)  (fused residual; r_out = RNE(h))
//   rrms   = rsqrt(sum(h*h) * (1/H) + eps)     in float32, eps inside the root
//   y      = (h * rrms) * w                     (w = 1 when weightless)
//   y      = fma((h * rrms) * w, 1 + scale, shift)   (AdaLN: "rocm-kernels",
//            "Core Kernel Implementations", 4. AdaLN; scale and shift come from
//            conditioning row i / rows_per_cond, in the weight's format)
//
// Layout of the work on the device:
//   * A "row group" of 64*wpr threads (wpr whole waves) owns one row at a
//     time; a workgroup holds rpw row groups.  Workgroups walk the rows
//     grid-stride: row group `slot` of workgroup b takes rows
//     (b + it*gridDim.x)*rpw + slot for it = 0 .. iters-1.  iters is the same
//     for every thread, so the workgroup barriers inside row_sum are reached
//     uniformly; rows past M are processed as zeros and never stored.
//   * Thread t of a row group owns the VEC-element vectors t, t+64*wpr, ...,
//     t+(VPT-1)*64*wpr of the row, so a wave's load is 64 consecutive 16-byte
//     vectors (1 KiB) and the columns a thread owns never change between
//     rows; the weight is loaded once into registers.
//   * Resident path (the row fits: nvec <= 64*wpr*VPT): the row is loaded
//     once, stays in registers through the reduction and is scaled and
//     stored from registers -- one HBM read and one write per element
//     ("Required reasoning process", step 3, the persistent pattern).
//   * Two-pass path (longer rows): pass 1 sums squares chunk by chunk, pass 2
//     reloads each chunk with the same bounds and scales it (step 11).
//   * MIS kernels take rows off the 16-byte grid (a start that is not
//     16-byte aligned, or a length that is not a whole number of vectors) in
//     the same 16-byte vectors, each read and written with one access at the
//     row's own byte offset.  When a row's last vector is only partly inside
//     the row, its lane takes the row's last 16 bytes instead (columns
//     H - VEC .. H - 1): the window's leading `dup` columns are also the
//     previous vector's and are left out of its sum of squares.  Resident,
//     it computes and writes the same values for them after the row's
//     reduction; in two passes it reads the window in pass 1 only and writes
//     its own columns one by one.  No access leaves the row.
//   * NT kernels stream x, r, y and r_out past the caches (non-temporal
//     accesses); the weight and rrms use ordinary cached accesses.
//   * The reduction is a per-thread float32 sum over the thread's elements in
//     column order, then a DPP wave sum and, for wpr > 1, a fixed-order sum
//     of the wave totals through LDS.  The tree depends only on (H, VEC, VPT,
//     wpr), never on strides, alignment of rows or timing.
#pragma once

#include "numerics.hpp"

namespace rmsn {

struct FwdParams {
    const void *x;
    const void *r;   // residual (fused form only)
    const void *w;   // may be null (weightless)
    void *y;
    void *ro;        // residual_out, may be null
    float *rrms;     // may be null
    int64_t xs, rs, ys, ros;  // row strides, elements
    int64_t M;
    int64_t iters;   // row-group iterations per workgroup
    int H;
    int nvec;        // vectors of VEC elements per row
    int wpr;         // waves per row group
    int rpw;         // row groups per workgroup
    int nchunks;     // two-pass: chunks of 64*wpr*VPT vectors
    float eps;
    float inv_h;     // float32(1/H)
    // AdaLN conditioning: scale and shift rows (parameter format), row i uses
    // conditioning row i / rows_per_cond
    const void *scale;
    const void *shift;
    int64_t cs;            // conditioning row stride, elements
    int64_t rows_per_cond;
};

enum : int { MODE_PLAIN = 0, MODE_RESID = 1, MODE_ADALN = 2 };

template <int XDT, int WDT, int VEC, int VPT, int MODE, bool TWO_PASS, bool NT, int MAXT, bool MIS = false>
__global__ void __launch_bounds__(MAXT) rmsnorm_fwd_kernel(const FwdParams p) {
    static_assert(!MIS || VEC * Fmt<XDT>::bytes == 16, "rows off the grid: 16-byte vector tiles");
    constexpr int ES = Fmt<XDT>::bytes;
    constexpr int WES = Fmt<WDT>::bytes;
    constexpr bool RESID = MODE == MODE_RESID;
    constexpr bool ADALN = MODE == MODE_ADALN;
    __shared__ float red[2][16];
    const int row_threads = 64 * p.wpr;
    const int slot = threadIdx.x / row_threads;
    const int t = threadIdx.x - slot * row_threads;
    const int wave_in_row = t >> 6;
    const int64_t gstride = (int64_t)gridDim.x;

    if constexpr (!TWO_PASS) {
        // Loaded data stays packed in registers and is widened at each use
        // (one VALU op per element), which halves the register footprint of
        // 16-bit formats; every widening of an element gives the same float.
        Raw<WDT, VEC> wr[VPT];
        // rows off the grid: first column of the thread's window, and how
        // many of its leading columns are the previous vector's
        int col0[VPT], dup[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = t + k * row_threads;
            col0[k] = MIS && v * VEC > p.H - VEC ? p.H - VEC : v * VEC;
            dup[k] = MIS ? v * VEC - col0[k] : 0;
            if (p.w != nullptr && v < p.nvec) {
                if constexpr (MIS) {
#pragma unroll
                    for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
                        wr[k].v[c] = load16_at<false>(static_cast<const char *>(p.w) + (int64_t)col0[k] * WES + 16 * c);
                } else {
                    wr[k].load(p.w, (int64_t)v * VEC);
                }
            } else {
                wr[k].fill_one();
            }
        }

        // AdaLN conditioning rows stay in registers while consecutive rows of
        // this row group use the same one (rows of one batch)
        Raw<WDT, VEC> scr[ADALN ? VPT : 1], shr[ADALN ? VPT : 1];
        int64_t have_crow = -1;
        // A row's loads are issued before the loop (first row) or at the end
        // of the previous iteration, never behind a wait: loaded before a loop
        // that uses them, the weights would otherwise be waited for in the
        // loop's preheader, ahead of the first row's loads, and every
        // workgroup would pay two memory latencies in a row.
        Raw<XDT, VEC> xr[VPT];
        Raw<XDT, VEC> rr[RESID ? VPT : 1];
        auto load_row = [&](int64_t it) {
            const int64_t row = ((int64_t)blockIdx.x + it * gstride) * p.rpw + slot;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if (row < p.M && v < p.nvec) {
                    if constexpr (MIS) {
                        xr[k].v[0] = load16_at<NT>(static_cast<const char *>(p.x) + (row * p.xs + col0[k]) * ES);
                        if constexpr (RESID)
                            rr[k].v[0] = load16_at<NT>(static_cast<const char *>(p.r) + (row * p.rs + col0[k]) * ES);
                    } else {
                        xr[k].template load<NT>(p.x, row * p.xs + (int64_t)v * VEC);
                        if constexpr (RESID) rr[k].template load<NT>(p.r, row * p.rs + (int64_t)v * VEC);
                    }
                } else {
                    xr[k].zero();
                    if constexpr (RESID) rr[k].zero();
                }
            }
            // the row's conditioning row travels with it (same wait), unless
            // the previous row already used it
            if constexpr (ADALN) {
                const int64_t crow = row / p.rows_per_cond;
                if (row < p.M && crow != have_crow) {
#pragma unroll
                    for (int k = 0; k < VPT; ++k) {
                        const int v = t + k * row_threads;
                        if (v < p.nvec) {
                            // cached: a conditioning row serves rows_per_cond rows
                            if constexpr (MIS) {
#pragma unroll
                                for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c) {
                                    const int64_t o = (crow * p.cs + col0[k]) * WES + 16 * c;
                                    scr[k].v[c] = load16_at<false>(static_cast<const char *>(p.scale) + o);
                                    shr[k].v[c] = load16_at<false>(static_cast<const char *>(p.shift) + o);
                                }
                            } else {
                                scr[k].load(p.scale, crow * p.cs + (int64_t)v * VEC);
                                shr[k].load(p.shift, crow * p.cs + (int64_t)v * VEC);
                            }
                        } else {
                            scr[k].zero();
                            shr[k].zero();
                        }
                    }
                    have_crow = crow;
                }
            }
        };
        load_row(0);
        for (int64_t it = 0; it < p.iters; ++it) {
            const int64_t row = ((int64_t)blockIdx.x + it * gstride) * p.rpw + slot;
            const bool valid = row < p.M;
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float hv[VEC];
                xr[k].widen_to(hv);
                if constexpr (RESID) {
                    float rv[VEC];
                    rr[k].widen_to(rv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                    // Aligned rows: each element is read and written by one
                    // thread, so r_out may go out now.  Off the grid it waits
                    // for the row barrier (below).
                    const int v = t + k * row_threads;
                    if (!MIS && p.ro != nullptr && valid && v < p.nvec)
                        store_elems<XDT, VEC, NT>(p.ro, row * p.ros + (int64_t)v * VEC, hv);
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float he = MIS && e < dup[k] ? 0.0f : hv[e];
                    acc = __builtin_fmaf(he, he, acc);
                }
            }
            const float ss = row_sum(acc, p.wpr, wave_in_row, &red[it & 1][slot * p.wpr]);
            const float rs = fast_rsqrt(ss * p.inv_h + p.eps);
            if (p.rrms != nullptr && valid && t == 0) p.rrms[row] = rs;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                xr[k].opaque();
                if constexpr (RESID) rr[k].opaque();
                // the weight (and AdaLN's rows) too: widened before the
                // reduction, their float32 copies would stay live across it
                wr[k].opaque();
                if constexpr (ADALN) {
                    scr[k].opaque();
                    shr[k].opaque();
                }
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if (valid && v < p.nvec) {
                    float hv[VEC], wv[VEC], o[VEC];
                    xr[k].widen_to(hv);
                    if constexpr (RESID) {
                        float rv[VEC];
                        rr[k].widen_to(rv);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                    }
                    if constexpr (RESID && MIS) {
                        // Off the grid, the window lane's leading columns are
                        // another lane's too, possibly in another wave.  When
                        // r_out is the same buffer as x or r, a store of them
                        // made before the window lane's load returned would
                        // change what it reads.  Here every load of the row
                        // has returned (the sum of squares used each one), in
                        // every wave of the row: several waves passed the
                        // row barrier, and a one-wave row issues its stores
                        // after its own loads.
                        if (p.ro != nullptr) {
                            u32x4 raw;
#pragma unroll
                            for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(hv + q * (4 / ES));
                            store16_at<NT>(static_cast<char *>(p.ro) + (row * p.ros + col0[k]) * ES, raw);
                        }
                    }
                    wr[k].widen_to(wv);
                    if constexpr (ADALN) {
                        float sc[VEC], sh[VEC];
                        scr[k].widen_to(sc);
                        shr[k].widen_to(sh);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf((hv[e] * rs) * wv[e], 1.0f + sc[e], sh[e]);
                    } else {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) o[e] = (hv[e] * rs) * wv[e];
                    }
                    if constexpr (MIS) {
                        u32x4 raw;
#pragma unroll
                        for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(o + q * (4 / ES));
                        store16_at<NT>(static_cast<char *>(p.y) + (row * p.ys + col0[k]) * ES, raw);
                    } else {
                        store_elems<XDT, VEC, NT>(p.y, row * p.ys + (int64_t)v * VEC, o);
                    }
                }
            }
            if (it + 1 < p.iters) load_row(it + 1);
        }
    } else {
        // Rows off the grid (MIS): the row's whole vectors are read and
        // written at the row's byte offset.  Pass 1 reads a last partial
        // vector as the window over the row's last 16 bytes and leaves its
        // leading columns out of the sum; pass 2 writes while other lanes may
        // still read the row (an output can be the same buffer as an input),
        // so there that lane takes only its own columns, one at a time.
        const int chunk = row_threads * VPT;
        const int nfull = MIS ? p.H / VEC : p.nvec;  // whole vectors of a row
        // VEC parameter-format elements at element offset `off` (weight,
        // AdaLN's rows)
        auto load_param = [&](const void *base, int64_t off, float *out) {
            if constexpr (MIS) {
                Raw<WDT, VEC> r;
#pragma unroll
                for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
                    r.v[c] = load16_at<false>(static_cast<const char *>(base) + off * WES + 16 * c);
                r.widen_to(out);
            } else {
                load_elems<WDT, VEC>(base, off, out);
            }
        };
        for (int64_t it = 0; it < p.iters; ++it) {
            const int64_t row = ((int64_t)blockIdx.x + it * gstride) * p.rpw + slot;
            const bool valid = row < p.M;
            // pass 1: sum of squares, chunk by chunk
            float acc = 0.0f;
            for (int c = 0; c < p.nchunks; ++c) {
                Raw<XDT, VEC> xr[VPT];
                Raw<XDT, VEC> rr[RESID ? VPT : 1];
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (valid && v < p.nvec) {
                        // cached: pass 2 reads the same chunk again
                        if constexpr (MIS) {
                            const int col = v >= nfull ? p.H - VEC : v * VEC;
                            xr[k].v[0] = load16_at<false>(static_cast<const char *>(p.x) + (row * p.xs + col) * ES);
                            if constexpr (RESID)
                                rr[k].v[0] = load16_at<false>(static_cast<const char *>(p.r) + (row * p.rs + col) * ES);
                        } else {
                            xr[k].load(p.x, row * p.xs + (int64_t)v * VEC);
                            if constexpr (RESID) rr[k].load(p.r, row * p.rs + (int64_t)v * VEC);
                        }
                    } else {
                        xr[k].zero();
                        if constexpr (RESID) rr[k].zero();
                    }
                }
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    // the window's leading columns, another lane's
                    const int dup = MIS && v >= nfull && v < p.nvec ? v * VEC - (p.H - VEC) : 0;
                    float hv[VEC];
                    xr[k].widen_to(hv);
                    if constexpr (RESID) {
                        float rv[VEC];
                        rr[k].widen_to(rv);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                    }
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (!MIS || e >= dup) acc = __builtin_fmaf(hv[e], hv[e], acc);
                }
            }
            const float ss = row_sum(acc, p.wpr, wave_in_row, &red[it & 1][slot * p.wpr]);
            const float rs = fast_rsqrt(ss * p.inv_h + p.eps);
            if (p.rrms != nullptr && valid && t == 0) p.rrms[row] = rs;
            // pass 2: reload each chunk with the same bounds, scale, store.
            // Every element is read and then written by the same thread, so an
            // output that is the same buffer as an input is safe.
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (valid && v < nfull) {
                        float hv[VEC], wv[VEC];
                        if constexpr (MIS) {
                            Raw<XDT, VEC> xv;
                            xv.v[0] = load16_at<NT>(static_cast<const char *>(p.x) +
                                                    (row * p.xs + (int64_t)v * VEC) * ES);
                            xv.widen_to(hv);
                        } else {
                            load_elems<XDT, VEC, NT>(p.x, row * p.xs + (int64_t)v * VEC, hv);
                        }
                        if constexpr (RESID) {
                            float rv[VEC];
                            if constexpr (MIS) {
                                Raw<XDT, VEC> rw;
                                rw.v[0] = load16_at<NT>(static_cast<const char *>(p.r) +
                                                        (row * p.rs + (int64_t)v * VEC) * ES);
                                rw.widen_to(rv);
                            } else {
                                load_elems<XDT, VEC, NT>(p.r, row * p.rs + (int64_t)v * VEC, rv);
                            }
#pragma unroll
                            for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                        }
                        if (p.w != nullptr) {
                            load_param(p.w, (int64_t)v * VEC, wv);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) wv[e] = 1.0f;
                        }
                        if constexpr (RESID) {
                            if (p.ro != nullptr) {
                                if constexpr (MIS) {
                                    u32x4 raw;
#pragma unroll
                                    for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(hv + q * (4 / ES));
                                    store16_at<NT>(static_cast<char *>(p.ro) + (row * p.ros + (int64_t)v * VEC) * ES,
                                                   raw);
                                } else {
                                    store_elems<XDT, VEC, NT>(p.ro, row * p.ros + (int64_t)v * VEC, hv);
                                }
                            }
                        }
                        float o[VEC];
                        if constexpr (ADALN) {
                            const int64_t crow = row / p.rows_per_cond;
                            float sc[VEC], sh[VEC];
                            load_param(p.scale, crow * p.cs + (int64_t)v * VEC, sc);
                            load_param(p.shift, crow * p.cs + (int64_t)v * VEC, sh);
#pragma unroll
                            for (int e = 0; e < VEC; ++e)
                                o[e] = __builtin_fmaf((hv[e] * rs) * wv[e], 1.0f + sc[e], sh[e]);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) o[e] = (hv[e] * rs) * wv[e];
                        }
                        if constexpr (MIS) {
                            u32x4 raw;
#pragma unroll
                            for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(o + q * (4 / ES));
                            store16_at<NT>(static_cast<char *>(p.y) + (row * p.ys + (int64_t)v * VEC) * ES, raw);
                        } else {
                            store_elems<XDT, VEC, NT>(p.y, row * p.ys + (int64_t)v * VEC, o);
                        }
                    } else if (MIS && valid && v < p.nvec) {
                        // the last partial vector, one element at a time
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int col = v * VEC + e;
                            if (col < p.H) {
                                float h, wv = 1.0f, o;
                                load_elems<XDT, 1, NT>(p.x, row * p.xs + col, &h);
                                if constexpr (RESID) {
                                    float rv;
                                    load_elems<XDT, 1, NT>(p.r, row * p.rs + col, &rv);
                                    h = h + rv;
                                    if (p.ro != nullptr) store_elems<XDT, 1, NT>(p.ro, row * p.ros + col, &h);
                                }
                                if (p.w != nullptr) load_elems<WDT, 1>(p.w, col, &wv);
                                if constexpr (ADALN) {
                                    const int64_t crow = row / p.rows_per_cond;
                                    float sc, sh;
                                    load_elems<WDT, 1>(p.scale, crow * p.cs + col, &sc);
                                    load_elems<WDT, 1>(p.shift, crow * p.cs + col, &sh);
                                    o = __builtin_fmaf((h * rs) * wv, 1.0f + sc, sh);
                                } else {
                                    o = (h * rs) * wv;
                                }
                                store_elems<XDT, 1, NT>(p.y, row * p.ys + col, &o);
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace rmsn
