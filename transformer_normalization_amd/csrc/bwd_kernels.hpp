// bwd_kernels.hpp -- gfx950 RMSNorm backward: dx per row, dw per column.
//
// What is computed ("Skill: Write a Triton RMSNorm Kernel", "Required
// reasoning process" step 12 and "Correctness requirements"), from the saved
// per-row rrms (read, never recomputed), all in float32:
//   xn = x * rrms,  g = dy * w   (w = 1 when weightless)
//   c  = sum over the row of g * xn
//   dx = rrms * g - xn * ((c * (1/H)) * rrms)
//   dw[j] = sum over rows of dy * xn
// With RES (the backward of the fused residual pre-norm, whose forward
// writes h = x + r back as the next residual stream), x is that stored h and
// the gradient arriving on the residual stream, dres, is added before the
// single rounding: dh = dx + dres, the gradient of both x and r.
//
// Kernel 1 (rmsnorm_bwd_kernel): workgroup b owns the rows b, b+P, b+2P, ...
// (or, optionally, a contiguous block of rows) and walks them one row at a
// time with all 64*wpr threads.  The columns a thread owns are fixed (vector v = t +
// k*64*wpr), so it keeps the weight and its dw partial sums in registers for
// the whole block and, at the end, writes its float32 partials to row b of the
// workspace `partial` (P x H).  Longer rows use two passes: pass 1 forms c,
// pass 2 reloads x and dy, writes dx and adds dy*xn into the dw partial sums
// -- registers for the first chunks, the workgroup's own workspace row for
// later ones (no other workgroup touches it, so no atomics).
//
// MIS kernels take rows off the 16-byte grid (a start that is not 16-byte
// aligned, or a length that is not a whole number of vectors) in the same
// 16-byte vectors, read and written at the row's byte offset (below).
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
    const void *dres;     // RES: gradient on the residual-stream output
    void *dx;
    float *partial;      // P x H float32, or null when dw is not wanted
    int64_t dys, xs, dxs, drs;  // row strides, elements
    int64_t M;
    int64_t rows_per_wg;  // contiguous order: rows of one workgroup
    int interleave;       // 1: workgroup b owns rows b, b+P, b+2P, ...
    int frame;            // MIS, one pass: 1 = vectors on memory's 16-byte grid (below)
    int H;
    int nvec;
    int wpr;
    int nchunks;
    float inv_h;
};

// ---- rows off the 16-byte grid -----------------------------------------------
// Vector v of a row holds the row's bytes [16v, 16v + 16) and is read and
// written with one 16-byte access at the row's own byte offset: gfx9 runs
// global memory in unaligned mode, where such an access at any element-aligned
// address is one instruction.  When the row's last vector is only partly
// inside the row, its lane takes the row's last 16 bytes instead (columns
// H - VEC .. H - 1): the leading `dup` columns of that window are also the
// previous vector's; its row-sum terms take them with a weight of zero.  In
// one pass, where every load of the row has returned before any store, the
// window lane also computes and writes the same dx values for them, and its
// dw partial sums for them are not stored; two passes use the window in
// pass 1 only (see there).  No access leaves the row.
//
// With `frame` set (one pass), the host has checked that x, dy, dres and dx
// rows all sit at the same offset a within their 16-byte chunks of memory,
// the same for every row of a workgroup.  Vector v then covers the aligned
// chunk (row start - a) + 16v, i.e. columns c = (16v - a)/ES ..; the first
// vector is moved to the row start (columns 0 ..) and the last one to the
// window over the row's last 16 bytes, so that every access stays inside the
// row, and only those two are unaligned.  Each lane owns the columns of its
// chunk that lie in the row, [max(c, 0), min(c + VEC, H)); the other columns
// of its vector are also a neighbour lane's, and it leaves them out of the
// row sum and the dw partial sums exactly as the window does.  a = 0 gives
// the vectors at the row's offset above, so one code path serves both.

// DEEP: one more row in flight per wave (three prefetched instead of two), for
// one-vector tiles that leave few waves resident per CU (the host's rule).
template <int XDT, int WDT, int VEC, int VPT, bool RES, bool TWO_PASS, bool NT, int MAXT, bool MIS = false,
          bool DEEP = false>
__global__ void __launch_bounds__(MAXT) rmsnorm_bwd_kernel(const BwdParams p) {
    static_assert(!MIS || VEC * Fmt<XDT>::bytes == 16, "rows off the grid: 16-byte vector tiles");
    static_assert(!DEEP || (!TWO_PASS && VPT == 1 && VEC > 1), "deeper prefetch: one-vector resident tiles");
    // (rows off the grid: at least 16 bytes long, so that the last 16 bytes lie inside the row)
    __shared__ float red[2][16];
    const int row_threads = 64 * p.wpr;  // == blockDim.x
    const int t = threadIdx.x;
    const int wave = t >> 6;
    // The workgroup's rows are start + j*step for j = 0 .. nsteps-1: either a
    // contiguous block, or interleaved with the other workgroups so that the
    // rows in flight across the GPU at any moment are neighbours in memory.
    int64_t start, step, nsteps;
    if (p.interleave) {
        start = blockIdx.x;
        step = gridDim.x;
        nsteps = (p.M - start + step - 1) / step;
    } else {
        start = (int64_t)blockIdx.x * p.rows_per_wg;
        step = 1;
        nsteps = start + p.rows_per_wg < p.M ? p.rows_per_wg : p.M - start;
    }
    float *part = p.partial != nullptr ? p.partial + (int64_t)blockIdx.x * p.H : nullptr;

    if constexpr (!TWO_PASS) {
        // x, dy and w stay packed in registers and are widened at each use;
        // only the dw partial sums are float32 registers.
        Raw<WDT, VEC> wr[VPT];
        float dwa[VPT][VEC];
        // rows off the grid: the rows' offset a in the 16-byte frame (0
        // without `frame`) and the vectors a row takes
        int fa = 0, nact = p.nvec;
        if constexpr (MIS) {
            if (p.frame)
                fa = (int)((reinterpret_cast<uintptr_t>(p.x) + (uint64_t)start * (uint64_t)p.xs * Fmt<XDT>::bytes) &
                           15u);
            nact = (fa + p.H * Fmt<XDT>::bytes + 15) >> 4;
        }
        // rows off the grid: first column of the thread's vector; own(k)
        // gives the columns [lo, hi) of it that the thread owns (recomputed
        // where needed rather than held across the row loop)
        int col0[VPT];
        auto own = [&](int k, int &lo, int &hi) {
            if constexpr (MIS) {
                const int c = (16 * (t + k * row_threads) - fa) / Fmt<XDT>::bytes;  // negative: the first chunk
                lo = (c < 0 ? 0 : c) - col0[k];
                hi = (c + VEC < p.H ? c + VEC : p.H) - col0[k];
            } else {
                lo = 0;
                hi = VEC;
            }
        };
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = t + k * row_threads;
            if constexpr (MIS) {
                const int c = (16 * v - fa) / Fmt<XDT>::bytes;
                col0[k] = c < 0 ? 0 : c > p.H - VEC ? p.H - VEC : c;
            } else {
                col0[k] = v * VEC;
            }
            if (p.w != nullptr && v < nact) {
                if constexpr (MIS) {
                    constexpr int WES = Fmt<WDT>::bytes;
#pragma unroll
                    for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
                        wr[k].v[c] = load16_at<false>(static_cast<const char *>(p.w) + (int64_t)col0[k] * WES + 16 * c);
                } else {
                    wr[k].load(p.w, (int64_t)v * VEC);
                }
            } else {
                wr[k].fill_one();
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) dwa[k][e] = 0.0f;
        }
        // the weights of the row-sum terms: w, with the window's leading
        // columns zeroed off the grid (fma(0, y, part) == part)
        Raw<WDT, VEC> wsum[MIS ? VPT : 1];
        if constexpr (MIS) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                constexpr int PER_WORD = 4 / Fmt<WDT>::bytes;
                float f[VEC];
                wr[k].widen_to(f);
                int lo, hi;
                own(k, lo, hi);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (e < lo || e >= hi) f[e] = 0.0f;
#pragma unroll
                for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
#pragma unroll
                    for (int q = 0; q < 4; ++q) wsum[k].v[c][q] = pack_word<WDT>(f + (c * 4 + q) * PER_WORD);
            }
        }
        // Software pipeline: the loads of rows row+1 .. row+PF are in flight
        // while row is reduced and stored (the barrier in row_sum waits on
        // LDS only).  The rows' saved rrms values are read 64 at a time, one
        // per lane, and taken with v_readlane, so that no vector load inside
        // the loop makes the in-order memory counter wait for the prefetch.
        // depth 2 for small tiles, 1 where three rows would not fit the
        // register budget (32-bit words holding x, dy and dres of one row),
        // 3 with DEEP
        constexpr int WORDS = (RES ? 3 : 2) * VPT * (int)(sizeof(Raw<XDT, VEC>) / 4);
        constexpr int PF = DEEP ? 3 : WORDS <= 16 ? 2 : 1;
        Raw<XDT, VEC> xb[PF + 1][VPT], db[PF + 1][VPT], gb[RES ? PF + 1 : 1][VPT];
        constexpr int ES = Fmt<XDT>::bytes;
        const int lane = t & 63;
        // rows in chunks of 64: one rrms value per lane for the chunk, loaded
        // before the chunk's row loads so that no wait inside the row loop
        // depends on a load issued after a prefetch
        for (int64_t base = 0; base < nsteps; base += 64) {
            const int64_t cend = base + 64 < nsteps ? base + 64 : nsteps;
            float rr_lane = (base + lane < cend) ? p.rrms[start + (base + lane) * step] : 0.0f;
            asm volatile("" : "+v"(rr_lane));  // complete it now, before the row loads
            // Row loads inside the steady-state loop are unconditional, so the
            // compiler can count them in order and wait only for the oldest;
            // vector indices past the row are clamped to its last vector
            // (same addresses within one wave access: no extra traffic) and
            // masked at use.
            auto load_row = [&](int64_t j, Raw<XDT, VEC> *xd, Raw<XDT, VEC> *dd, Raw<XDT, VEC> *gd) {
                const int64_t row = start + j * step;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int vv = t + k * row_threads;
                    const int v = vv < nact ? vv : nact - 1;
                    if constexpr (MIS) {
                        const int64_t o = (int64_t)(vv < nact ? col0[k] : p.H - VEC) * ES;
                        xd[k].v[0] = load16_at<NT>(static_cast<const char *>(p.x) + row * p.xs * ES + o);
                        dd[k].v[0] = load16_at<NT>(static_cast<const char *>(p.dy) + row * p.dys * ES + o);
                        if constexpr (RES)
                            gd[k].v[0] = load16_at<NT>(static_cast<const char *>(p.dres) + row * p.drs * ES + o);
                    } else {
                        xd[k].template load<NT>(p.x, row * p.xs + (int64_t)v * VEC);
                        dd[k].template load<NT>(p.dy, row * p.dys + (int64_t)v * VEC);
                        if constexpr (RES) gd[k].template load<NT>(p.dres, row * p.drs + (int64_t)v * VEC);
                    }
                }
            };
            auto process_row = [&](int64_t j, Raw<XDT, VEC> *xr, Raw<XDT, VEC> *dr, Raw<XDT, VEC> *gr) {
                const int64_t row = start + j * step;
                const float rs = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rr_lane), (int)(j - base)));
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    float xv[VEC], dv[VEC], wv[VEC];
                    xr[k].widen_to(xv);
                    dr[k].widen_to(dv);
                    if constexpr (MIS)
                        wsum[k].widen_to(wv);
                    else
                        wr[k].widen_to(wv);
                    float part = 0.0f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) part = __builtin_fmaf(dv[e] * wv[e], xv[e] * rs, part);
                    if (t + k * row_threads < nact) acc += part;
                }
                // Off the grid, the window lane's leading columns are another
                // lane's too, possibly in another wave, and dh may be the same
                // buffer as dres.  x and dy have returned here (the row sum
                // used them), but nothing else waits for dres before another
                // wave stores over it: take it now, so that every load of the
                // row has returned, in every wave, before any store of dh.
                if constexpr (MIS && RES) {
#pragma unroll
                    for (int k = 0; k < VPT; ++k) gr[k].opaque();
                }
                const float c = row_sum(acc, p.wpr, wave, &red[j & 1][0]);
                const float s = (c * p.inv_h) * rs;
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    xr[k].opaque();
                    dr[k].opaque();
                    if constexpr (RES) gr[k].opaque();
                }
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = t + k * row_threads;
                    float xv[VEC], dv[VEC], wv[VEC], o[VEC];
                    xr[k].widen_to(xv);
                    dr[k].widen_to(dv);
                    wr[k].widen_to(wv);
                    if (v < nact) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const float xn = xv[e] * rs;
                            o[e] = rs * (dv[e] * wv[e]) - xn * s;
                            dwa[k][e] = __builtin_fmaf(dv[e], xn, dwa[k][e]);
                        }
                        if constexpr (RES) {
                            float gv[VEC];
                            gr[k].widen_to(gv);
#pragma unroll
                            for (int e = 0; e < VEC; ++e) o[e] += gv[e];
                        }
                        if constexpr (MIS) {
                            u32x4 raw;
#pragma unroll
                            for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(o + q * (4 / ES));
                            store16_at<NT>(static_cast<char *>(p.dx) + (row * p.dxs + col0[k]) * ES, raw);
                        } else
                            store_elems<XDT, VEC, NT>(p.dx, row * p.dxs + (int64_t)v * VEC, o);
                    }
                }
            };
            // prologue: unconditional too (a chunk shorter than PF rows reads
            // its last row again rather than branching)
#pragma unroll
            for (int j = 0; j < PF; ++j) load_row(base + j < cend ? base + j : cend - 1, xb[j], db[j], gb[RES ? j : 0]);
            // Steady state, unrolled by PF+1 so that row r always lives in
            // slot (r - base) % (PF+1) (copying registers whose loads are in
            // flight would wait for them).  It runs while every prefetched row
            // exists, so its loads need no condition.
            int64_t row = base;  // step index
            for (; row + 2 * PF < cend; row += PF + 1) {
#pragma unroll
                for (int u = 0; u <= PF; ++u) {
                    load_row(row + u + PF, xb[(u + PF) % (PF + 1)], db[(u + PF) % (PF + 1)],
                             gb[RES ? (u + PF) % (PF + 1) : 0]);
                    process_row(row + u, xb[u], db[u], gb[RES ? u : 0]);
                }
            }
            // the last rows (at most 2*PF), with conditional prefetch
#pragma unroll
            for (int u = 0; u < 2 * PF; ++u) {
                if (row + u < cend) {
                    if (row + u + PF < cend)
                        load_row(row + u + PF, xb[(u + PF) % (PF + 1)], db[(u + PF) % (PF + 1)],
                                 gb[RES ? (u + PF) % (PF + 1) : 0]);
                    process_row(row + u, xb[u % (PF + 1)], db[u % (PF + 1)], gb[RES ? u % (PF + 1) : 0]);
                }
            }
        }
        if (part != nullptr) {
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if constexpr (MIS) {
                    // the workspace rows are H floats apart, so off the grid too
                    int lo, hi;
                    own(k, lo, hi);
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (v < nact && e >= lo && e < hi) part[(int64_t)col0[k] + e] = dwa[k][e];
                } else {
                    if (v < p.nvec) store_elems<DT_F32, VEC>(part, (int64_t)v * VEC, dwa[k]);
                }
            }
        }
    } else {
        const int chunk = row_threads * VPT;
        // The dw partial sums of the first RCH chunks stay in registers
        // across the workgroup's rows and are stored once (64 floats per
        // thread: eight chunks of single elements, four of float32 vectors,
        // two of 16-bit vectors -- rows up to 65536 elements; 78-110 VGPRs
        // at 1024 threads, no spills); the sums of later chunks are added
        // into the workgroup's workspace row at each row.  Either way each
        // column adds its rows in row order, so dw has the same bits.
        //
        // Rows off the grid (MIS): the row's whole vectors are read and
        // written at the row's byte offset.  A last partial vector (the
        // row's last H mod VEC columns) is read in pass 1 as the window over
        // the row's last 16 bytes, its leading columns left out of the sum;
        // in pass 2 its lane takes only its own columns, one element at a
        // time.  Pass 2 writes dx while other lanes still read the row, and
        // later chunks read-modify-write the workspace row, so there no two
        // lanes may touch the same column.
        constexpr int RCH = 64 / (VPT * VEC) > 0 ? 64 / (VPT * VEC) : 1;
        constexpr int ES = Fmt<XDT>::bytes;
        constexpr int WES = Fmt<WDT>::bytes;
        const int nfull = MIS ? p.H / VEC : p.nvec;  // whole vectors of a row
        float dwr[RCH > 0 ? RCH : 1][VPT][VEC];
#pragma unroll
        for (int c = 0; c < (RCH > 0 ? RCH : 1); ++c)
#pragma unroll
            for (int k = 0; k < VPT; ++k)
#pragma unroll
                for (int e = 0; e < VEC; ++e) dwr[c][k][e] = 0.0f;
        // VEC float32 partial sums of vector v in the workspace row; off the
        // grid the row is only 4-byte aligned (rows H floats apart), and the
        // last partial vector holds H - v*VEC of them
        auto part_load = [&](int v, float *pa) {
            if constexpr (MIS) {
                if (v < nfull) {
#pragma unroll
                    for (int c = 0; c < VEC / 4; ++c) {
                        const u32x4 r =
                            load16_at<false>(reinterpret_cast<const char *>(part + (int64_t)v * VEC + 4 * c));
#pragma unroll
                        for (int q = 0; q < 4; ++q) pa[4 * c + q] = __builtin_bit_cast(float, r[q]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) pa[e] = v * VEC + e < p.H ? part[(int64_t)v * VEC + e] : 0.0f;
                }
            } else {
                load_elems<DT_F32, VEC>(part, (int64_t)v * VEC, pa);
            }
        };
        auto part_store = [&](int v, const float *pa) {
            if constexpr (MIS) {
                if (v < nfull) {
#pragma unroll
                    for (int c = 0; c < VEC / 4; ++c) {
                        u32x4 r;
#pragma unroll
                        for (int q = 0; q < 4; ++q) r[q] = __builtin_bit_cast(uint32_t, pa[4 * c + q]);
                        store16_at<false>(reinterpret_cast<char *>(part + (int64_t)v * VEC + 4 * c), r);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (v * VEC + e < p.H) part[(int64_t)v * VEC + e] = pa[e];
                }
            } else {
                store_elems<DT_F32, VEC>(part, (int64_t)v * VEC, pa);
            }
        };
        if (part != nullptr) {
            const float z[VEC] = {};
            for (int v = RCH * chunk + t; v < p.nvec; v += row_threads) part_store(v, z);
        }
        // the VEC weights of vector v starting at column col (1 when weightless)
        auto load_w = [&](int col, float *wv) {
            if (p.w != nullptr) {
                if constexpr (MIS) {
                    Raw<WDT, VEC> wr;
#pragma unroll
                    for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
                        wr.v[c] = load16_at<false>(static_cast<const char *>(p.w) + (int64_t)col * WES + 16 * c);
                    wr.widen_to(wv);
                } else {
                    load_elems<WDT, VEC>(p.w, col, wv);
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) wv[e] = 1.0f;
            }
        };
        // VEC elements of a row at column col, off the grid at the row's byte offset
        auto load_vec = [&](const void *base, int64_t rowoff, int col, float *out, auto nt) {
            constexpr bool NTL = decltype(nt)::value;
            if constexpr (MIS) {
                Raw<XDT, VEC> r;
                r.v[0] = load16_at<NTL>(static_cast<const char *>(base) + (rowoff + col) * ES);
                r.widen_to(out);
            } else {
                load_elems<XDT, VEC, NTL>(base, rowoff + col, out);
            }
        };
        using Cached = std::false_type;
        using Stream = std::integral_constant<bool, NT>;
        int parity = 0;
        for (int64_t j = 0; j < nsteps; ++j, parity ^= 1) {
            const int64_t row = start + j * step;
            const float rs = p.rrms[row];
            // the column offsets are recomputed in every row from an opaque
            // copy of t: hoisted out of the row loop, those of all the
            // unrolled chunks would stay live (over 100 VGPRs)
            int tc = t;
            asm volatile("" : "+v"(tc));
            float acc = 0.0f;
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + tc + k * row_threads;
                    if (v < p.nvec) {
                        // the last partial vector: the window over the row's
                        // last VEC columns, whose first `dup` are another lane's
                        const int col = MIS && v >= nfull ? p.H - VEC : v * VEC;
                        const int dup = v * VEC - col;
                        float xv[VEC], dv[VEC], wv[VEC];
                        // cached: pass 2 reads the same chunk again
                        load_vec(p.x, row * p.xs, col, xv, Cached{});
                        load_vec(p.dy, row * p.dys, col, dv, Cached{});
                        load_w(col, wv);
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            if (!MIS || e >= dup) acc = __builtin_fmaf(dv[e] * wv[e], xv[e] * rs, acc);
                    }
                }
            }
            const float cs = row_sum(acc, p.wpr, wave, &red[parity][0]);
            const float s = (cs * p.inv_h) * rs;
            // pass 2 over chunk c; dw_add(k, v, dv, xn) receives dy * xn
            // (zero in the columns past the row's end)
            auto pass2 = [&](int c, auto &&dw_add) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + tc + k * row_threads;
                    if (v < nfull) {
                        float xv[VEC], dv[VEC], wv[VEC], o[VEC];
                        load_vec(p.x, row * p.xs, v * VEC, xv, Stream{});
                        load_vec(p.dy, row * p.dys, v * VEC, dv, Stream{});
                        load_w(v * VEC, wv);
                        float xn[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            xn[e] = xv[e] * rs;
                            o[e] = rs * (dv[e] * wv[e]) - xn[e] * s;
                        }
                        if constexpr (RES) {
                            float gv[VEC];
                            load_vec(p.dres, row * p.drs, v * VEC, gv, Stream{});
#pragma unroll
                            for (int e = 0; e < VEC; ++e) o[e] += gv[e];
                        }
                        if constexpr (MIS) {
                            u32x4 raw;
#pragma unroll
                            for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(o + q * (4 / ES));
                            store16_at<NT>(static_cast<char *>(p.dx) + (row * p.dxs + (int64_t)v * VEC) * ES, raw);
                        } else {
                            store_elems<XDT, VEC, NT>(p.dx, row * p.dxs + (int64_t)v * VEC, o);
                        }
                        dw_add(k, v, dv, xn);
                    } else if (MIS && v < p.nvec) {
                        // the last partial vector, one element at a time
                        float dv[VEC], xn[VEC];
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const int col = v * VEC + e;
                            dv[e] = 0.0f;
                            xn[e] = 0.0f;
                            if (col < p.H) {
                                float xv, wv = 1.0f, o;
                                load_elems<XDT, 1, NT>(p.x, row * p.xs + col, &xv);
                                load_elems<XDT, 1, NT>(p.dy, row * p.dys + col, &dv[e]);
                                if (p.w != nullptr) load_elems<WDT, 1>(p.w, col, &wv);
                                xn[e] = xv * rs;
                                o = rs * (dv[e] * wv) - xn[e] * s;
                                if constexpr (RES) {
                                    float gv;
                                    load_elems<XDT, 1, NT>(p.dres, row * p.drs + col, &gv);
                                    o += gv;
                                }
                                store_elems<XDT, 1, NT>(p.dx, row * p.dxs + col, &o);
                            }
                        }
                        dw_add(k, v, dv, xn);
                    }
                }
            };
#pragma unroll
            for (int c = 0; c < RCH; ++c) {
                if (c < p.nchunks)
                    pass2(c, [&](int k, int, const float *dv, const float *xn) {
#pragma unroll
                        for (int e = 0; e < VEC; ++e) dwr[c][k][e] = __builtin_fmaf(dv[e], xn[e], dwr[c][k][e]);
                    });
                // one chunk's loads at a time: interleaving the unrolled
                // chunks would hold all of their elements at once
                __builtin_amdgcn_sched_barrier(0);
            }
            for (int c = RCH; c < p.nchunks; ++c)
                pass2(c, [&](int, int v, const float *dv, const float *xn) {
                    if (part != nullptr) {
                        float pa[VEC];
                        part_load(v, pa);
#pragma unroll
                        for (int e = 0; e < VEC; ++e) pa[e] = __builtin_fmaf(dv[e], xn[e], pa[e]);
                        part_store(v, pa);
                    }
                });
        }
        if (part != nullptr) {
#pragma unroll
            for (int c = 0; c < RCH; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (c < p.nchunks && v < p.nvec) part_store(v, dwr[c][k]);
                }
            }
        }
    }
}

// dw[j] = sum over p of partial[p][j]: 32 columns x 16 slices per workgroup
// of 512 threads (a wave reads 128 contiguous bytes from each of two partial
// rows).  Thread (col, s) sums p = s, s+16, ... in increasing p, loading 16
// at a time before adding; the 16 slice sums of a column are then added in
// slice order.  The order is fixed, so dw has the same bits on every run
// (and for any columns-per-workgroup or batch: measured on gfx950, 32 x 16
// with batches of 16 took about 1 us less than 64 x 16 with batches of 8 at
// H <= 2048, the same at H = 6144 and 8192).
constexpr int kFinCols = 32;
constexpr int kFinSlices = 16;
constexpr int kFinBatch = 16;  // partial rows loaded per thread before they are added
// (defined in kernels_bwd.hip)

}  // namespace rmsn
