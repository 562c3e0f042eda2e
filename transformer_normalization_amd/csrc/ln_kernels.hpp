// ln_kernels.hpp -- gfx950 LayerNorm forward, plain and fused with the
// residual add that precedes it in a pre-LayerNorm transformer block (the
// page "SpeedROCm: shape-aware Triton acceleration for Transformer
// inference", "How the solution addresses the problem", item 4).
//
// What is computed, all in float32 (torch.nn's LayerNorm semantics):
//   h     = x, or float32(x) + float32(r) with r_out = RNE(h)
//   mean  = sum(h) * (1/H)
//   var   = sum((h - mean)^2) * (1/H)      (population variance, centred)
//   rstd  = rsqrt(var + eps)
//   y     = fma((h - mean) * rstd, w, b)    (w = 1, b = 0 when absent)
//
// The variance is taken about the computed mean in a second reduction, never
// as mean(h^2) - mean^2, which cancels when |mean| >> std.
//
// Work layout as the RMSNorm forward (fwd_kernels.hpp): row groups of wpr
// waves own a row at a time, rpw row groups per workgroup, grid-stride over
// the rows with a uniform trip count; thread t owns the vectors t, t +
// 64*wpr, ... of the row; weight and bias stay packed in registers.
//   * Resident path: the row (and the residual) stays packed in registers
//     for both reductions and the output -- one HBM read per input element
//     and one write per output element.
//   * Long rows: pass 1 sums h, pass 2 sums (h - mean)^2, pass 3 writes y
//     (and r_out); passes 1 and 2 use cached loads.
#pragma once

#include "numerics.hpp"

namespace rmsn {

struct LnParams {
    const void *x;
    const void *r;    // residual (fused form only)
    const void *w;    // may be null
    const void *b;    // may be null
    void *y;
    void *ro;         // residual_out, may be null
    float *mean;      // may be null
    float *rstd;      // may be null
    int64_t xs, rs, ys, ros;  // row strides, elements
    int64_t M;
    int64_t iters;    // row-group iterations per workgroup
    int H;
    int nvec;
    int wpr;
    int rpw;
    int nchunks;
    float eps;
    float inv_h;
};

// MIS: rows off the 16-byte grid in the same 16-byte vectors, each read and
// written with one access at the row's own byte offset; a row's last vector,
// when only partly inside the row, is the window over the row's last 16
// bytes, whose leading `dup` columns (the previous vector's) are left out of
// both sums.  Resident, the window lane writes them again with the same
// values after the reductions; on long rows it writes only its own columns,
// one at a time (fwd_kernels.hpp).
template <int XDT, int WDT, int VEC, int VPT, bool RESID, bool TWO_PASS, bool NT, int MAXT, bool MIS = false>
__global__ void __launch_bounds__(MAXT) layernorm_fwd_kernel(const LnParams p) {
    static_assert(!MIS || VEC * Fmt<XDT>::bytes == 16, "rows off the grid: 16-byte vector tiles");
    constexpr int ES = Fmt<XDT>::bytes;
    constexpr int WES = Fmt<WDT>::bytes;
    // one LDS area per reduction of a row; consecutive reductions alternate
    // areas, so one barrier per reduction suffices (see row_sum)
    __shared__ float red[2][16];
    const int row_threads = 64 * p.wpr;
    const int slot = threadIdx.x / row_threads;
    const int t = threadIdx.x - slot * row_threads;
    const int wave_in_row = t >> 6;
    const int64_t gstride = (int64_t)gridDim.x;

    if constexpr (!TWO_PASS) {
        Raw<WDT, VEC> wr[VPT], br[VPT];
        int col0[VPT], dup[VPT];
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int v = t + k * row_threads;
            col0[k] = MIS && v * VEC > p.H - VEC ? p.H - VEC : v * VEC;
            dup[k] = MIS ? v * VEC - col0[k] : 0;
            if constexpr (MIS) {
#pragma unroll
                for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c) {
                    const int64_t o = (int64_t)col0[k] * WES + 16 * c;
                    wr[k].v[c] = p.w != nullptr && v < p.nvec ? load16_at<false>(static_cast<const char *>(p.w) + o)
                                                               : u32x4{0u, 0u, 0u, 0u};
                    br[k].v[c] = p.b != nullptr && v < p.nvec ? load16_at<false>(static_cast<const char *>(p.b) + o)
                                                               : u32x4{0u, 0u, 0u, 0u};
                }
                if (p.w == nullptr || v >= p.nvec) wr[k].fill_one();
            } else {
                if (p.w != nullptr && v < p.nvec)
                    wr[k].load(p.w, (int64_t)v * VEC);
                else
                    wr[k].fill_one();
                if (p.b != nullptr && v < p.nvec)
                    br[k].load(p.b, (int64_t)v * VEC);
                else
                    br[k].zero();
            }
        }
        // a row's loads are issued before the loop (first row) or at the end
        // of the previous iteration, never behind a wait: the weight and bias
        // would otherwise be waited for in the loop's preheader, ahead of the
        // first row's loads (two memory latencies in a row)
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
        };
        // 16 bytes of float32 values, in x's format, written at column col0[k]
        auto store_window = [&](void *base, int64_t row_off, int k, const float *vals) {
            u32x4 raw;
#pragma unroll
            for (int q = 0; q < 4; ++q) raw[q] = pack_word<XDT>(vals + q * (4 / ES));
            store16_at<NT>(static_cast<char *>(base) + (row_off + col0[k]) * ES, raw);
        };
        load_row(0);
        for (int64_t it = 0; it < p.iters; ++it) {
            const int64_t row = ((int64_t)blockIdx.x + it * gstride) * p.rpw + slot;
            const bool valid = row < p.M;
            // h of vector k, widened (and summed with the residual) again at
            // each use; every widening gives the same floats
            auto widen_h = [&](int k, float *hv) {
                xr[k].widen_to(hv);
                if constexpr (RESID) {
                    float rv[VEC];
                    rr[k].widen_to(rv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                }
            };
            float s1 = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                float hv[VEC];
                widen_h(k, hv);
                // Aligned rows: each element is read and written by one
                // thread, so r_out may go out now.  Off the grid it waits for
                // the row's reductions (below).
                if constexpr (RESID && !MIS) {
                    const int v = t + k * row_threads;
                    if (p.ro != nullptr && valid && v < p.nvec)
                        store_elems<XDT, VEC, NT>(p.ro, row * p.ros + (int64_t)v * VEC, hv);
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) s1 += MIS && e < dup[k] ? 0.0f : hv[e];
            }
            const float mean = row_sum(s1, p.wpr, wave_in_row, &red[0][slot * p.wpr]) * p.inv_h;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                xr[k].opaque();
                if constexpr (RESID) rr[k].opaque();
            }
            float s2 = 0.0f;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                float hv[VEC];
                widen_h(k, hv);
                if (v < p.nvec) {  // padding lanes hold h = 0, not mean
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const float d = MIS && e < dup[k] ? 0.0f : hv[e] - mean;
                        s2 = __builtin_fmaf(d, d, s2);
                    }
                }
            }
            const float var = row_sum(s2, p.wpr, wave_in_row, &red[1][slot * p.wpr]) * p.inv_h;
            const float rs = fast_rsqrt(var + p.eps);
            if (valid && t == 0) {
                if (p.mean != nullptr) p.mean[row] = mean;
                if (p.rstd != nullptr) p.rstd[row] = rs;
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                xr[k].opaque();
                if constexpr (RESID) rr[k].opaque();
                // weight and bias too: widened early, their float32 copies
                // would stay live across both reductions
                wr[k].opaque();
                br[k].opaque();
            }
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const int v = t + k * row_threads;
                if (valid && v < p.nvec) {
                    float hv[VEC], wv[VEC], bv[VEC], o[VEC];
                    widen_h(k, hv);
                    // Off the grid, the window lane's leading columns are
                    // another lane's too, possibly in another wave; r_out may
                    // be the same buffer as x or r.  Every load of the row has
                    // returned here (both sums used each one), in every wave
                    // of the row, so this store cannot change what any lane
                    // reads.
                    if constexpr (RESID && MIS) {
                        if (p.ro != nullptr) store_window(p.ro, row * p.ros, k, hv);
                    }
                    wr[k].widen_to(wv);
                    br[k].widen_to(bv);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf((hv[e] - mean) * rs, wv[e], bv[e]);
                    if constexpr (MIS)
                        store_window(p.y, row * p.ys, k, o);
                    else
                        store_elems<XDT, VEC, NT>(p.y, row * p.ys + (int64_t)v * VEC, o);
                }
            }
            if (it + 1 < p.iters) load_row(it + 1);
        }
    } else {
        // Rows off the grid (MIS): whole vectors at the row's byte offset;
        // a last partial vector is the window over the row's last 16 bytes
        // in the two reduction passes (its leading columns left out of both
        // sums) and, in pass 3, which writes while other lanes may still read
        // the row, only its own columns, one at a time.
        const int chunk = row_threads * VPT;
        const int nfull = MIS ? p.H / VEC : p.nvec;  // whole vectors of a row
        auto load_param = [&](const void *base, int v, float *out) {
            if constexpr (MIS) {
                Raw<WDT, VEC> r;
#pragma unroll
                for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c)
                    r.v[c] = load16_at<false>(static_cast<const char *>(base) + (int64_t)v * VEC * WES + 16 * c);
                r.widen_to(out);
            } else {
                load_elems<WDT, VEC>(base, (int64_t)v * VEC, out);
            }
        };
        for (int64_t it = 0; it < p.iters; ++it) {
            const int64_t row = ((int64_t)blockIdx.x + it * gstride) * p.rpw + slot;
            const bool valid = row < p.M;
            // h of the VEC columns from col (cached loads for the two
            // reduction passes)
            auto load_h = [&](int col, float *hv, auto nt_tag) {
                constexpr bool LNT = decltype(nt_tag)::value;
                if constexpr (MIS) {
                    Raw<XDT, VEC> xr;
                    xr.v[0] = load16_at<LNT>(static_cast<const char *>(p.x) + (row * p.xs + col) * ES);
                    xr.widen_to(hv);
                } else {
                    load_elems<XDT, VEC, LNT>(p.x, row * p.xs + col, hv);
                }
                if constexpr (RESID) {
                    float rv[VEC];
                    if constexpr (MIS) {
                        Raw<XDT, VEC> rr;
                        rr.v[0] = load16_at<LNT>(static_cast<const char *>(p.r) + (row * p.rs + col) * ES);
                        rr.widen_to(rv);
                    } else {
                        load_elems<XDT, VEC, LNT>(p.r, row * p.rs + col, rv);
                    }
#pragma unroll
                    for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                }
            };
            // the first column a reduction pass reads for vector v, and how
            // many of its leading columns are another lane's
            auto window = [&](int v, int *dup) {
                const int col = MIS && v >= nfull ? p.H - VEC : v * VEC;
                *dup = v * VEC - col;
                return col;
            };
            using cached = std::integral_constant<bool, false>;
            using streamed = std::integral_constant<bool, NT>;
            // pass 1: sum of h
            float s1 = 0.0f;
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (valid && v < p.nvec) {
                        int dup;
                        const int col = window(v, &dup);
                        float hv[VEC];
                        load_h(col, hv, cached{});
#pragma unroll
                        for (int e = 0; e < VEC; ++e)
                            if (!MIS || e >= dup) s1 += hv[e];
                    }
                }
            }
            const float mean = row_sum(s1, p.wpr, wave_in_row, &red[0][slot * p.wpr]) * p.inv_h;
            // pass 2: sum of (h - mean)^2
            float s2 = 0.0f;
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (valid && v < p.nvec) {
                        int dup;
                        const int col = window(v, &dup);
                        float hv[VEC];
                        load_h(col, hv, cached{});
#pragma unroll
                        for (int e = 0; e < VEC; ++e) {
                            const float d = hv[e] - mean;
                            if (!MIS || e >= dup) s2 = __builtin_fmaf(d, d, s2);
                        }
                    }
                }
            }
            const float var = row_sum(s2, p.wpr, wave_in_row, &red[1][slot * p.wpr]) * p.inv_h;
            const float rs = fast_rsqrt(var + p.eps);
            if (valid && t == 0) {
                if (p.mean != nullptr) p.mean[row] = mean;
                if (p.rstd != nullptr) p.rstd[row] = rs;
            }
            // pass 3: reload, normalise, store (each element is read and
            // written by the same thread, so in-place outputs are safe)
            for (int c = 0; c < p.nchunks; ++c) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    const int v = c * chunk + t + k * row_threads;
                    if (valid && v < nfull) {
                        float hv[VEC], wv[VEC], bv[VEC], o[VEC];
                        load_h(v * VEC, hv, streamed{});
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
                        if (p.w != nullptr) {
                            load_param(p.w, v, wv);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) wv[e] = 1.0f;
                        }
                        if (p.b != nullptr) {
                            load_param(p.b, v, bv);
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e) bv[e] = 0.0f;
                        }
#pragma unroll
                        for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf((hv[e] - mean) * rs, wv[e], bv[e]);
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
                                float h, wv = 1.0f, bv = 0.0f, o;
                                load_elems<XDT, 1, NT>(p.x, row * p.xs + col, &h);
                                if constexpr (RESID) {
                                    float rv;
                                    load_elems<XDT, 1, NT>(p.r, row * p.rs + col, &rv);
                                    h = h + rv;
                                    if (p.ro != nullptr) store_elems<XDT, 1, NT>(p.ro, row * p.ros + col, &h);
                                }
                                if (p.w != nullptr) load_elems<WDT, 1>(p.w, col, &wv);
                                if (p.b != nullptr) load_elems<WDT, 1>(p.b, col, &bv);
                                o = __builtin_fmaf((h - mean) * rs, wv, bv);
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
