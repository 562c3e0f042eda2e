// staged_kernels.hpp -- gfx950 forward RMSNorm and LayerNorm (plain and
// fused residual) for rows that are not 16-byte aligned: H not a whole number
// of 16-byte vectors, or a base or row stride off the 16-byte grid.
//
// What is computed is exactly the forward of fwd_kernels.hpp (and of
// ln_kernels.hpp for LayerNorm), resident tile: the same float32 expressions
// in the same order ("Skill: Write a Triton RMSNorm Kernel", "Required
// reasoning process" steps 1-11; LayerNorm: "SpeedROCm: shape-aware Triton
// acceleration for Transformer inference", "How the solution addresses the
// problem", item 4).  Only the movement of the data differs:
//   * A row group of 64*wpr threads owns one row; a workgroup holds rpw row
//     groups, each with its own LDS buffers, and handles rpw consecutive
//     rows.  There is no loop over rows: straight-line code keeps few
//     registers live, and the host splits a call of more than 2^31 - 1
//     workgroups into launches.
//   * Each input row (x, and the residual) is copied into LDS as the aligned
//     16-byte blocks that hold its bytes -- every block loaded holds at least
//     one byte of the row, so no load leaves the row's pages -- and the row's
//     byte i then sits at LDS byte delta + i, delta being the row's offset in
//     its first block.
//   * Thread t takes the same column vectors as on the aligned path (VEC
//     elements each: vectors t, t + 64*wpr, ...), read from LDS as five
//     aligned dwords joined with v_alignbyte.  The sum of squares follows the
//     aligned path's tree for the tile; the tile depends on H only, so any
//     two layouts of the same rows (offsets, row pitches) give the same bits.
//     Elements past H count as 0, as the aligned path's padding vectors do.
//   * A thread holds its packed vectors (and the weight) in registers from
//     the sum to the outputs, as the aligned path does.  Each thread writes
//     its outputs over its own input bytes in LDS, then the output row is
//     copied out: every aligned 16-byte block lying wholly inside it with one
//     16-byte store (its bytes joined from LDS as above), and the at most two
//     blocks it shares with its neighbours element by element, so nothing
//     outside the row is written.
//   * The weight (16-byte aligned) is read as column vectors; a 16-byte chunk
//     is loaded only if it holds an element below H, so the load stays inside
//     the weight's pages.
#pragma once

#include "fwd_kernels.hpp"
#include "ln_kernels.hpp"

namespace rmsn {

// Bytes of one staging buffer for rows of nvec column vectors: the row's
// bytes start at delta < 16 and end before 16 * (nvec + 1); every LDS read
// (five dwords from a 4-byte boundary at or below a row byte) ends before
// 16 * (nvec + 2).
__host__ __device__ constexpr int64_t staged_buffer_bytes(int64_t nvec) { return 16 * (nvec + 2); }
// LDS the staged kernels may use per workgroup (rpw row groups, one buffer
// each for the plain form, two for the fused residual)
constexpr int64_t kStagedMaxLds = 60 * 1024;

// 16 bytes at LDS byte offset `off` (any alignment): the five aligned dwords
// that hold them, each output word shifted out of a neighbouring pair.
__device__ __forceinline__ u32x4 lds_read16(const unsigned char *l, int off) {
    const uint32_t *d = reinterpret_cast<const uint32_t *>(l + (off & ~3));
    const uint32_t s = (uint32_t)(off & 3);
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = d[i];
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], s);
    return r;
}

// 16 bytes to LDS byte offset `off`, a multiple of 2, writing no byte
// outside [off, off + 16): dword stores when off is a multiple of 4, else a
// halfword, three realigned dwords and a halfword.
__device__ __forceinline__ void lds_write16(unsigned char *l, int off, u32x4 v) {
    if ((off & 3) == 0) {
        uint32_t *d = reinterpret_cast<uint32_t *>(l + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = v[i];
    } else {
        *reinterpret_cast<uint16_t *>(l + off) = (uint16_t)v[0];
        uint32_t *d = reinterpret_cast<uint32_t *>(l + off + 2);
#pragma unroll
        for (int i = 0; i < 3; ++i) d[i] = __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2u);
        *reinterpret_cast<uint16_t *>(l + off + 14) = (uint16_t)(v[3] >> 16);
    }
}

// The aligned blocks holding row bytes [a, a + row_bytes): b = t + i*nthreads
// for i < BLK, loaded into registers (blocks past the row are not loaded,
// nor any block of a row that is not there).
template <bool NT, int BLK>
struct Staged {
    u32x4 v[BLK];
    int delta;
    int nblk;
    __device__ __forceinline__ void load(const void *row, bool present, int64_t row_bytes, int t, int nthreads) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(row);
        delta = (int)(a & 15u);
        nblk = present ? (int)((delta + row_bytes + 15) >> 4) : 0;
        const u32x4 *blk = reinterpret_cast<const u32x4 *>(a - (uintptr_t)delta);
#pragma unroll
        for (int i = 0; i < BLK; ++i) {
            const int b = t + i * nthreads;
            if (b < nblk) {
                if constexpr (NT)
                    v[i] = __builtin_nontemporal_load(blk + b);
                else
                    v[i] = blk[b];
            }
        }
    }
    __device__ __forceinline__ void store(unsigned char *l, int t, int nthreads) const {
#pragma unroll
        for (int i = 0; i < BLK; ++i) {
            const int b = t + i * nthreads;
            if (b < nblk) *reinterpret_cast<u32x4 *>(l + 16 * b) = v[i];
        }
    }
};

// Elements past H read as 0: bytes [H*ES, nvec*16) of the row's last vector
// (at LDS offset delta) are read by the vector's owner alone -- a
// neighbour's read of a shared dword uses only its own bytes -- so that
// thread clears them, for x and (RESID) the residual, after the barrier that
// follows staging and before its own reads.
template <int XDT, bool RESID>
__device__ __forceinline__ void zero_tail(unsigned char *lx, int dx, unsigned char *lr, int dr, int64_t row_bytes,
                                          int nvec, int t, int row_threads) {
    using T = typename Fmt<XDT>::T;
    if (t != (nvec - 1) % row_threads) return;
    for (int off = (int)row_bytes; off < 16 * nvec; off += Fmt<XDT>::bytes) {
        *reinterpret_cast<T *>(lx + dx + off) = 0;
        if constexpr (RESID) *reinterpret_cast<T *>(lr + dr + off) = 0;
    }
}

// Copy the row held in l at byte offset `src` (row byte i at l + src + i) to
// the row at `row`: whole aligned blocks with 16-byte stores, the blocks
// shared with the neighbours element by element.  At most BLK blocks per
// thread.
template <int XDT, bool NT, int BLK>
__device__ __forceinline__ void unstage_row(const unsigned char *l, int src, void *row, int64_t row_bytes, int t,
                                            int nthreads) {
    constexpr int ES = Fmt<XDT>::bytes;
    using T = typename Fmt<XDT>::T;
    const uintptr_t a = reinterpret_cast<uintptr_t>(row);
    const int d = (int)(a & 15u);
    unsigned char *base = reinterpret_cast<unsigned char *>(a - (uintptr_t)d);
    const int64_t end = d + row_bytes;
    const int nblk = (int)((end + 15) >> 4);
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
        const int b = t + i * nthreads;
        if (b >= nblk) continue;
        const int lo = 16 * b, hi = lo + 16;
        if (lo >= d && hi <= end) {
            const u32x4 v = lds_read16(l, src + lo - d);
            u32x4 *dst = reinterpret_cast<u32x4 *>(base + lo);
            if constexpr (NT)
                __builtin_nontemporal_store(v, dst);
            else
                *dst = v;
        } else {
            const int s = lo > d ? lo : d, e = hi < end ? hi : (int)end;
            for (int off = s; off < e; off += ES)
                *reinterpret_cast<T *>(base + off) = *reinterpret_cast<const T *>(l + src + (off - d));
        }
    }
}

// The weight (and bias) of a staged kernel as column vectors: a 16-byte
// chunk is loaded only if it holds an element below H.
template <int WDT, int VEC, int VPT>
__device__ __forceinline__ void load_param_staged(Raw<WDT, VEC> *pr, const void *param, int t, int row_threads,
                                                  int nvec, int H) {
    constexpr int WPC = 16 / Fmt<WDT>::bytes;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (param != nullptr && v < nvec) {
#pragma unroll
            for (int c = 0; c < Raw<WDT, VEC>::CHUNKS; ++c) {
                const int j0 = v * VEC + c * WPC;
                if (j0 < H)
                    pr[k].v[c] = *reinterpret_cast<const u32x4 *>(static_cast<const char *>(param) +
                                                                   (int64_t)j0 * Fmt<WDT>::bytes);
            }
        }
    }
}

template <int XDT, int WDT, int VPT, bool RESID, bool NT, int MAXT>
__global__ void __launch_bounds__(MAXT) rmsnorm_fwd_staged_kernel(const FwdParams p) {
    constexpr int ES = Fmt<XDT>::bytes;
    constexpr int VEC = 16 / ES;
    constexpr int BLK = VPT + 1;  // a row spans at most nvec + 1 <= 64*wpr*VPT + 1 blocks
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[16];
    const int row_threads = 64 * p.wpr;
    const int slot = threadIdx.x / row_threads;
    const int t = threadIdx.x - slot * row_threads;
    const int wave_in_row = t >> 6;
    const int64_t buf = staged_buffer_bytes(p.nvec);
    unsigned char *lx = smem + (RESID ? 2 : 1) * slot * buf;
    unsigned char *lr = lx + buf;
    const int64_t row_bytes = (int64_t)p.H * ES;

    // the row's blocks first, then the weight, so that storing the blocks to
    // LDS does not wait for the weight
    const int64_t row = (int64_t)blockIdx.x * p.rpw + slot;
    const bool valid = row < p.M;
    Staged<NT, BLK> sx;
    Staged<NT, RESID ? BLK : 1> sr;
    sx.load(static_cast<const char *>(p.x) + row * p.xs * ES, valid, row_bytes, t, row_threads);
    if constexpr (RESID) sr.load(static_cast<const char *>(p.r) + row * p.rs * ES, valid, row_bytes, t, row_threads);

    Raw<WDT, VEC> wr[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) wr[k].fill_one();
    load_param_staged<WDT, VEC, VPT>(wr, p.w, t, row_threads, p.nvec, p.H);

    sx.store(lx, t, row_threads);
    if constexpr (RESID) sr.store(lr, t, row_threads);
    const int dx = sx.delta;
    const int dr = RESID ? sr.delta : 0;
    __syncthreads();
    zero_tail<XDT, RESID>(lx, dx, lr, dr, row_bytes, p.nvec, t, row_threads);

    // pass 1: sum of squares; the packed vectors stay in registers for pass 2
    float acc = 0.0f;
    Raw<XDT, VEC> xr[VPT], rr[RESID ? VPT : 1];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (v < p.nvec) {
            xr[k].v[0] = lds_read16(lx, dx + 16 * v);
            if constexpr (RESID) rr[k].v[0] = lds_read16(lr, dr + 16 * v);
        } else {
            xr[k].zero();
            if constexpr (RESID) rr[k].zero();
        }
        float hv[VEC];
        xr[k].widen_to(hv);
        if constexpr (RESID) {
            float rv[VEC];
            rr[k].widen_to(rv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(hv[e], hv[e], acc);
    }
    const float ss = row_sum(acc, p.wpr, wave_in_row, &red[slot * p.wpr]);
    const float rs = fast_rsqrt(ss * p.inv_h + p.eps);
    if (p.rrms != nullptr && valid && t == 0) p.rrms[row] = rs;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        wr[k].opaque();
        xr[k].opaque();
        if constexpr (RESID) rr[k].opaque();
    }

    // pass 2: outputs over the thread's own input bytes (values past H stay
    // in the buffer and are never copied out).  A neighbour still reading
    // its vector may read a dword this thread writes into, but it uses only
    // its own bytes of it, which no other thread writes.
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (v < p.nvec) {
            float hv[VEC], wv[VEC], o[VEC];
            xr[k].widen_to(hv);
            if constexpr (RESID) {
                float rv[VEC];
                rr[k].widen_to(rv);
#pragma unroll
                for (int e = 0; e < VEC; ++e) hv[e] = hv[e] + rv[e];
                if (p.ro != nullptr) {
                    u32x4 q;
#pragma unroll
                    for (int w = 0; w < 4; ++w) q[w] = pack_word<XDT>(hv + w * (4 / ES));
                    lds_write16(lr, dr + 16 * v, q);
                }
            }
            wr[k].widen_to(wv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = (hv[e] * rs) * wv[e];
            u32x4 q;
#pragma unroll
            for (int w = 0; w < 4; ++w) q[w] = pack_word<XDT>(o + w * (4 / ES));
            lds_write16(lx, dx + 16 * v, q);
        }
    }
    __syncthreads();
    if (valid) {
        unstage_row<XDT, NT, BLK>(lx, dx, static_cast<char *>(p.y) + row * p.ys * ES, row_bytes, t, row_threads);
        if constexpr (RESID)
            if (p.ro != nullptr)
                unstage_row<XDT, NT, BLK>(lr, dr, static_cast<char *>(p.ro) + row * p.ros * ES, row_bytes, t,
                                          row_threads);
    }
}

// LayerNorm (plain or fused with the residual add) on rows off the 16-byte
// grid: the staging of rmsnorm_fwd_staged_kernel around the two reductions
// of layernorm_fwd_kernel.  Elements past H read as 0, which adds nothing to
// the sum; the centred sum skips them.
template <int XDT, int WDT, int VPT, bool RESID, bool NT, int MAXT>
__global__ void __launch_bounds__(MAXT) layernorm_fwd_staged_kernel(const LnParams p) {
    constexpr int ES = Fmt<XDT>::bytes;
    constexpr int VEC = 16 / ES;
    constexpr int BLK = VPT + 1;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ float red[2][16];
    const int row_threads = 64 * p.wpr;
    const int slot = threadIdx.x / row_threads;
    const int t = threadIdx.x - slot * row_threads;
    const int wave_in_row = t >> 6;
    const int64_t buf = staged_buffer_bytes(p.nvec);
    unsigned char *lx = smem + (RESID ? 2 : 1) * slot * buf;
    unsigned char *lr = lx + buf;
    const int64_t row_bytes = (int64_t)p.H * ES;

    const int64_t row = (int64_t)blockIdx.x * p.rpw + slot;
    const bool valid = row < p.M;
    Staged<NT, BLK> sx;
    Staged<NT, RESID ? BLK : 1> sr;
    sx.load(static_cast<const char *>(p.x) + row * p.xs * ES, valid, row_bytes, t, row_threads);
    if constexpr (RESID) sr.load(static_cast<const char *>(p.r) + row * p.rs * ES, valid, row_bytes, t, row_threads);

    Raw<WDT, VEC> wr[VPT], br[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        wr[k].fill_one();
        br[k].zero();
    }
    load_param_staged<WDT, VEC, VPT>(wr, p.w, t, row_threads, p.nvec, p.H);
    load_param_staged<WDT, VEC, VPT>(br, p.b, t, row_threads, p.nvec, p.H);

    sx.store(lx, t, row_threads);
    if constexpr (RESID) sr.store(lr, t, row_threads);
    const int dx = sx.delta;
    const int dr = RESID ? sr.delta : 0;
    __syncthreads();
    zero_tail<XDT, RESID>(lx, dx, lr, dr, row_bytes, p.nvec, t, row_threads);

    Raw<XDT, VEC> xr[VPT], rr[RESID ? VPT : 1];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (v < p.nvec) {
            xr[k].v[0] = lds_read16(lx, dx + 16 * v);
            if constexpr (RESID) rr[k].v[0] = lds_read16(lr, dr + 16 * v);
        } else {
            xr[k].zero();
            if constexpr (RESID) rr[k].zero();
        }
    }
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
#pragma unroll
        for (int e = 0; e < VEC; ++e) s1 += hv[e];
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
        if (v < p.nvec) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if (v * VEC + e < p.H) {  // elements past H are 0, not mean
                    const float d = hv[e] - mean;
                    s2 = __builtin_fmaf(d, d, s2);
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
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        xr[k].opaque();
        if constexpr (RESID) rr[k].opaque();
        wr[k].opaque();
        br[k].opaque();
    }

    // outputs over the thread's own input bytes, then copied out
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (v < p.nvec) {
            float hv[VEC], wv[VEC], bv[VEC], o[VEC];
            widen_h(k, hv);
            if constexpr (RESID) {
                if (p.ro != nullptr) {
                    u32x4 q;
#pragma unroll
                    for (int w = 0; w < 4; ++w) q[w] = pack_word<XDT>(hv + w * (4 / ES));
                    lds_write16(lr, dr + 16 * v, q);
                }
            }
            wr[k].widen_to(wv);
            br[k].widen_to(bv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf((hv[e] - mean) * rs, wv[e], bv[e]);
            u32x4 q;
#pragma unroll
            for (int w = 0; w < 4; ++w) q[w] = pack_word<XDT>(o + w * (4 / ES));
            lds_write16(lx, dx + 16 * v, q);
        }
    }
    __syncthreads();
    if (valid) {
        unstage_row<XDT, NT, BLK>(lx, dx, static_cast<char *>(p.y) + row * p.ys * ES, row_bytes, t, row_threads);
        if constexpr (RESID)
            if (p.ro != nullptr)
                unstage_row<XDT, NT, BLK>(lr, dr, static_cast<char *>(p.ro) + row * p.ros * ES, row_bytes, t,
                                          row_threads);
    }
}

}  // namespace rmsn
