// staged_kernels.hpp -- gfx950 forward RMSNorm (plain and fused residual)
// for rows that are not 16-byte aligned: H not a whole number of 16-byte
// vectors, or a base or row stride off the 16-byte grid.
//
// What is computed is exactly the forward of fwd_kernels.hpp, resident tile:
// the same float32 expressions in the same order ("Skill: Write a Triton
// RMSNorm Kernel", "Required reasoning process" steps 1-11).  Only the movement of the data differs:
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
//     elements each: vectors t, t + 64*wpr, ...), read from LDS as the two
//     aligned 16-byte blocks that hold them, joined with v_alignbyte by the
//     row's offset (the same in every lane, so every LDS access of a wave is
//     a run of consecutive 16-byte blocks, free of bank conflicts).  The sum of squares follows the
//     aligned path's tree for the tile; the tile depends on H only, so any
//     two layouts of the same rows (offsets, row pitches) give the same bits.
//     Elements past H count as 0, as the aligned path's padding vectors do.
//   * A thread holds its packed vectors (and the weight) in registers from
//     the sum to the outputs, as the aligned path does, and writes its output
//     vector to the aligned slot 16 v of the input's buffer.  The output row
//     is then copied out: every aligned 16-byte block lying wholly inside it
//     with one 16-byte store (its bytes joined from LDS as above), and the at
//     most two blocks it shares with its neighbours element by element, so
//     nothing outside the row is written.
//   * The weight (16-byte aligned) is read as column vectors; a 16-byte chunk
//     is loaded only if it holds an element below H, so the load stays inside
//     the weight's pages.
#pragma once

#include "fwd_kernels.hpp"

namespace rmsn {

// Bytes of one staging buffer for rows of nvec column vectors: the row's
// bytes start at delta < 16 and end before 16 * (nvec + 1); a read of a
// vector takes the block after the one holding its first byte, which ends by
// 16 * (nvec + 1) too, and the buffer keeps one block of slack.
__host__ __device__ constexpr int64_t staged_buffer_bytes(int64_t nvec) { return 16 * (nvec + 2); }
// LDS the staged kernels may use per workgroup (rpw row groups, one buffer
// each for the plain form, two for the fused residual)
constexpr int64_t kStagedMaxLds = 60 * 1024;

// 16 bytes at LDS byte offset blk*16 + sh (0 <= sh < 16, wave-uniform):
// the two aligned 16-byte blocks that hold them, read with ds_read_b128
// (consecutive lanes read consecutive blocks: no bank conflicts), and the
// bytes picked with a wave-uniform shift.
__device__ __forceinline__ u32x4 lds_read16_blocks(const unsigned char *l, int blk, int sh) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(l + 16 * blk);
    if (sh == 0) return a;
    const u32x4 b = *reinterpret_cast<const u32x4 *>(l + 16 * blk + 16);
    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    const uint32_t s = (uint32_t)(sh & 3);
    u32x4 r;
    switch (sh >> 2) {
#define RMSN_PICK(Q)                                                                      \
    case Q:                                                                               \
        for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbyte(w[Q + i + 1], w[Q + i], s); \
        break;
        RMSN_PICK(0)
        RMSN_PICK(1)
        RMSN_PICK(2)
        default:
        RMSN_PICK(3)
#undef RMSN_PICK
    }
    return r;
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
    const int d = __builtin_amdgcn_readfirstlane((int)(a & 15u));  // one row per wave: the same in every lane
    unsigned char *base = reinterpret_cast<unsigned char *>(a - (uintptr_t)d);
    const int64_t end = d + row_bytes;
    const int nblk = (int)((end + 15) >> 4);
#pragma unroll
    for (int i = 0; i < BLK; ++i) {
        const int b = t + i * nthreads;
        if (b >= nblk) continue;
        const int lo = 16 * b, hi = lo + 16;
        if (lo >= d && hi <= end) {
            const int off = src + lo - d;  // = 16 * (off >> 4) + (off & 15), the shift wave-uniform
            const u32x4 v = lds_read16_blocks(l, off >> 4, off & 15);
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
    const int dx = __builtin_amdgcn_readfirstlane(sx.delta);  // the same in every lane of the wave
    const int dr = RESID ? __builtin_amdgcn_readfirstlane(sr.delta) : 0;
    __syncthreads();
    zero_tail<XDT, RESID>(lx, dx, lr, dr, row_bytes, p.nvec, t, row_threads);

    // pass 1: sum of squares; the packed vectors stay in registers for pass 2
    float acc = 0.0f;
    Raw<XDT, VEC> xr[VPT], rr[RESID ? VPT : 1];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
        const int v = t + k * row_threads;
        if (v < p.nvec) {
            xr[k].v[0] = lds_read16_blocks(lx, v, dx);
            if constexpr (RESID) rr[k].v[0] = lds_read16_blocks(lr, v, dr);
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

    // pass 2: outputs at the aligned slot 16 v of the input's buffer (every
    // read of the inputs ended before the reduction's barrier, or, for a
    // one-wave row, before these writes in the wave's own order)
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
                    *reinterpret_cast<u32x4 *>(lr + 16 * v) = q;
                }
            }
            wr[k].widen_to(wv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = (hv[e] * rs) * wv[e];
            u32x4 q;
#pragma unroll
            for (int w = 0; w < 4; ++w) q[w] = pack_word<XDT>(o + w * (4 / ES));
            *reinterpret_cast<u32x4 *>(lx + 16 * v) = q;
        }
    }
    __syncthreads();
    if (valid) {
        unstage_row<XDT, NT, BLK>(lx, 0, static_cast<char *>(p.y) + row * p.ys * ES, row_bytes, t, row_threads);
        if constexpr (RESID)
            if (p.ro != nullptr)
                unstage_row<XDT, NT, BLK>(lr, 0, static_cast<char *>(p.ro) + row * p.ros * ES, row_bytes, t,
                                          row_threads);
    }
}

}  // namespace rmsn
