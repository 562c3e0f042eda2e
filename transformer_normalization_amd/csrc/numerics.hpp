// numerics.hpp -- storage formats, vector memory access and reductions for the
// gfx950 RMSNorm kernels.
//
// Storage formats are widened to float32 right after loading and narrowed
// with round-to-nearest-even right before storing (gfx950's v_cvt_pk_bf16_f32
// and v_cvt_pk_f16_f32).  All squares, sums and scales happen in float32, as
// "Skill: Write a Triton RMSNorm Kernel" requires in "Kernel design rules"
// (cast before squaring, float32 accumulator).  Kernels are built with
// float32 and float16 denormals enabled, so subnormal outputs are kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rmsn {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT>
struct Fmt;
template <>
struct Fmt<DT_F32> {
    using T = float;
    static constexpr int bytes = 4;
};
template <>
struct Fmt<DT_F16> {
    using T = uint16_t;
    static constexpr int bytes = 2;
};
template <>
struct Fmt<DT_BF16> {
    using T = uint16_t;
    static constexpr int bytes = 2;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- scalar conversions --------------------------------------------------

template <int DT>
__device__ __forceinline__ float widen(typename Fmt<DT>::T v);
template <>
__device__ __forceinline__ float widen<DT_F32>(float v) { return v; }
template <>
__device__ __forceinline__ float widen<DT_F16>(uint16_t v) {
    return (float)__builtin_bit_cast(_Float16, v);
}
template <>
__device__ __forceinline__ float widen<DT_BF16>(uint16_t v) {
    return __builtin_bit_cast(float, (uint32_t)v << 16);
}

template <int DT>
__device__ __forceinline__ typename Fmt<DT>::T narrow(float v);
template <>
__device__ __forceinline__ float narrow<DT_F32>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t narrow<DT_F16>(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
template <>
__device__ __forceinline__ uint16_t narrow<DT_BF16>(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// ---- packed 32-bit words ---------------------------------------------------

template <int DT>
__device__ __forceinline__ void unpack_word(uint32_t u, float *out);  // 32/bits elements
template <>
__device__ __forceinline__ void unpack_word<DT_F32>(uint32_t u, float *out) {
    out[0] = __builtin_bit_cast(float, u);
}
template <>
__device__ __forceinline__ void unpack_word<DT_F16>(uint32_t u, float *out) {
    f16x2 h = __builtin_bit_cast(f16x2, u);
    out[0] = (float)h.x;
    out[1] = (float)h.y;
}
template <>
__device__ __forceinline__ void unpack_word<DT_BF16>(uint32_t u, float *out) {
    out[0] = __builtin_bit_cast(float, u << 16);
    out[1] = __builtin_bit_cast(float, u & 0xffff0000u);
}

template <int DT>
__device__ __forceinline__ uint32_t pack_word(const float *in);
template <>
__device__ __forceinline__ uint32_t pack_word<DT_F32>(const float *in) {
    return __builtin_bit_cast(uint32_t, in[0]);
}
template <>
__device__ __forceinline__ uint32_t pack_word<DT_F16>(const float *in) {
    f32x2 v = {in[0], in[1]};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
template <>
__device__ __forceinline__ uint32_t pack_word<DT_BF16>(const float *in) {
    f32x2 v = {in[0], in[1]};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- N contiguous elements ------------------------------------------------
// N * bytes is either a multiple of 16 (one or more 16-byte accesses, which
// need 16-byte aligned addresses) or N == 1 (one element).

template <int DT, int N, bool NT = false>
__device__ __forceinline__ void load_elems(const void *base, int64_t elem, float *out) {
    constexpr int ES = Fmt<DT>::bytes;
    constexpr int BYTES = N * ES;
    const char *p = static_cast<const char *>(base) + elem * ES;
    if constexpr (BYTES % 16 == 0) {
        constexpr int PER_WORD = 4 / ES;
#pragma unroll
        for (int c = 0; c < BYTES / 16; ++c) {
            const u32x4 *q = reinterpret_cast<const u32x4 *>(p + 16 * c);
            u32x4 raw;
            if constexpr (NT)
                raw = __builtin_nontemporal_load(q);
            else
                raw = *q;
#pragma unroll
            for (int w = 0; w < 4; ++w) unpack_word<DT>(raw[w], out + (c * 4 + w) * PER_WORD);
        }
    } else {
        static_assert(N == 1, "sub-16-byte accesses are single elements");
        const typename Fmt<DT>::T *q = reinterpret_cast<const typename Fmt<DT>::T *>(p);
        if constexpr (NT)
            out[0] = widen<DT>(__builtin_nontemporal_load(q));
        else
            out[0] = widen<DT>(*q);
    }
}

// NT = true marks a streaming access (non-temporal: the line is not kept in
// the caches), for data each kernel touches exactly once.
template <int DT, int N, bool NT = false>
__device__ __forceinline__ void store_elems(void *base, int64_t elem, const float *in) {
    constexpr int ES = Fmt<DT>::bytes;
    constexpr int BYTES = N * ES;
    char *p = static_cast<char *>(base) + elem * ES;
    if constexpr (BYTES % 16 == 0) {
        constexpr int PER_WORD = 4 / ES;
#pragma unroll
        for (int c = 0; c < BYTES / 16; ++c) {
            u32x4 raw;
#pragma unroll
            for (int q = 0; q < 4; ++q) raw[q] = pack_word<DT>(in + (c * 4 + q) * PER_WORD);
            if constexpr (NT)
                __builtin_nontemporal_store(raw, reinterpret_cast<u32x4 *>(p + 16 * c));
            else
                *reinterpret_cast<u32x4 *>(p + 16 * c) = raw;
        }
    } else {
        static_assert(N == 1, "sub-16-byte accesses are single elements");
        if constexpr (NT)
            __builtin_nontemporal_store(narrow<DT>(in[0]), reinterpret_cast<typename Fmt<DT>::T *>(p));
        else
            *reinterpret_cast<typename Fmt<DT>::T *>(p) = narrow<DT>(in[0]);
    }
}

// Raw (still packed) loads, so that all of a row's loads can be issued
// before any of them is widened.  Vector tiles hold CHUNKS 16-byte words;
// single-element tiles hold one 32-bit word.
template <int DT, int N>
struct Raw {
    static constexpr int ES = Fmt<DT>::bytes;
    static constexpr bool VEC = (N * ES) % 16 == 0;
    static constexpr int CHUNKS = VEC ? (N * ES) / 16 : 1;
    static_assert(VEC || N == 1, "sub-16-byte accesses are single elements");
    using Word = typename std::conditional<VEC, u32x4, uint32_t>::type;
    Word v[CHUNKS];

    template <bool NT = false>
    __device__ __forceinline__ void load(const void *base, int64_t elem) {
        const char *p = static_cast<const char *>(base) + elem * ES;
        if constexpr (VEC) {
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c) {
                const u32x4 *q = reinterpret_cast<const u32x4 *>(p + 16 * c);
                if constexpr (NT)
                    v[c] = __builtin_nontemporal_load(q);
                else
                    v[c] = *q;
            }
        } else if constexpr (DT == DT_F32) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
            v[0] = NT ? __builtin_nontemporal_load(q) : *q;
        } else {
            const uint16_t *q = reinterpret_cast<const uint16_t *>(p);
            v[0] = NT ? __builtin_nontemporal_load(q) : *q;
        }
    }
    // Hide the value from the optimiser so that widening it again after a
    // reduction is recomputed from these packed registers instead of keeping
    // float32 copies alive across the reduction (no instruction is emitted).
    __device__ __forceinline__ void opaque() {
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) asm volatile("" : "+v"(v[c]));
    }
    // every element set to 1.0 (stands in for an absent weight; x * 1.0 is exact)
    __device__ __forceinline__ void fill_one() {
        uint32_t one;
        if constexpr (DT == DT_F32)
            one = 0x3F800000u;
        else if constexpr (DT == DT_F16)
            one = 0x3C003C00u;
        else
            one = 0x3F803F80u;
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            if constexpr (VEC)
                v[c] = u32x4{one, one, one, one};
            else
                v[c] = one;
        }
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int c = 0; c < CHUNKS; ++c) {
            if constexpr (VEC)
                v[c] = u32x4{0u, 0u, 0u, 0u};
            else
                v[c] = 0u;
        }
    }
    __device__ __forceinline__ void widen_to(float *out) const {
        if constexpr (VEC) {
            constexpr int PER_WORD = 4 / ES;
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) unpack_word<DT>(v[c][q], out + (c * 4 + q) * PER_WORD);
        } else if constexpr (DT == DT_F32) {
            out[0] = __builtin_bit_cast(float, v[0]);
        } else {
            out[0] = widen<DT>((uint16_t)v[0]);
        }
    }
};

// ---- 16-byte vectors at element-aligned addresses ---------------------------
// gfx9 runs global memory in unaligned mode: a 16-byte access at any
// element-aligned address is one global_load_dwordx4 / global_store_dwordx4.
// (Rows off the 16-byte grid: the kernels that use these keep every access
// inside the row.)

// 16 bytes at an address that is only element-aligned
typedef uint32_t u32x4_elem_aligned __attribute__((ext_vector_type(4), aligned(2)));

template <bool NT>
__device__ __forceinline__ u32x4 load16_at(const char *a) {
    const u32x4_elem_aligned *q = reinterpret_cast<const u32x4_elem_aligned *>(a);
    const u32x4_elem_aligned v = NT ? __builtin_nontemporal_load(q) : *q;
    return u32x4{v[0], v[1], v[2], v[3]};
}

template <bool NT>
__device__ __forceinline__ void store16_at(char *a, u32x4 v) {
    u32x4_elem_aligned *q = reinterpret_cast<u32x4_elem_aligned *>(a);
    const u32x4_elem_aligned u = {v[0], v[1], v[2], v[3]};
    if constexpr (NT)
        __builtin_nontemporal_store(u, q);
    else
        *q = u;
}

// ---- reductions -------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over all 64 lanes of the wave; every lane receives the same value.
// Lanes within a row of 16 combine through DPP (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror, row_mirror); each combine adds two
// equal-order partial sums, so all 16 lanes hold bit-identical row sums.  The
// four row sums are then read with v_readlane and added as (r0+r1)+(r2+r3).
// Every lane of the wave must be active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_perm<0xB1>(v);
    v += dpp_perm<0x4E>(v);
    v += dpp_perm<0x141>(v);
    v += dpp_perm<0x140>(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// Sum over the `waves` consecutive waves that share one row.  `slots` is this
// row's LDS area of at least `waves` floats for the current parity; the
// caller alternates between two areas on consecutive calls so that one
// barrier per call suffices (a wave can only come back to an area after every
// wave has passed the barrier of the call in between).  Every thread of the
// workgroup must make the call, the same number of times.
__device__ __forceinline__ float row_sum(float v, int waves, int wave_in_row, float *slots) {
    const float w = wave_sum(v);
    if (waves == 1) return w;
    if ((threadIdx.x & 63) == 0) slots[wave_in_row] = w;
    __syncthreads();
    float s = slots[0];
    for (int i = 1; i < waves; ++i) s += slots[i];
    return s;
}

__device__ __forceinline__ float fast_rsqrt(float v) { return __builtin_amdgcn_rsqf(v); }

// ---- register budgets ---------------------------------------------------------
// Largest workgroup a register tile of `elems` elements per thread may use, so
// that __launch_bounds__ leaves enough VGPRs (512 per SIMD lane shared by the
// waves of a SIMD) to hold the tile without spilling.  The host geometry uses
// the same functions.  The forward keeps x (and the residual) packed; the
// backward keeps x, dy and w packed plus float32 dw partial sums.
// es = 2 when x and its parameters (weight, AdaLN's scale and shift, LayerNorm's
// bias) are all 16-bit: then the plain forward's tiles of 48 and 64 elements
// (91-121 VGPRs), the fused residual's and AdaLN's of 24 and 32 (95-124) and
// LayerNorm's of 24 (69-108) fit 1024 threads, so longer rows stay resident
// (a float32 parameter adds 4 VGPRs per vector, and those tiles would spill).
constexpr int fwd_max_threads(int elems, int mode, int es = 4) {  // mode: 0 plain, 1 residual, 2 AdaLN
    return mode == 0 ? (elems <= 32 || (es == 2 && elems <= 64) ? 1024 : 512)
                     : (elems <= 16 || (es == 2 && elems <= 32) ? 1024 : elems <= 32 ? 512 : 256);
}
// LayerNorm keeps x (and the residual) packed plus packed weight and bias
constexpr int ln_max_threads(int elems, int es = 4) {
    return elems <= 16 || (es == 2 && elems <= 24) ? 1024 : elems <= 32 ? 512 : 256;
}
// (res: the residual backward holds a third row tile, dres, in registers;
// es: bytes per element of x.  16-bit residual tiles of 16 elements, two
// 16-byte vectors per row stream, take 111-128 VGPRs and fit 1024 threads;
// measured on gfx950 against the 512-thread cap, which sent rows of 8193 to
// 16384 elements to two passes: bf16 2048 x 16384 59.9 % of peak against
// 50.4 %, 4096 x 10240 66.3 % against 48.1 %.)
constexpr int bwd_max_threads(int elems, bool res = false, int es = 4) {
    return res ? (elems <= 8 || (es == 2 && elems <= 16) ? 1024 : elems <= 16 ? 512 : 256)
               : (elems <= 16 ? 1024 : elems <= 32 ? 512 : 256);
}

}  // namespace rmsn
