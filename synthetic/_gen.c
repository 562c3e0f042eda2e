/*
 * _gen.c -- seeded synthetic inputs (draws only; no normalisation arithmetic).
 *
 * Counter-based SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the stream
 * for (seed, stream id) starts from key = mix64(seed * GOLDEN + stream + 1)
 * and its i-th output is mix64(key + (i + 1) * GOLDEN).  Uniforms take the top
 * 53 bits; normals use Box-Muller on outputs (2k, 2k+1):
 * rad = sqrt(-2 ln(1 - u0)), theta = 2 pi u1, element 2k = rad cos(theta),
 * element 2k+1 = rad sin(theta).  Every element depends only on its position,
 * so any range of a stream can be produced on its own and in parallel.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, int stream) {
    return mix64(seed * GOLDEN + (uint64_t)(stream + 1));
}

static inline double unit53(uint64_t bits) { return (double)(bits >> 11) * 0x1.0p-53; }

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

/* out[j] = j-th uniform in [0, 1) of the stream, for j in [start, start + n) */
void syn_uniform(uint64_t seed, int stream, int64_t start, int64_t n, double *out) {
    const uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = unit53(draw(key, (uint64_t)(start + j)));
}

/* out[j] = mean + std * (normal draw at position start + j) */
void syn_normal(uint64_t seed, int stream, int64_t start, int64_t n, double mean, double sd, double *out) {
    const uint64_t key = stream_key(seed, stream);
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        const uint64_t pos = (uint64_t)(start + j);
        const uint64_t pair = pos >> 1;
        const double u0 = unit53(draw(key, 2 * pair));
        const double u1 = unit53(draw(key, 2 * pair + 1));
        const double rad = sqrt(-2.0 * log1p(-u0));
        const double th = two_pi * u1;
        const double z = (pos & 1) ? rad * sin(th) : rad * cos(th);
        out[j] = mean + sd * z;
    }
}

/* Replace each element independently with probability frac by sign * U(lo, hi)
 * (sign +1 or -1 with equal odds); positions are absolute (start + j). */
void syn_outliers(uint64_t seed, int mask_stream, int value_stream, int64_t start, int64_t n, double frac,
                  double lo, double hi, double *inout) {
    const uint64_t km = stream_key(seed, mask_stream), kv = stream_key(seed, value_stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        const uint64_t pos = (uint64_t)(start + j);
        if (unit53(draw(km, pos)) < frac) {
            const double us = unit53(draw(kv, 2 * pos));
            const double um = unit53(draw(kv, 2 * pos + 1));
            inout[j] = (us < 0.5 ? 1.0 : -1.0) * (lo + (hi - lo) * um);
        }
    }
}
