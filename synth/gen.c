/*
 * Seeded, counter-based synthetic input generator.
 *
 * This module only draws random numbers: it holds none of the MoE layer's
 * arithmetic.  Both the fp64 oracle and the GPU path receive the very bits
 * written here, so they see identical inputs.
 *
 * Definition (every value is a pure function of (seed, stream, index), so any
 * slice of any tensor can be produced independently and in parallel):
 *
 *   key(seed, stream)    = mix(seed * G + stream)
 *   word(seed, stream, i) = mix(key + (i + 1) * G)
 *
 * where G = 0x9E3779B97F4A7C15 and mix() is the splitmix64 output function
 * (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number Generators",
 * OOPSLA 2014): word(., ., i) is the (i+1)-th output of a splitmix64 sequence
 * started at state key.
 *
 *   unit(w)   = ((w >> 11) + 1) * 2^-53                     in (0, 1]
 *   normal(i) : Box-Muller on the word pair (2p, 2p+1), p = i / 2:
 *               r = sqrt(-2 ln unit(word(2p))), th = 2 pi unit(word(2p+1)),
 *               even i -> r cos th, odd i -> r sin th.
 *
 * Storage rounding: value = sigma * normal (fp64) -> fp32 (round to nearest
 * even) -> bf16 (round to nearest even) for the bf16 tensors.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t syn_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t syn_key(uint64_t seed, uint64_t stream) {
    return syn_mix(seed * SYN_GOLDEN + stream);
}

uint64_t synth_word(uint64_t seed, uint64_t stream, uint64_t idx) {
    return syn_mix(syn_key(seed, stream) + (idx + 1) * SYN_GOLDEN);
}

static inline double syn_unit(uint64_t w) {
    return (double)((w >> 11) + 1) * 0x1.0p-53;
}

/* Both normals of pair p. */
static inline void syn_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    uint64_t w0 = syn_mix(key + (2 * p + 1) * SYN_GOLDEN);
    uint64_t w1 = syn_mix(key + (2 * p + 2) * SYN_GOLDEN);
    double r = sqrt(-2.0 * log(syn_unit(w0)));
    double th = 6.283185307179586476925286766559 * syn_unit(w1);
    *z0 = r * cos(th);
    *z1 = r * sin(th);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t idx) {
    double z0, z1;
    syn_pair(syn_key(seed, stream), idx >> 1, &z0, &z1);
    return (idx & 1) ? z1 : z0;
}

static inline uint16_t syn_f32_to_bf16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    if ((x & 0x7F800000u) == 0x7F800000u) return (uint16_t)(x >> 16); /* inf/nan: truncate */
    x += 0x7FFFu + ((x >> 16) & 1u);
    return (uint16_t)(x >> 16);
}

/*
 * Fill out[j] for j in [0, n) with element (offset + j) of the stream, times
 * sigma * row_scale[(offset + j) / row_len] when row_scale is not NULL.
 * kind: 0 -> fp64, 1 -> fp32, 2 -> bf16 (uint16 bits).
 */
static void syn_fill(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                     const double* row_scale, int64_t row_len, int kind, void* out) {
    const uint64_t key = syn_key(seed, stream);
    const int64_t chunk = 1 << 16;
    const int64_t nchunks = (n + chunk - 1) / chunk;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < nchunks; ++c) {
        int64_t j0 = c * chunk;
        int64_t j1 = j0 + chunk < n ? j0 + chunk : n;
        for (int64_t j = j0; j < j1;) {
            uint64_t idx = offset + (uint64_t)j;
            double z0, z1;
            syn_pair(key, idx >> 1, &z0, &z1);
            /* emit the element idx, and its partner too when it is the next one in range */
            for (int h = (int)(idx & 1); h < 2 && j < j1; ++h, ++j, ++idx) {
                double v = sigma * (h ? z1 : z0);
                if (row_scale) v *= row_scale[idx / (uint64_t)row_len];
                if (kind == 0) {
                    ((double*)out)[j] = v;
                } else if (kind == 1) {
                    ((float*)out)[j] = (float)v;
                } else {
                    ((uint16_t*)out)[j] = syn_f32_to_bf16((float)v);
                }
            }
        }
    }
}

void synth_fill_f64(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                    double* out) {
    syn_fill(seed, stream, offset, n, sigma, NULL, 1, 0, out);
}

void synth_fill_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                    const double* row_scale, int64_t row_len, float* out) {
    syn_fill(seed, stream, offset, n, sigma, row_scale, row_len, 1, out);
}

void synth_fill_bf16(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double sigma,
                     const double* row_scale, int64_t row_len, uint16_t* out) {
    syn_fill(seed, stream, offset, n, sigma, row_scale, row_len, 2, out);
}

/* fp32 -> bf16 bits, round to nearest even (used to store hand-made inputs). */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = syn_f32_to_bf16(in[j]);
}

/* A seeded permutation of 0..n-1 (Fisher-Yates, j = word(i) mod (i + 1)). */
void synth_permutation(uint64_t seed, uint64_t stream, int64_t n, int32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
    for (int64_t i = n - 1; i > 0; --i) {
        uint64_t j = synth_word(seed, stream, (uint64_t)i) % (uint64_t)(i + 1);
        int32_t t = out[i];
        out[i] = out[j];
        out[j] = t;
    }
}

/* The plain splitmix64 sequence started at `state` (for checking the mixer). */
void synth_splitmix64(uint64_t state, int64_t n, uint64_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = syn_mix(state + (uint64_t)(i + 1) * SYN_GOLDEN);
}
