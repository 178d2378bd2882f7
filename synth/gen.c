/*
 * Seeded synthetic inputs for causal differential attention.
 *
 * This module only draws numbers: it holds none of the attention arithmetic,
 * and both the HIP path's tests and the fp64 oracle take their inputs from it.
 *
 * Generator (counter-based, so any element can be drawn on its own):
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): the k-th output (k = 0, 1, ...) of a generator
 *     seeded with x is mix(x + (k + 1) * 0x9E3779B97F4A7C15), where mix is the
 *     variant-13 finaliser below.
 *   - Stream key of (seed, tensor id): output 0 of SplitMix64 seeded with
 *     (seed << 8) | tensor_id.
 *   - Element n of a stream uses outputs 2n and 2n + 1 of SplitMix64 seeded
 *     with the stream key, as u1 = (z0 >> 11 + 1) * 2^-53 in (0, 1] and
 *     u2 = (z1 >> 11) * 2^-53 in [0, 1).
 *   - Standard normal by Box and Muller (1958), cosine branch:
 *     sqrt(-2 ln u1) * cos(2 pi u2), in fp64.
 *   - bf16 values are the fp64 normal rounded once, to nearest-even, to 8
 *     significant bits (no double rounding through fp32).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* k-th output (0-based) of SplitMix64 seeded with x. */
uint64_t synth_splitmix64(uint64_t x, uint64_t k) { return sm64_mix(x + (k + 1) * GOLDEN_GAMMA); }

uint64_t synth_stream_key(uint64_t seed, uint32_t tensor_id) {
    return synth_splitmix64((seed << 8) | (uint64_t)(tensor_id & 0xFF), 0);
}

static inline double normal_at(uint64_t key, uint64_t n) {
    uint64_t z0 = synth_splitmix64(key, 2 * n), z1 = synth_splitmix64(key, 2 * n + 1);
    double u1 = (double)((z0 >> 11) + 1) * 0x1p-53;
    double u2 = (double)(z1 >> 11) * 0x1p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline double uniform_at(uint64_t key, uint64_t n) {
    return (double)(synth_splitmix64(key, n) >> 11) * 0x1p-53;
}

/* fp64 -> bf16 bits, one rounding to nearest-even (normal and subnormal bf16 range). */
uint16_t synth_f64_to_bf16(double x) {
    if (x != x) return 0x7FC0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    frexp(x, &e);                  /* |x| = f * 2^e, f in [0.5, 1) */
    int q = e - 8;                 /* quantum of an 8-significant-bit value */
    if (q < -133) q = -133;        /* bf16 subnormal quantum 2^-133 */
    double r = nearbyint(ldexp(x, -q));
    double y = ldexp(r, q);
    if (fabs(y) > 3.3895313892515355e38) return signbit(y) ? 0xFF80 : 0x7F80; /* beyond max bf16 */
    float f = (float)y;            /* exact: y has <= 8 significant bits in fp32 range */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* n standard normals of stream (seed, tensor_id) starting at element `first`, as fp64. */
void synth_normal_f64(uint64_t seed, uint32_t tensor_id, uint64_t first, int64_t n, double* out) {
    uint64_t key = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, first + (uint64_t)i);
}

/* n standard normals rounded to bf16 (bit patterns). */
void synth_normal_bf16(uint64_t seed, uint32_t tensor_id, uint64_t first, int64_t n, uint16_t* out) {
    uint64_t key = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = synth_f64_to_bf16(normal_at(key, first + (uint64_t)i));
}

/* n values mean + std * N(0,1), rounded once to fp32. */
void synth_normal_f32(uint64_t seed, uint32_t tensor_id, uint64_t first, int64_t n, double mean, double std, float* out) {
    uint64_t key = synth_stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal_at(key, first + (uint64_t)i));
}

/* n values uniform on [lo, hi), rounded once to fp32. */
void synth_uniform_f32(uint64_t seed, uint32_t tensor_id, uint64_t first, int64_t n, double lo, double hi, float* out) {
    uint64_t key = synth_stream_key(seed, tensor_id);
    for (int64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * uniform_at(key, first + (uint64_t)i));
}
