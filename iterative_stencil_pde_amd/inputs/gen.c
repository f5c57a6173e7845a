/* Seeded, counter-based input draws for the synthetic workloads.
 *
 * This file holds no arithmetic of the iteration itself: it only produces the
 * random numbers and coordinate functions that the workloads are built from.
 * The same bytes are handed to the CPU oracle and to the GPU engine.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used as a counter-based hash. Draw k of
 * stream s under seed S is splitmix64(key) with
 *     key = (S << 40) ^ (s << 32) ^ k,      k < 2^32, s < 256, S < 2^24.
 * A uniform on [0,1) takes the top 53 bits: (x >> 11) * 2^-53.
 * Normals use the Box-Muller transform on streams s and s+1:
 *     z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2).
 * Built with -O2 -ffp-contract=off against the C library's log/cos/sin.
 */
#include <math.h>
#include <stdint.h>

static uint64_t splitmix64(uint64_t key) {
    uint64_t z = key + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double unit_draw(uint64_t seed, uint64_t stream, uint64_t k) {
    const uint64_t key = (seed << 40) ^ (stream << 32) ^ k;
    return (double)(splitmix64(key) >> 11) * 0x1.0p-53;
}

/* out[k] = lo + (hi - lo) * U_k for k in [0, n). Returns -1 on bad arguments. */
int pkgen_uniform(uint64_t seed, uint32_t stream, int64_t n, double lo, double hi, double* out) {
    if (n < 0 || n > ((int64_t)1 << 32) || stream > 255 || seed >= ((uint64_t)1 << 24) || !out)
        return -1;
    const double span = hi - lo;
    for (int64_t k = 0; k < n; ++k) out[k] = lo + span * unit_draw(seed, stream, (uint64_t)k);
    return 0;
}

/* out[k] = mean + sd * Z_k, Z_k standard normal from streams (stream, stream+1). */
int pkgen_normal(uint64_t seed, uint32_t stream, int64_t n, double mean, double sd, double* out) {
    if (n < 0 || n > ((int64_t)1 << 32) || stream > 254 || seed >= ((uint64_t)1 << 24) || !out)
        return -1;
    const double two_pi = 6.283185307179586476925286766559;
    for (int64_t k = 0; k < n; ++k) {
        const double u1 = 1.0 - unit_draw(seed, stream, (uint64_t)k); /* (0, 1] */
        const double u2 = unit_draw(seed, stream + 1u, (uint64_t)k);
        out[k] = mean + sd * (sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
    }
    return 0;
}

/* out[j] = sin(p * pi * j * h) for j in [0, n): the grid samples of sin(p pi x). */
int pkgen_sinpi(int64_t n, double h, double p, double* out) {
    if (n < 0 || !out) return -1;
    const double pi = 3.14159265358979323846264338327950288;
    for (int64_t j = 0; j < n; ++j) out[j] = sin(p * pi * ((double)j * h));
    return 0;
}
