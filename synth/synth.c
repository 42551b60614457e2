/*
 * synth.c -- seeded, counter-based normal samples for synthetic inputs.
 *
 * Holds no arithmetic of the MoE method: only a random number generator.
 * Element j of a stream (seed, tag) is a pure function of (seed, tag, j), so
 * any slice can be generated on its own and the result does not depend on
 * the thread count.
 *
 *   key      = mix(seed ^ mix(tag * G + 1))
 *   z1, z2   = mix(key + (2j + 1) * G), mix(key + (2j + 2) * G)
 *   u1       = ((z1 >> 11) + 1) * 2^-53        in (0, 1]
 *   u2       =  (z2 >> 11)      * 2^-53        in [0, 1)
 *   n        = sqrt(-2 ln u1) * cos(2 pi u2)   (Box-Muller, in double)
 *   out[j]   = (float)(mean + std * n)
 *
 * mix() is the SplitMix64 output function (S. Vigna), G = 0x9E3779B97F4A7C15.
 */
#include <math.h>
#include <stdint.h>

static uint64_t mix(uint64_t z)
{
    z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27; z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

#define GOLDEN 0x9E3779B97F4A7C15ULL

static double normal_at(uint64_t key, uint64_t j)
{
    uint64_t z1 = mix(key + (2 * j + 1) * GOLDEN);
    uint64_t z2 = mix(key + (2 * j + 2) * GOLDEN);
    double u1 = (double)((z1 >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(z2 >> 11) * 0x1.0p-53;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* out[j] = mean + std * N(0,1) sample number (first + j) of stream (seed, tag). */
void synth_normal_f32(uint64_t seed, uint64_t tag, int64_t first, int64_t n,
                      double mean, double std, float* out)
{
    uint64_t key = mix(seed ^ mix(tag * GOLDEN + 1));
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = (float)(mean + std * normal_at(key, (uint64_t)(first + j)));
}

/* Same stream in double precision (for inputs built from several parts). */
void synth_normal_f64(uint64_t seed, uint64_t tag, int64_t first, int64_t n,
                      double mean, double std, double* out)
{
    uint64_t key = mix(seed ^ mix(tag * GOLDEN + 1));
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = mean + std * normal_at(key, (uint64_t)(first + j));
}
