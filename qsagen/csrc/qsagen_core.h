/*
 * qsagen_core.h -- seeded synthetic-input generator shared by the host and
 * the device fills.  It holds no arithmetic of the attention method: only a
 * counter-based hash and two fixed-point distributions.
 *
 * Hash: the splitmix64 output function (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; constants as in
 * Vigna's public-domain splitmix64.c).
 *
 * normal(stream, e): Irwin-Hall sum of twelve 16-bit uniforms taken from
 *   three consecutive hashes (4 x 16 bits each), centred and scaled by
 *   2^-16.  The sum is an exact integer and the conversion to float is
 *   exact, so host and device produce identical bits.  Mean 0, variance
 *   ~1, support [-6, 6].
 * unit(stream, e): the top 23 bits of one hash times 2^-23, exact in
 *   float, in [0, 1).  Adding 0.5f is also exact (gives U[0.5, 1.5)).
 */
#ifndef QSAGEN_CORE_H
#define QSAGEN_CORE_H
#include <stdint.h>

#if defined(__HIPCC__)
#define QSAGEN_FN __host__ __device__ static inline
#else
#define QSAGEN_FN static inline
#endif

QSAGEN_FN uint64_t qsagen_mix(uint64_t x)
{
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* One independent stream per (seed, tensor id). */
QSAGEN_FN uint64_t qsagen_stream(uint64_t seed, uint64_t tensor_id)
{
    return qsagen_mix(seed ^ qsagen_mix(tensor_id));
}

QSAGEN_FN float qsagen_normal(uint64_t stream, uint64_t e)
{
    const uint64_t c = stream + 3ull * e;
    int32_t s = 0;
    for (int j = 0; j < 3; ++j) {
        const uint64_t h = qsagen_mix(c + (uint64_t)j);
        s += (int32_t)(h & 0xffffu) + (int32_t)((h >> 16) & 0xffffu) +
             (int32_t)((h >> 32) & 0xffffu) + (int32_t)(h >> 48);
    }
    return (float)(s - 393210) * (1.0f / 65536.0f);
}

QSAGEN_FN float qsagen_unit(uint64_t stream, uint64_t e)
{
    return (float)(qsagen_mix(stream + e) >> 41) * (1.0f / 8388608.0f);
}

#endif
