/*
 * Seeded synthetic inputs shared by the oracle and the HIP path.
 *
 * This file holds no arithmetic of the vision encoder itself: it only draws
 * random numbers.  Every value is a pure function of (seed, stream, index), so
 * any slice can be regenerated independently and in parallel.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; constants as published by S. Vigna), used as
 * a counter-based hash of  seed ^ (stream << 40) ^ index.
 * Normals: Box-Muller on two 53-bit uniforms, in double.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

static uint64_t mix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index)
{
    return mix64(seed ^ (stream << 40) ^ index);
}

/* Uniform double in [0, 1) with 53 random bits. */
static double unit53(uint64_t r) { return (double)(r >> 11) * (1.0 / 9007199254740992.0); }

/* fp32 -> bf16 bits, round to nearest even (finite inputs only). */
static uint16_t to_bf16_bits(float f)
{
    union { float f; uint32_t u; } v = { f };
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Standard normal number e of a stream: Box-Muller on the uniform pair (2p, 2p+1),
 * p = e / 2; even e takes the cosine branch and odd e the sine branch. */
static void normals(uint64_t seed, uint64_t stream, uint64_t offset, size_t n,
                    double mean, double std, float *outf, uint16_t *outb)
{
    const double two_pi = 6.283185307179586476925286766559;
    size_t i = 0;
    while (i < n) {
        uint64_t e = offset + i, p = e >> 1;
        double u1 = 1.0 - unit53(synth_u64(seed, stream, 2u * p));       /* (0, 1] */
        double u2 = unit53(synth_u64(seed, stream, 2u * p + 1u));
        double r = sqrt(-2.0 * log(u1)), a = two_pi * u2;
        for (uint64_t k = e & 1u; k < 2u && i < n; ++k, ++i) {
            float v = (float)(mean + std * r * (k ? sin(a) : cos(a)));
            if (outf) outf[i] = v;
            if (outb) outb[i] = to_bf16_bits(v);
        }
    }
}

/* out[i] = bf16(float(mean + std * N(0,1)_e)), e = offset + i. */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, size_t n,
                       double mean, double std, uint16_t *out)
{
    normals(seed, stream, offset, n, mean, std, 0, out);
}

/* Same draws as synth_normal_bf16, kept in fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, size_t n,
                      double mean, double std, float *out)
{
    normals(seed, stream, offset, n, mean, std, out, 0);
}

/* Uniform bytes U{0..255}: the top 8 bits of each draw. */
void synth_bytes(uint64_t seed, uint64_t stream, uint64_t offset, size_t n, uint8_t *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = (uint8_t)(synth_u64(seed, stream, offset + i) >> 56);
}

/* Uniform doubles in [0, 1). */
void synth_uniform(uint64_t seed, uint64_t stream, uint64_t offset, size_t n, double *out)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = unit53(synth_u64(seed, stream, offset + i));
}
