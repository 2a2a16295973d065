/* Seeded synthetic tensors for the Qwen-Image-2.1 denoiser workloads.
 *
 * Test and benchmark infrastructure: this file holds no arithmetic of the
 * denoiser itself, only the counter-based generator that both the CPU
 * oracle's tests and the GPU runs draw their inputs from.  The same
 * generator is written a second time with torch integer ops (synth.py) so
 * that full-size weights can be produced directly in device memory; the two
 * must agree bit for bit, and a test checks that they do.
 *
 * Definition (per element i of a tensor with 32-bit key k):
 *   mix(x)  = x ^= x>>16; x *= 0x21f0aaad; x ^= x>>15; x *= 0x735a2d97;
 *             x ^= x>>15                       (all mod 2^32)
 *   h1      = mix(mix(lo32(i) ^ k) ^ hi32(i)),  h2 = mix(h1 ^ 0x9e3779b9)
 *   s       = sum of the four 16-bit halves of h1 and h2
 *   value   = f32( f64(2s + 4 - 2^18) * scale + offset )
 * where scale = sigma * sqrt(3) / 2^17, so that value is an Irwin-Hall(4)
 * approximation of N(offset, sigma^2): mean offset, variance sigma^2, tails
 * cut at 3.46 sigma.  With round_bf16 the f32 value is rounded to the
 * nearest bfloat16 (ties to even) and returned widened back to f32.
 *
 * Built with -ffp-contract=off so that the multiply and the add stay two
 * separately rounded f64 operations, exactly as in the torch version.
 */
#include <stdint.h>
#include <string.h>

static inline uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x21f0aaadu;
    x ^= x >> 15;
    x *= 0x735a2d97u;
    x ^= x >> 15;
    return x;
}

static inline float round_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
    memcpy(&f, &u, 4);
    return f;
}

void synth_fill_f32(float *out, int64_t start, int64_t count, uint32_t key,
                    double scale, double offset, int round_bf16)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j) {
        uint64_t i = (uint64_t)(start + j);
        uint32_t h1 = mix32(mix32((uint32_t)i ^ key) ^ (uint32_t)(i >> 32));
        uint32_t h2 = mix32(h1 ^ 0x9e3779b9u);
        int64_t s = (int64_t)(h1 & 0xffffu) + (int64_t)(h1 >> 16)
                  + (int64_t)(h2 & 0xffffu) + (int64_t)(h2 >> 16);
        double z = (double)(2 * s + 4 - 262144) * scale;
        z = z + offset;
        float f = (float)z;
        out[j] = round_bf16 ? round_to_bf16(f) : f;
    }
}

uint32_t synth_mix32(uint32_t x) { return mix32(x); }
