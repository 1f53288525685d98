/*
 * synth_gen.h -- seeded synthetic inputs, integer-only so that the host build (gcc) and
 * the device build (hipcc) produce bit-identical values.
 *
 * This header generates test and benchmark inputs only.  It contains no part of the
 * quantization or attention arithmetic; both the CPU oracle and the GPU library receive
 * the tensors it produces.
 *
 * Generator: the splitmix64 output mixer (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to a per-element counter.  Each
 * element sums twelve 16-bit uniforms (Irwin-Hall, n = 12): S - 6*65535 has mean 0 and
 * variance 12 * (65536^2 - 1) / 12 ~= 2^32, so x = (S - 393210) * 2^-16 approximates
 * N(0, 1) on (-6, 6) and is exact in binary32.
 *
 * Element addressing is by coordinates, not by a tensor's allocated shape: element
 * (b, t, h, c) of stream (seed, kind, layer) is the same value whatever slice of the
 * tensor is generated, so any sub-block can be regenerated independently.
 */
#ifndef KVQ_SYNTH_GEN_H
#define KVQ_SYNTH_GEN_H

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define SG_FN __host__ __device__ static inline
#else
#define SG_FN static inline
#endif

#define SG_GOLDEN 0x9E3779B97F4A7C15ULL

SG_FN uint64_t sg_mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* one stream per (seed, tensor kind, layer) */
SG_FN uint64_t sg_stream_key(uint64_t seed, uint32_t kind, uint32_t layer)
{
    return sg_mix64(seed ^ sg_mix64(((uint64_t)kind << 32) | (uint64_t)layer));
}

/* element coordinates: b < 2^24, t < 2^24, h < 256, c < 256 */
SG_FN uint64_t sg_counter(uint32_t b, uint32_t t, uint32_t h, uint32_t c)
{
    return ((uint64_t)b << 40) | ((uint64_t)t << 16) | ((uint64_t)h << 8) | (uint64_t)c;
}

SG_FN float sg_normal(uint64_t key, uint64_t ctr)
{
    uint64_t base = sg_mix64(key + ctr * SG_GOLDEN);
    int32_t S = 0;
    for (int i = 1; i <= 3; ++i) {
        uint64_t r = sg_mix64(base + (uint64_t)i * SG_GOLDEN);
        S += (int32_t)(r & 0xFFFFu) + (int32_t)((r >> 16) & 0xFFFFu) +
             (int32_t)((r >> 32) & 0xFFFFu) + (int32_t)(r >> 48);
    }
    return (float)(S - 393210) * (1.0f / 65536.0f);
}

/* bfloat16 bits of a finite binary32 value, round to nearest even (input preparation) */
SG_FN uint16_t sg_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* Value of element (b, t, h, c); chan_mult (may be NULL) is a per (h, c) multiplier used
 * for outlier channels, applied in binary32 before any rounding to bf16. */
SG_FN float sg_value(uint64_t key, uint32_t b, uint32_t t, uint32_t h, uint32_t c,
                     const float *chan_mult, int head_dim)
{
    float x = sg_normal(key, sg_counter(b, t, h, c));
    if (chan_mult) x *= chan_mult[h * head_dim + c];
    return x;
}

#endif
