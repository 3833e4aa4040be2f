/*
 * Seeded synthetic inputs for the long-range branch workloads.
 *
 * This file holds no arithmetic of the attention method: it only draws the
 * query/key/value tensors that the method consumes, so that the GPU path and
 * the fp64 CPU oracle can be fed the very same numbers.
 *
 * Generator: a counter-based stream built from the SplitMix64 output function
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014).  Every value is a pure function of (seed, stream, index), so
 * any slice of any tensor can be regenerated on its own.  Normal deviates use
 * the Box-Muller transform in fp64 (one pair of uniforms per pair of indices,
 * the cosine branch for even indices and the sine branch for odd ones).
 */
#include <math.h>
#include <stdint.h>

#define GEN_PI 3.14159265358979323846

static inline uint64_t splitmix_out(uint64_t z)
{
    z += 0x9e3779b97f4a7c15ULL;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

/* Base key of one stream: independent of the index. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream)
{
    return splitmix_out(splitmix_out(seed) ^ (stream * 0xd1b54a32d192ed03ULL));
}

/* 64 random bits at counter `idx` of stream `key`. */
static inline uint64_t bits_at(uint64_t key, uint64_t idx)
{
    return splitmix_out(key + 0x632be59bd9b4e019ULL * idx);
}

/* Raw 64-bit draws for indices [start, start+count). */
void synth_bits(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, uint64_t *out)
{
    const uint64_t key = stream_key(seed, stream);
    for (uint64_t n = 0; n < count; ++n)
        out[n] = bits_at(key, start + n);
}

/* Standard normal at index idx of the stream (Box-Muller on the pair idx/2). */
static inline double normal_at(uint64_t key, uint64_t idx)
{
    const uint64_t pair = idx >> 1;
    const uint64_t z1 = bits_at(key, 2 * pair);
    const uint64_t z2 = bits_at(key, 2 * pair + 1);
    const double u1 = ((double)(z1 >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    const double u2 = (double)(z2 >> 11) * 0x1.0p-53;         /* [0, 1) */
    const double r = sqrt(-2.0 * log(u1));
    const double t = 2.0 * GEN_PI * u2;
    return (idx & 1) ? r * sin(t) : r * cos(t);
}

/* Standard normals for indices [start, start+count), in fp64. */
void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, double *out)
{
    const uint64_t key = stream_key(seed, stream);
    for (uint64_t n = 0; n < count; ++n)
        out[n] = normal_at(key, start + n);
}

static inline uint16_t f32_to_bf16_rne(float f)
{
    union { float f; uint32_t u; } c;
    c.f = f;
    uint32_t u = c.u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/*
 * One [rows, d] slab of a feature tensor: element (r, f) is the normal at flat
 * index (row0 + r) * d + f of the stream, multiplied by row_scale[r] (or 1 when
 * row_scale is NULL), computed in fp64 and rounded to fp32.  When out_bf16 is
 * non-NULL the fp32 value is further rounded (nearest-even) to bf16 bits and
 * stored there instead of out_f32.
 */
void synth_rows(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t rows, uint32_t d,
                const double *row_scale, float *out_f32, uint16_t *out_bf16)
{
    const uint64_t key = stream_key(seed, stream);
    for (uint64_t r = 0; r < rows; ++r) {
        const double sc = row_scale ? row_scale[r] : 1.0;
        const uint64_t base = (row0 + r) * (uint64_t)d;
        for (uint32_t f = 0; f < d; ++f) {
            const uint64_t idx = base + f;
            double z;
            if (!(idx & 1) && f + 1 < d) {
                /* both members of the Box-Muller pair land in this row */
                const uint64_t z1 = bits_at(key, idx);
                const uint64_t z2 = bits_at(key, idx + 1);
                const double u1 = ((double)(z1 >> 11) + 1.0) * 0x1.0p-53;
                const double u2 = (double)(z2 >> 11) * 0x1.0p-53;
                const double rr = sqrt(-2.0 * log(u1));
                const double t = 2.0 * GEN_PI * u2;
                const float x0 = (float)(rr * cos(t) * sc);
                const float x1 = (float)(rr * sin(t) * sc);
                if (out_bf16) {
                    out_bf16[r * d + f] = f32_to_bf16_rne(x0);
                    out_bf16[r * d + f + 1] = f32_to_bf16_rne(x1);
                } else {
                    out_f32[r * d + f] = x0;
                    out_f32[r * d + f + 1] = x1;
                }
                ++f;
                continue;
            }
            z = normal_at(key, idx);
            const float x = (float)(z * sc);
            if (out_bf16)
                out_bf16[r * d + f] = f32_to_bf16_rne(x);
            else
                out_f32[r * d + f] = x;
        }
    }
}
