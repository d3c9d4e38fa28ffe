/*
 * Seeded synthetic inputs for the CSA2 decode / prefill workloads.
 *
 * This module produces INPUTS only: Gaussian latents, RMS-normalised latent
 * rows with sparse outliers, bf16 query vectors, uniform head weights and
 * rotary cos/sin tables.  It holds none of the method's arithmetic (no
 * rotary application, no FP4/FP8 encoding, no scoring, no selection, no
 * attention).  Both the GPU path and the CPU oracle consume what it writes.
 *
 * Random numbers are counter based, so any slice of any tensor can be
 * regenerated on its own and in parallel:
 *   - SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom
 *     number generators", OOPSLA 2014) applied to key + (counter+1)*golden;
 *   - uniforms on the open interval (0,1) from the top 53 bits;
 *   - standard normals by the Box-Muller transform in double, one pair of
 *     normals (cos and sin branch) per pair of uniforms.
 *
 * Distribution recipe (the latent amplitude argument of the DeepSeek-V4.1
 * reading notes, section 2.3 "FP4 main KV cache": a 512-channel latent after
 * RMSNorm has L2 norm at most sqrt(512), training saw magnitudes of about
 * 10): each latent row is N(0,1) per channel, each channel is replaced by
 * +-10 with probability 1e-3, then the row is RMS-normalised (eps 1e-6, no
 * gain) in double and rounded to fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Value number `ctr` of the counter-based stream `key`. */
static inline uint64_t draw(uint64_t key, uint64_t ctr)
{
    return mix64(key + (ctr + 1ULL) * GOLDEN);
}

/* Uniform in the open interval (0,1): 53 random bits plus one half. */
static inline double u01(uint64_t h)
{
    return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Stream key for (seed, config, tensor tag, layer, sequence). */
uint64_t synth_key(uint64_t seed, uint64_t config, uint64_t tag, uint64_t layer, uint64_t seq)
{
    uint64_t k = draw(seed, config);
    k = draw(k, tag);
    k = draw(k, layer);
    return draw(k, seq);
}

/* Standard normal number i of stream `key` (Box-Muller on pair i/2). */
static inline double normal_at(uint64_t key, uint64_t i)
{
    uint64_t p = i >> 1;
    double u1 = u01(draw(key, 2 * p));
    double u2 = u01(draw(key, 2 * p + 1));
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

/* out[i] = fp32(scale * z[start + i]), z standard normal. */
void synth_normal_f32(uint64_t key, int64_t start, int64_t n, double scale, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(scale * normal_at(key, (uint64_t)(start + i)));
}

/* Round an fp32 value to bf16 (round to nearest, ties to even); finite input. */
static inline uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* out[i] = bf16(fp32(scale * z[start + i])). */
void synth_normal_bf16(uint64_t key, int64_t start, int64_t n, double scale, uint16_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = f32_to_bf16((float)(scale * normal_at(key, (uint64_t)(start + i))));
}

/* out[i] = fp32(lo + (hi - lo) * u[start + i]), u uniform on (0,1). */
void synth_uniform_f32(uint64_t key, int64_t start, int64_t n, double lo, double hi, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (float)(lo + (hi - lo) * u01(draw(key, (uint64_t)(start + i))));
}

/*
 * Latent rows [row0, row0 + rows) of a C-channel tensor: N(0,1) channels,
 * each replaced by +-outlier with probability p_out (sign from the draw's low
 * bit), then RMS-normalised in double with eps and rounded to fp32.
 * Element (r, c) uses counter r*C + c in both streams.
 */
void synth_latent_rows(uint64_t key, uint64_t key_out, int64_t row0, int64_t rows, int32_t C,
                       double p_out, double outlier, double eps, float* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double x[4096];
        uint64_t base = (uint64_t)(row0 + r) * (uint64_t)C;
        double ss = 0.0;
        for (int32_t c = 0; c < C; ++c) {
            double v = normal_at(key, base + (uint64_t)c);
            uint64_t h = draw(key_out, base + (uint64_t)c);
            if (u01(h) < p_out)
                v = (h & 1ULL) ? -outlier : outlier;
            x[c] = v;
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)C + eps);
        for (int32_t c = 0; c < C; ++c)
            out[r * (int64_t)C + c] = (float)(x[c] * inv);
    }
}

/*
 * Rotary tables for positions pos[0..rows): angle_i = pos * base^(-2i/rope_dim)
 * for i < rope_dim/2, cos and sin in double, rounded to fp32.  Layout
 * [rows, rope_dim/2].
 */
void synth_rope_table(const int64_t* pos, int64_t rows, int32_t rope_dim, double base,
                      float* cos_out, float* sin_out)
{
    int32_t half = rope_dim / 2;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t i = 0; i < half; ++i) {
            double inv_freq = pow(base, -2.0 * (double)i / (double)rope_dim);
            double a = (double)pos[r] * inv_freq;
            cos_out[r * half + i] = (float)cos(a);
            sin_out[r * half + i] = (float)sin(a);
        }
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int synth_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
