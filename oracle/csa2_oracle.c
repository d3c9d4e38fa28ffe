/*
 * CPU oracle of the CSA2 decode / chunked-prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this file.  It shares no
 * code with the GPU library: its own format decoders and encoders, its own
 * loops, double precision throughout (fp32 only where the method itself fixes
 * fp32: the rotary step of the encoder, which works on fp32 rows).
 *
 * Sources (titles of the three web pages the method is read from):
 *   [N]  "DeepSeek V4.1: model architecture and system design, close reading"
 *        (reading notes; section 1 configuration, 2.2 CSA2, 2.3 FP4 main KV)
 *   [A]  "DeepSeek-V4.1-Flash: pushing KV cache compression to the limit"
 *        (translated abstract; 3.3 CSA2, 3.4 hierarchical sparse indexer,
 *        3.6 FP4 main KV cache)
 *   [S]  "DeepSeek-V4 model structure (7): structure decides the system"
 *        (V4 predecessor; KV cache section: top-k compressed entries plus 128
 *        window entries; closing summary: K = V single-head MQA on a
 *        512-dim latent)
 *
 * What each function follows is stated on it.  Where the pages leave a step
 * open, the reading taken is stated too.  Parity unpinned: the exact indexer
 * score nonlinearity (the pages give heads and dims, not the formula).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Formats                                                                   */
/* ------------------------------------------------------------------------- */

/*
 * OCP FP8 E4M3FN byte -> value.  [N] 2.3 and [A] 3.6 fix the scale format as
 * E4M3 with maximum 448 (448 x 6 = 2688), which is the FN variant (bias 7, no
 * infinities, S.1111.111 is NaN).
 */
double oracle_e4m3_decode(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * FP4 E2M1 nibble -> value ([N] 2.3, [A] 3.6: the main-KV element format):
 * sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is
 * subnormal.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_decode(uint8_t nib)
{
    int sign = (nib >> 3) & 1;
    int e = (nib >> 1) & 3;
    int m = nib & 1;
    double v = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, e - 1);
    return sign ? -v : v;
}

/*
 * Non-negative value -> E4M3FN byte, round to nearest, ties to the even code,
 * saturating at 448: the nearest of the 127 finite non-negative codes by
 * exhaustive search.  (Reading: the pages give the scale format, not its
 * rounding; round-to-nearest-even with saturation is the plain choice.)
 */
uint8_t oracle_e4m3_encode(double v)
{
    int best = 0;
    double bd = fabs(v - oracle_e4m3_decode(0));
    for (int c = 1; c < 127; ++c) {
        double d = fabs(v - oracle_e4m3_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)best;
}

/*
 * Signed value -> E4M3FN byte (sliding-window KV, [N] 2.3: kept in FP8, no
 * scale).  Reading: a plain sign-magnitude cast, so a negative value that
 * rounds to zero keeps its sign (-0).
 */
uint8_t oracle_e4m3_encode_signed(double v)
{
    uint8_t c = oracle_e4m3_encode(fabs(v));
    return signbit(v) ? (uint8_t)(c | 0x80) : c;
}

/* ------------------------------------------------------------------------- */
/* Encoder: rotary then MXFP4 ([N] 2.3, [A] 3.6: quantised after RoPE)       */
/* ------------------------------------------------------------------------- */

/*
 * Rotary on the pairs (x[off+2i], x[off+2i+1]), i < rope_dim/2, with the
 * caller's fp32 cos/sin:  a' = a*c - b*s,  b' = a*s + b*c, each product and
 * sum rounded to fp32 (this file is compiled without contraction).
 * Reading: the pages say only "after RoPE" and rotary on 64 of 512 dims;
 * the rotated dims are the last 64, interleaved pairs.
 */
void oracle_rope_row(float* x, const float* cs, const float* sn, int32_t off, int32_t rope_dim)
{
    for (int32_t i = 0; i < rope_dim / 2; ++i) {
        float a = x[off + 2 * i];
        float b = x[off + 2 * i + 1];
        float c = cs[i];
        float s = sn[i];
        float ac = a * c;
        float bs = b * s;
        float as = a * s;
        float bc = b * c;
        x[off + 2 * i] = ac - bs;
        x[off + 2 * i + 1] = as + bc;
    }
}

/*
 * One 16-channel group -> one E4M3 scale byte and 16 E2M1 codes
 * ([N] 2.3, [A] 3.6: E2M1 elements, one E4M3 scale per 16 channels, no
 * second-level global scale).  Reading: scale = RNE(amax / 6) in E4M3 (6 is
 * the largest E2M1 magnitude); each element is the nearest E2M1 value of
 * x / scale, ties to the even code, saturating at 6; a zero scale gives all
 * codes 0; a zero magnitude code never carries the sign (no -0).
 */
void oracle_encode_group(const float* x, uint8_t* codes16, uint8_t* scale)
{
    double amax = 0.0;
    for (int i = 0; i < 16; ++i)
        if (fabs((double)x[i]) > amax)
            amax = fabs((double)x[i]);
    uint8_t sb = oracle_e4m3_encode(amax / 6.0);
    double s = oracle_e4m3_decode(sb);
    *scale = sb;
    for (int i = 0; i < 16; ++i) {
        double a = fabs((double)x[i]);
        int best = 0;
        if (s > 0.0) {
            double bd = a;
            for (int c = 1; c < 8; ++c) {
                double d = fabs(a - oracle_e2m1_decode((uint8_t)c) * s);
                if (d < bd || (d == bd && (c & 1) == 0)) {
                    best = c;
                    bd = d;
                }
            }
        }
        if (best != 0 && x[i] < 0.0f)
            best |= 8;
        codes16[i] = (uint8_t)best;
    }
}

/*
 * Rows of C channels (C % 16 == 0) -> packed codes [rows, C/2] (channel 2j in
 * the low nibble of byte j, 2j+1 in the high nibble) and scales [rows, C/16]
 * (scale g covers channels [16g, 16g+16)).  If rope_dim > 0 the rotary step
 * runs first on a copy of each row, with cos/sin row r at cs + r*rope_dim/2.
 */
void oracle_quantize_rows(const float* x, int64_t rows, int32_t C,
                          const float* cs, const float* sn, int32_t rope_off, int32_t rope_dim,
                          uint8_t* codes, uint8_t* scales)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float row[4096];
        uint8_t q[16];
        memcpy(row, x + r * C, sizeof(float) * (size_t)C);
        if (rope_dim > 0)
            oracle_rope_row(row, cs + r * (rope_dim / 2), sn + r * (rope_dim / 2), rope_off, rope_dim);
        for (int32_t g = 0; g < C / 16; ++g) {
            oracle_encode_group(row + 16 * g, q, scales + r * (C / 16) + g);
            for (int j = 0; j < 8; ++j)
                codes[r * (C / 2) + 8 * g + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
        }
    }
}

/* fp32 rows -> E4M3FN bytes, element by element (sliding-window KV). */
void oracle_encode_fp8(const float* x, int64_t n, uint8_t* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode_signed((double)x[i]);
}

/* Decode one MXFP4 row of C channels to doubles. */
void oracle_dequant_row(const uint8_t* codes, const uint8_t* scales, int32_t C, double* out)
{
    for (int32_t c = 0; c < C; ++c) {
        uint8_t byte = codes[c / 2];
        uint8_t nib = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
        out[c] = oracle_e2m1_decode(nib) * oracle_e4m3_decode(scales[c / 16]);
    }
}

static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------- */
/* Indexer ([N] 1: 32 heads x 128; [N] 2.2, [A] 3.4: hierarchical indexer)   */
/* ------------------------------------------------------------------------- */

/*
 * Score of every entry j < n_vis for one query:
 *     s_j = sum_h w_h * max(0, sum_c q[h,c] * k_j[c]),  h < H, c < D,
 * with q bf16 [H, D], w fp32 [H], k_j the dequantised MXFP4 indexer key.
 * Reading: the pages give 32 heads x 128 and no formula; per-head dots, a
 * ReLU and a weighted head sum is the plainest form consistent with a
 * [queries*32 x 128] x [128 x entries] contraction.  Parity unpinned beyond
 * this reading.
 */
void oracle_index_scores(const uint16_t* q, const float* w, int32_t H, int32_t D,
                         const uint8_t* codes, const uint8_t* scales, int64_t n_vis, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_vis; ++j) {
        double k[1024];
        oracle_dequant_row(codes + j * (D / 2), scales + j * (D / 16), D, k);
        double s = 0.0;
        for (int32_t h = 0; h < H; ++h) {
            double d = 0.0;
            for (int32_t c = 0; c < D; ++c)
                d += bf16_value(q[h * D + c]) * k[c];
            s += (double)w[h] * (d > 0.0 ? d : 0.0);
        }
        out[j] = s;
    }
}

/*
 * Block maxima ([A] 3.4: a block's score is the largest index score among
 * its positions).  Block b covers entries [b*block, b*block + block); only
 * visible entries count; out has ceil(n_vis / block) values.
 */
void oracle_block_max(const double* s, int64_t n_vis, int32_t block, double* out)
{
    int64_t nb = (n_vis + block - 1) / block;
    for (int64_t b = 0; b < nb; ++b) {
        double m = -INFINITY;
        for (int64_t j = b * block; j < (b + 1) * block && j < n_vis; ++j)
            if (s[j] > m)
                m = s[j];
        out[b] = m;
    }
}

typedef struct {
    double s;
    int32_t i;
} scored_t;

static int by_score_then_index(const void* pa, const void* pb)
{
    const scored_t* a = (const scored_t*)pa;
    const scored_t* b = (const scored_t*)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i < b->i) ? -1 : (a->i > b->i);
}

static int ascending_i32(const void* pa, const void* pb)
{
    int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

/*
 * Top-k ([N] 1: top-k 512; [A] 3.4): the k best of n (score, index) pairs
 * under the total order (score descending, index ascending), returned as
 * ascending indices, padded with -1 to k.  Pairs with index -1 are skipped.
 * Reading: the pages do not fix a tie-break; the lower index wins.  -0 and +0
 * compare equal.  Returns the number selected.
 */
int64_t oracle_select(const double* s, const int32_t* idx, int64_t n, int64_t k, int32_t* out)
{
    scored_t* v = (scored_t*)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t j = 0; j < n; ++j) {
        int32_t id = idx ? idx[j] : (int32_t)j;
        if (id < 0)
            continue;
        v[m].s = s[j];
        v[m].i = id;
        ++m;
    }
    qsort(v, (size_t)m, sizeof(scored_t), by_score_then_index);
    int64_t take = m < k ? m : k;
    for (int64_t t = 0; t < take; ++t)
        out[t] = v[t].i;
    qsort(out, (size_t)take, sizeof(int32_t), ascending_i32);
    for (int64_t t = take; t < k; ++t)
        out[t] = -1;
    free(v);
    return take;
}

/*
 * Positions of the pool ([N] 2.2, [A] 3.4: 2048 blocks x 8 positions): block
 * b contributes b*block + r for r < block, visible entries only.  Blocks are
 * ascending with -1 padding; out has n_blocks*block slots, -1 where a slot is
 * not a visible position.
 */
void oracle_pool_positions(const int32_t* blocks, int32_t n_blocks, int32_t block, int64_t n_vis,
                           int32_t* out)
{
    for (int32_t t = 0; t < n_blocks; ++t)
        for (int32_t r = 0; r < block; ++r) {
            int64_t p = blocks[t] < 0 ? -1 : (int64_t)blocks[t] * block + r;
            out[t * block + r] = (p >= 0 && p < n_vis) ? (int32_t)p : -1;
        }
}

/*
 * Reindex scoring ([N] 2.2, [A] 3.3-3.4: a Reindex layer scores only inside
 * the Full layer's pool with its own indexer query).  out[t] is the score of
 * position pos[t], -inf where pos[t] is -1.
 */
void oracle_index_scores_at(const uint16_t* q, const float* w, int32_t H, int32_t D,
                            const uint8_t* codes, const uint8_t* scales,
                            const int32_t* pos, int64_t n, double* out)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        if (pos[t] < 0) {
            out[t] = -INFINITY;
            continue;
        }
        oracle_index_scores(q, w, H, D, codes + (int64_t)pos[t] * (D / 2),
                            scales + (int64_t)pos[t] * (D / 16), 1, out + t);
    }
}

/* ------------------------------------------------------------------------- */
/* Sparse MLA attention                                                      */
/* ([N] 1: 64 query heads x 512; [S]: K = V single-head MQA on the 512-dim  */
/*  latent, top-k compressed entries plus 128 sliding-window entries)       */
/* ------------------------------------------------------------------------- */

/*
 * One query: the key set is the valid top-k entries (0 <= sel[t] < n_cap) of
 * the MXFP4 main KV plus window rows [max(0, end - n_win), end) of the FP8
 * window buffer, all in one softmax (reading: the pages list the two sets
 * side by side; one joint softmax, no de-duplication, no sink).  For every
 * head h:  l_j = scale * q_h . v_j,  p = softmax(l),  o_h = sum_j p_j v_j,
 * lse_h = ln sum_j exp(l_j).  An empty key set gives o = 0, lse = -inf.
 * q bf16 [H, D]; out [H, D] and lse [H] in double.
 */
void oracle_attention(const uint16_t* q, int32_t H, int32_t D,
                      const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                      const int32_t* sel, int32_t k,
                      const uint8_t* swa, int64_t swa_cap, int64_t swa_end, int32_t n_win,
                      double scale, double* out, double* lse)
{
    int64_t lo = swa_end - n_win;
    if (lo < 0) lo = 0;
    int64_t hi = swa_end < swa_cap ? swa_end : swa_cap;
    int64_t n_keys = 0;
    for (int32_t t = 0; t < k; ++t)
        if (sel[t] >= 0 && sel[t] < n_cap)
            ++n_keys;
    if (hi > lo)
        n_keys += hi - lo;
    if (n_keys == 0) {
        for (int64_t i = 0; i < (int64_t)H * D; ++i)
            out[i] = 0.0;
        for (int32_t h = 0; h < H; ++h)
            lse[h] = -INFINITY;
        return;
    }
    double* v = (double*)malloc(sizeof(double) * (size_t)(n_keys * D));
    int64_t r = 0;
    for (int32_t t = 0; t < k; ++t)
        if (sel[t] >= 0 && sel[t] < n_cap)
            oracle_dequant_row(kv_codes + (int64_t)sel[t] * (D / 2),
                               kv_scales + (int64_t)sel[t] * (D / 16), D, v + (r++) * D);
    for (int64_t row = lo; row < hi; ++row, ++r)
        for (int32_t c = 0; c < D; ++c)
            v[r * D + c] = oracle_e4m3_decode(swa[row * D + c]);

    #pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < H; ++h) {
        double* l = (double*)malloc(sizeof(double) * (size_t)n_keys);
        double mx = -INFINITY;
        for (int64_t j = 0; j < n_keys; ++j) {
            double d = 0.0;
            for (int32_t c = 0; c < D; ++c)
                d += bf16_value(q[h * D + c]) * v[j * D + c];
            l[j] = scale * d;
            if (l[j] > mx)
                mx = l[j];
        }
        double sum = 0.0;
        for (int64_t j = 0; j < n_keys; ++j) {
            l[j] = exp(l[j] - mx);
            sum += l[j];
        }
        for (int32_t c = 0; c < D; ++c) {
            double o = 0.0;
            for (int64_t j = 0; j < n_keys; ++j)
                o += l[j] * v[j * D + c];
            out[h * D + c] = o / sum;
        }
        lse[h] = mx + log(sum);
        free(l);
    }
    free(v);
}

/*
 * bf16 (1 sign, 8 exponent, 7 stored significand bits) nearest to a double,
 * ties to the even significand; overflow to infinity, NaN to the quiet NaN
 * 0x7FC0.  Written from the format definition: the value is split as
 * M * 2^q with the quantum q of the binade (8 significant bits, or the fixed
 * subnormal quantum 2^-133), M is rounded to an integer with ties to even,
 * and the result, exactly a bf16 value, is read off its float bit pattern.
 */
uint16_t oracle_bf16_rne(double x)
{
    if (isnan(x))
        return 0x7FC0;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e;
    frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1): binade [2^(e-1), 2^e) */
    int q = e - 8;         /* 8 significant bits */
    if (e - 1 < -126)
        q = -133;          /* subnormal range: fixed quantum */
    const double M = ldexp(a, -q);          /* exact */
    double r = floor(M);
    const double frac = M - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    const double v = ldexp(r, q);           /* a bf16 value, or 2^128 on overflow */
    const float f = (float)v;               /* exact (or infinity past the bf16 range) */
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

/*
 * Output epilogue of the attention ([S] sequence dimension: the output is
 * rotated back to restore relative position; [N] 4 inference side: the fused
 * RoPE-attention-RoPE-cast kernel).  Reading: the rotary channels of the
 * output are rotated by minus the query position's angle, the inverse of the
 * rotation the encoder applies to keys:  a' = a c + b s,  b' = b c - a s,
 * for pairs (x[off+2i], x[off+2i+1]) with the query's (c_i, s_i); then every
 * channel is rounded to bf16.  o [H, D] double in, bits [H, D] out.
 */
void oracle_inverse_rope_bf16(const double* o, int32_t H, int32_t D, const float* cs,
                              const float* sn, int32_t off, int32_t rope_dim, uint16_t* bits)
{
    for (int32_t h = 0; h < H; ++h) {
        const double* row = o + (int64_t)h * D;
        for (int32_t c = 0; c < D; ++c) {
            double v = row[c];
            if (c >= off && c < off + rope_dim) {
                const int32_t i = (c - off) / 2;
                const double co = cs[i], si = sn[i];
                if ((c - off) % 2 == 0)
                    v = row[c] * co + row[c + 1] * si;
                else
                    v = row[c] * co - row[c - 1] * si;
            }
            bits[(int64_t)h * D + c] = oracle_bf16_rne(v);
        }
    }
}

/*
 * Indexer-key projection of new entries ([A] 3.3: a Full layer projects the
 * indexer key from the main KV; [N] 2.2: indexer K is projected from the main
 * KV): y[r, o] = sum_c x[r, c] * w[o, c], x fp32 [rows, D], w bf16 [O, D],
 * in double.  Reading: x is the main latent before its rotary.
 */
void oracle_project_rows(const float* x, int64_t rows, int32_t D, const uint16_t* w, int32_t O,
                         double* y)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t o = 0; o < O; ++o) {
            double acc = 0.0;
            for (int32_t c = 0; c < D; ++c)
                acc += (double)x[r * D + c] * bf16_value(w[(int64_t)o * D + c]);
            y[r * O + o] = acc;
        }
}

/* Sets the threads of the library's OpenMP regions (timing harness only; the
 * results do not depend on it).  n < 1 restores the runtime's default. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    static int deflt = 0;
    if (deflt == 0)
        deflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : deflt);
#else
    (void)n;
#endif
}

/* Threads an OpenMP region of this library uses. */
int oracle_threads(void)
{
    int n = 1;
#ifdef _OPENMP
    #pragma omp parallel
    {
        #pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
