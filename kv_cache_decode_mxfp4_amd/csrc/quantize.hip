// Encoders of new cache rows:
//   - MXFP4 main KV / indexer key: rotary (fp32, no contraction) then E2M1
//     codes with one E4M3FN scale per 16 channels ([N] 2.3 and [A] 3.6 of the
//     DeepSeek-V4.1 pages: quantised after RoPE, E2M1 + E4M3 per 16, no global
//     scale);
//   - FP8 E4M3FN window rows ([N] 2.3: window KV kept in FP8).
// One thread per 16-channel group; memory-bound and tiny per decode step.
#include "device_common.h"

// Every product and sum of the encoders rounds on its own (the library is built
// with -ffp-contract=off): contracting the rotary a*c - b*s into a fused
// multiply-add moves results by an ulp and flips rounding ties of the scale and
// element codes.

namespace csa2 {
namespace {

// Non-negative finite fp32 -> E4M3FN code, round to nearest even, saturating
// at 448 (0x7E).  Values in [448, 464) round to 448; 464 and above would
// round past the largest finite code and saturate.
__device__ __forceinline__ uint32_t e4m3_rne(float v)
{
    if (!(v < 464.0f))
        return 0x7Eu;
    uint32_t u = __float_as_uint(v);
    int e = (int)(u >> 23) - 127;
    if (e < -6) {
        // subnormal range: value = m * 2^-9, m = RNE(v * 2^9) in 0..8 (8 is 2^-6)
        return (uint32_t)__builtin_rintf(v * 512.0f);
    }
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    uint32_t rem = mant & 0xFFFFFu;
    uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u)))
        code += 1u;  // a mantissa carry moves into the exponent field
    return code;
}

__device__ __forceinline__ float e4m3_value(uint32_t b)
{
    uint32_t e = b >> 3, m = b & 7u;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code of a = |x| for scale s > 0: the nearest of
// {0, .5, 1, 1.5, 2, 3, 4, 6} * s with ties to the even code.  Every
// threshold t * s is exact in fp32 (t has at most 3 significant bits, s 4).
__device__ __forceinline__ uint32_t e2m1_code(float a, float s)
{
    return (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
           (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
           (uint32_t)(a > 5.0f * s);
}

__global__ void __launch_bounds__(256)
quantize_kv_kernel(const float* __restrict__ x, int64_t rows, int32_t C,
                   const float* __restrict__ cs, const float* __restrict__ sn, int32_t rope_off,
                   int32_t rope_dim, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                   int64_t dst_stride)
{
    const int32_t G = C / 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * G)
        return;
    const int64_t r = t / G;
    const int32_t g = (int32_t)(t % G);
    const float4* src = reinterpret_cast<const float4*>(x + r * C + 16 * g);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    const int32_t half = rope_dim / 2;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int32_t c = 16 * g + 2 * p;
        if (rope_dim > 0 && c >= rope_off && c < rope_off + rope_dim) {
            const int32_t i = (c - rope_off) / 2;
            const float co = cs[r * half + i];
            const float si = sn[r * half + i];
            const float a = v[2 * p], b = v[2 * p + 1];
            v[2 * p] = __fsub_rn(__fmul_rn(a, co), __fmul_rn(b, si));
            v[2 * p + 1] = __fadd_rn(__fmul_rn(a, si), __fmul_rn(b, co));
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = e4m3_rne(__fdiv_rn(amax, 6.0f));
    const float s = e4m3_value(sb);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t c = s > 0.0f ? e2m1_code(fabsf(v[i]), s) : 0u;
        if (c != 0u && v[i] < 0.0f)
            c |= 8u;
        packed[i / 8] |= c << (4 * (i % 8));
    }
    const int64_t orow = r * dst_stride;
    *reinterpret_cast<uint2*>(codes + orow * (C / 2) + 8 * g) = make_uint2(packed[0], packed[1]);
    scales[orow * G + g] = (uint8_t)sb;
}

// Four consecutive elements per thread; row_len % 4 == 0.
__global__ void __launch_bounds__(256)
quantize_swa_kernel(const float* __restrict__ x, int64_t n, int32_t row_len,
                    uint8_t* __restrict__ out, int64_t dst_stride)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (4 * t >= n)
        return;
    const float4 f = reinterpret_cast<const float4*>(x)[t];
    const float v[4] = {f.x, f.y, f.z, f.w};
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t c = e4m3_rne(fabsf(v[i]));
        if (__float_as_uint(v[i]) >> 31)
            c |= 0x80u;
        word |= c << (8 * i);
    }
    const int64_t e = 4 * t;
    const int64_t r = e / row_len;
    const int64_t c = e % row_len;
    *reinterpret_cast<uint32_t*>(out + r * dst_stride * row_len + c) = word;
}

}  // namespace

hipError_t launch_quantize_kv(const float* x, int64_t rows, int32_t channels, const float* cs,
                              const float* sn, int32_t rope_off, int32_t rope_dim, uint8_t* codes,
                              uint8_t* scales, int64_t dst_stride, hipStream_t stream)
{
    const int64_t threads = rows * (channels / 16);
    if (threads == 0)
        return hipSuccess;
    const int64_t grid = (threads + 255) / 256;
    quantize_kv_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(
        x, rows, channels, cs, sn, rope_off, rope_dim, codes, scales, dst_stride);
    return hipGetLastError();
}

hipError_t launch_quantize_swa(const float* x, int64_t n, int32_t row_len, uint8_t* out,
                               int64_t dst_stride, hipStream_t stream)
{
    const int64_t threads = n / 4;
    if (threads == 0)
        return hipSuccess;
    const int64_t grid = (threads + 255) / 256;
    quantize_swa_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(x, n, row_len, out,
                                                                        dst_stride);
    return hipGetLastError();
}

}  // namespace csa2
