// Device helpers shared by the gfx950 kernels of libcsa2: vector types, MXFP4 /
// E4M3 conversions (hardware converters, verified against the format
// definitions by the parity tests), wave and workgroup reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dims.h"

namespace csa2 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// --------------------------------------------------------------- formats

// Selection order of a score as an unsigned key: larger score <=> larger key,
// -0 ranks as +0; key 0 is below every score and marks "no entry".
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;  // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Byte offset of code byte c (< 64) of indexer-key entry f in the tiled key
// cache (layout in dims.h).
__device__ __forceinline__ int64_t key_code_offset(int64_t f, int c)
{
    return (f >> 5) * kKeyTileBytes + (c >> 4) * kKeyPlane + (f & 31) * 16 + (c & 15);
}


// 8 E2M1 codes (one dword, channel 2j in the low nibble of byte j) times the
// scale s -> 8 fp16 values in channel order.  The hardware converter applies
// only the exponent of its fp32 scale, so it runs with 1.0 and the E4M3 scale
// (its value exact in fp16) is applied by a packed fp16 multiply.  Every
// E2M1 x E4M3 product has at most 5 significant bits and lies in
// [2^-10, 2688], so the result is exact.
__device__ __forceinline__ half8 dequant8_fp4(uint32_t word, _Float16 s)
{
    half2v ss = {s, s};
    half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * ss;
    half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * ss;
    half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * ss;
    half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * ss;
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// Four E4M3FN bytes of one dword -> four fp16 (exact: E4M3 is a subset of fp16).
__device__ __forceinline__ half4v e4m3x4_to_f16(uint32_t word)
{
    half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
    half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true);
    half4v r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = hi[0]; r[3] = hi[1];
    return r;
}

// Byte `i` of a dword as an E4M3 value in fp16.
__device__ __forceinline__ _Float16 e4m3_byte_to_f16(uint32_t word, int i)
{
    half4v v = e4m3x4_to_f16(word);
    return v[i];
}

__device__ __forceinline__ _Float16 bf16_to_f16(uint16_t b)
{
    return (_Float16)__uint_as_float((uint32_t)b << 16);
}

// --------------------------------------------------------------- reductions
//
// DPP forms: row_shr:n moves lane i-n -> i inside each row of 16 lanes (lanes
// without a source read `old`); rows are then combined through v_readlane.

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, kCtrl, 0xF, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x, int lane)
{
    x += dpp_u32<0x111>(0u, x);
    x += dpp_u32<0x112>(0u, x);
    x += dpp_u32<0x114>(0u, x);
    x += dpp_u32<0x118>(0u, x);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = lane >> 4;
    x += row >= 1 ? r0 : 0u;
    x += row >= 2 ? r1 : 0u;
    x += row >= 3 ? r2 : 0u;
    return x;
}

// Wave-uniform maximum / minimum / sum of unsigned values.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x)
{
    x = max(x, dpp_u32<0x111>(0u, x));
    x = max(x, dpp_u32<0x112>(0u, x));
    x = max(x, dpp_u32<0x114>(0u, x));
    x = max(x, dpp_u32<0x118>(0u, x));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x)
{
    x = min(x, dpp_u32<0x111>(0xFFFFFFFFu, x));
    x = min(x, dpp_u32<0x112>(0xFFFFFFFFu, x));
    x = min(x, dpp_u32<0x114>(0xFFFFFFFFu, x));
    x = min(x, dpp_u32<0x118>(0xFFFFFFFFu, x));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_sum(x, lane), 63);
}

// Number of lanes below `lane` whose bit is set in a wave-wide ballot.
__device__ __forceinline__ uint32_t lanes_below(uint64_t ballot, int lane)
{
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    return (uint32_t)__popcll(ballot & below);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, kWave);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane)
{
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(v, o, kWave);
        if (lane >= o)
            v += t;
    }
    return v;
}

}  // namespace csa2
