// Indexer score of one entry for one query on MFMA, shared by the full scan
// and the pool scans ([N] 2.2 and [A] 3.4 of
// the DeepSeek-V4.1 pages: the indexer scores entries with 32 heads x 128
// dims; reading: s_j = sum_h w_h * max(0, q_h . k_j), the pages fixing the
// shape, not the formula).  Every caller scores with these functions, so a
// position's score is bit-identical whichever kernel computes it.
//
// MFMA mapping (v_mfma_f32_32x32x16_f16, one wave):
//   A = q   [32 heads x 16 channels per k-step], B = k^T [16 channels x 32
//   entries], D [32 heads x 32 entries] in fp32.  Lane l owns entry l%32 and
//   the channel half h = l/32: k-step t covers channels 64h + 8t .. +8 on both
//   operands, so a lane reads code bytes [32h, 32h + 32) of its entry (chunks
//   2h and 2h + 1 of the tiled key layout) and one dword of scales.  Keys are
//   dequantised in registers (exact in fp16; the E4M3-per-16 scale is not
//   gfx950's E8M0-per-32 MX scale, so the scaled MFMA cannot take it).  Each
//   query head is pre-multiplied by a power of two that brings its largest |q|
//   to [2^14, 2^15), which keeps the bf16 -> fp16 cast exact for every value
//   within 2^28 of that maximum; the head weight absorbs the inverse power, so
//   the score is unchanged.
#pragma once

#include "device_common.h"

namespace csa2 {

struct QueryOperand {
    half8 a[8];      // A operand of k-steps 0..7
    float wr[16];    // weight (times 2^-shift) of the head of accumulator row r
};

// Load one query's indexer q (bf16 [32, 128]) and w (fp32 [32]) into the
// operand layout of the calling wave.
__device__ __forceinline__ void load_query(const uint16_t* __restrict__ q,
                                           const float* __restrict__ w, int lane,
                                           QueryOperand& Q)
{
    const int head = lane & 31;
    const int half = lane >> 5;
    const uint4* src = reinterpret_cast<const uint4*>(q + head * kIdxDim + 64 * half);
    float m = 0.0f;
    uint4 raw[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
        raw[t] = src[t];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t d[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m = fmaxf(m, fabsf(__uint_as_float(d[i] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(d[i] & 0xFFFF0000u)));
        }
    }
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    // power of two bringing max|q_h| into [2^14, 2^15); 0 for an all-zero head
    int shift = 0;
    if (m > 0.0f) {
        const int e = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
        shift = 14 - e;
        shift = shift < -100 ? -100 : (shift > 100 ? 100 : shift);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t d[4] = {raw[t].x, raw[t].y, raw[t].z, raw[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Q.a[t][2 * i] = (_Float16)ldexpf(__uint_as_float(d[i] << 16), shift);
            Q.a[t][2 * i + 1] = (_Float16)ldexpf(__uint_as_float(d[i] & 0xFFFF0000u), shift);
        }
    }
    // accumulator row r of lane l is head 8*(r/4) + 4*(l/32) + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int hr = 8 * (r / 4) + 4 * half + (r % 4);
        const int sh = __shfl(shift, hr, kWave);
        Q.wr[r] = ldexpf(w[hr], -sh);
    }
}

struct KeyTile {
    u32x4 c0, c1;   // code bytes [32h, 32h+32) of the lane's entry
    uint32_t sc;    // scale bytes [4h, 4h+4)
};

// The query operand of a workgroup's row, prepared once: wave 0 converts it
// (load_query) and stores it lane-major to LDS; after the barrier every other
// wave reads it back, so the workgroup does the conversion once instead of
// once per wave.  The values are load_query's, bit for bit.  Every wave of
// the workgroup must call it (one barrier).
struct QueryLds {
    uint4 v[12][kWave];  // a[0..7], then wr in groups of four
};

__device__ __forceinline__ void shared_query(const uint16_t* __restrict__ q,
                                             const float* __restrict__ w, int lane, int wave,
                                             QueryLds& sl, QueryOperand& Q)
{
    if (wave == 0) {
        load_query(q, w, lane, Q);
#pragma unroll
        for (int t = 0; t < 8; ++t)
            sl.v[t][lane] = __builtin_bit_cast(uint4, Q.a[t]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sl.v[8 + j][lane] = make_uint4(__float_as_uint(Q.wr[4 * j]), __float_as_uint(Q.wr[4 * j + 1]),
                                           __float_as_uint(Q.wr[4 * j + 2]),
                                           __float_as_uint(Q.wr[4 * j + 3]));
    }
    __syncthreads();
    if (wave != 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            Q.a[t] = __builtin_bit_cast(half8, sl.v[t][lane]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 u = sl.v[8 + j][lane];
            Q.wr[4 * j] = __uint_as_float(u.x);
            Q.wr[4 * j + 1] = __uint_as_float(u.y);
            Q.wr[4 * j + 2] = __uint_as_float(u.z);
            Q.wr[4 * j + 3] = __uint_as_float(u.w);
        }
    }
}

// Weighted ReLU head sum of one query's accumulators (both lanes of an entry
// return the same value).
__device__ __forceinline__ float head_sum(const QueryOperand& Q, const f32x16& acc)
{
    // max(0, x) as a signed-integer max of the bit pattern: one instruction,
    // the same value as fmaxf for every non-NaN x (-0 and negatives give +0)
    float part = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float relu = __int_as_float(max(__float_as_int(acc[r]), 0));
        part = __builtin_fmaf(Q.wr[r], relu, part);
    }
    // add the two channel halves: lanes l and l^32 hold the same entry, and
    // the swap hands every lane both partial sums (the same addition on both)
    const auto pair = __builtin_amdgcn_permlane32_swap(__float_as_uint(part),
                                                       __float_as_uint(part), false, false);
    return __uint_as_float(pair[0]) + __uint_as_float(pair[1]);
}

// Score of the lane's entry (both lanes of an entry return the same value).
__device__ __forceinline__ float score_entry(const QueryOperand& Q, const KeyTile& K)
{
    const uint32_t words[8] = {K.c0[0], K.c0[1], K.c0[2], K.c0[3], K.c1[0], K.c1[1], K.c1[2], K.c1[3]};
    f32x16 acc = {};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const _Float16 s = e4m3_byte_to_f16(K.sc, t / 2);
        const half8 b = dequant8_fp4(words[t], s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(Q.a[t], b, acc, 0, 0, 0);
    }
    return head_sum(Q, acc);
}

}  // namespace csa2
