// Encoders of new cache rows:
//   - MXFP4 main KV / indexer key: rotary (fp32, no contraction) then E2M1
//     codes with one E4M3FN scale per 16 channels ([N] 2.3 and [A] 3.6 of the
//     DeepSeek-V4.1 pages: quantised after RoPE, E2M1 + E4M3 per 16, no global
//     scale);
//   - FP8 E4M3FN window rows ([N] 2.3: window KV kept in FP8).
// One thread per 16-channel group; memory-bound and tiny per decode step.
#include "device_common.h"
#include "launch.h"

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

// Rotary on the pairs of one 16-channel group g of row r that fall inside
// [rope_off, rope_off + rope_dim): a' = a*c - b*s, b' = a*s + b*c, every
// product and sum rounded to fp32.
__device__ __forceinline__ void rope_group(float (&v)[16], int32_t g, int64_t r,
                                           const float* __restrict__ cs,
                                           const float* __restrict__ sn, int32_t rope_off,
                                           int32_t rope_dim)
{
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
}

// E4M3 scale byte of a group whose largest magnitude is amax: RNE(amax / 6).
__device__ __forceinline__ uint32_t group_scale(float amax)
{
    return e4m3_rne(__fdiv_rn(amax, 6.0f));
}

// Signed E2M1 nibble of x under scale value s (no -0 nibble; scale 0 -> 0).
__device__ __forceinline__ uint32_t e2m1_nibble(float x, float s)
{
    uint32_t c = s > 0.0f ? e2m1_code(fabsf(x), s) : 0u;
    if (c != 0u && x < 0.0f)
        c |= 8u;
    return c;
}

// One 16-channel group: codes (channel 2j in the low nibble of byte j) and
// the scale byte.
__device__ __forceinline__ uint32_t encode_group(const float (&v)[16], uint32_t (&packed)[2])
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sb = group_scale(amax);
    const float s = e4m3_value(sb);
    packed[0] = packed[1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        packed[i / 8] |= e2m1_nibble(v[i], s) << (4 * (i % 8));
    return sb;
}

// Four fp32 values -> four E4M3FN bytes (RNE, saturating, sign kept).
__device__ __forceinline__ uint32_t fp8_word(float4 f)
{
    const float v[4] = {f.x, f.y, f.z, f.w};
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t c = e4m3_rne(fabsf(v[i]));
        if (__float_as_uint(v[i]) >> 31)
            c |= 0x80u;
        word |= c << (8 * i);
    }
    return word;
}

// Thread t of a group-per-thread launch: group g of row r of a [rows, C] input,
// written to row orow of the outputs: row-major codes, or the tiled
// indexer-key layout when C is the indexer-key width.
__device__ __forceinline__ void encode_row_group(const float* __restrict__ x, int64_t r,
                                                 int32_t g, int32_t C,
                                                 const float* __restrict__ cs,
                                                 const float* __restrict__ sn, int32_t rope_off,
                                                 int32_t rope_dim, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, int64_t orow)
{
    const float4* src = reinterpret_cast<const float4*>(x + r * C + 16 * g);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 f = src[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
    rope_group(v, g, r, cs, sn, rope_off, rope_dim);
    uint32_t packed[2];
    const uint32_t sb = encode_group(v, packed);
    // bytes [8g, 8g + 8) of the row: one aligned 8-byte store in either layout
    const int64_t co = C == kIdxDim ? key_code_offset(orow, 8 * g) : orow * (C / 2) + 8 * g;
    *reinterpret_cast<uint2*>(codes + co) = make_uint2(packed[0], packed[1]);
    scales[orow * (C / 16) + g] = (uint8_t)sb;
}

__global__ void __launch_bounds__(256)
quantize_kv_kernel(const float* __restrict__ x, int64_t rows, int32_t C,
                   const float* __restrict__ cs, const float* __restrict__ sn, int32_t rope_off,
                   int32_t rope_dim, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                   int64_t dst_row, int64_t dst_stride)
{
    const int32_t G = C / 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * G)
        return;
    encode_row_group(x, t / G, (int32_t)(t % G), C, cs, sn, rope_off, rope_dim, codes, scales,
                     dst_row + (t / G) * dst_stride);
}

// Four consecutive elements per thread; row_len % 4 == 0.
__global__ void __launch_bounds__(256)
quantize_swa_kernel(const float* __restrict__ x, int64_t n, int32_t row_len,
                    uint8_t* __restrict__ out, int64_t dst_stride)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (4 * t >= n)
        return;
    const uint32_t word = fp8_word(reinterpret_cast<const float4*>(x)[t]);
    const int64_t e = 4 * t;
    const int64_t r = e / row_len;
    const int64_t c = e % row_len;
    *reinterpret_cast<uint32_t*>(out + r * dst_stride * row_len + c) = word;
}

// New cache entries of one step in one launch ([A] 3.3: a Full layer computes
// the main KV and projects the indexer key from it; [N] 2.2: the indexer key
// is now projected from the main KV; [N] 2.3: window rows stay FP8).
// Workgroups [0, wg_kv) encode the main-KV rows (rotary + MXFP4, one thread per
// 16-channel group); [wg_kv, wg_kv + wg_idx) the indexer-key rows, either from
// their own fp32 rows (one thread per group) or projected from the main
// latent before its rotary (one workgroup per row: wave q sums channels
// [128q, 128q+128) for every output in four fixed-order partial sums of fp32
// fused multiply-adds (channel c to partial c % 4, in increasing c), adds
// them (p0 + p1) + (p2 + p3), the four quarters are added (q0 + q1) + (q2 + q3),
// and wave 0 encodes the row, lane l holding channels 2l and 2l+1, a group of
// 16 channels being 8 lanes); the rest encode the window rows.  Row r of the
// caches goes to row kv_dst[r] (else r * stride) and window row r to row
// swa_dst[r] (else r * swa_stride): with per-sequence positions that is each
// sequence's own append position, and for the window a ring slot.  Without
// kv_dst, cache row r goes to dst0 + r * stride.  Indexer-key codes use the
// tiled key layout.
struct EntryJob {
    int32_t rows;
    const float* kv_x; const float* cs; const float* sn; int32_t rope_off, rope_dim;
    uint8_t* kv_codes; uint8_t* kv_scales; int64_t kv_stride;
    const int64_t* kv_dst;   // per-row destination row of the caches, or null
    int64_t dst0;            // without kv_dst: row r goes to dst0 + r * stride
    int64_t kv_cap;          // rows of the caches (destinations outside are skipped)
    const float* idx_x; const uint16_t* w_idx;
    uint8_t* idx_codes; uint8_t* idx_scales; int64_t idx_stride; float* idx_y;
    const float* swa_x; int32_t swa_rows; uint8_t* swa_out; int64_t swa_stride;
    const int64_t* swa_dst;  // per-row destination row of the window buffer, or null
    int64_t swa_cap;         // rows of the window buffer
    int32_t wg_kv, wg_idx;  // workgroups of the first two parts
};

// Destination row of input row r: dst[r] (-1 when outside [0, cap): skipped)
// or dst0 + r * stride.
__device__ __forceinline__ int64_t dst_row(const int64_t* __restrict__ dst, int64_t dst0,
                                           int64_t r, int64_t stride, int64_t cap)
{
    if (dst == nullptr)
        return dst0 + r * stride;
    const int64_t d = dst[r];
    return d >= 0 && d < cap ? d : -1;
}

__device__ __forceinline__ float max8_lanes(float m)
{
    m = fmaxf(m, __uint_as_float(dpp_u32<0xB1>(0u, __float_as_uint(m))));
    m = fmaxf(m, __uint_as_float(dpp_u32<0x4E>(0u, __float_as_uint(m))));
    return fmaxf(m, __uint_as_float(dpp_u32<0x141>(0u, __float_as_uint(m))));
}

__global__ void __launch_bounds__(256)
encode_entries_kernel(EntryJob J)
{
    constexpr int kKv = kDim / 16;       // 32 groups per main-KV row
    constexpr int kIdx = kIdxDim / 16;   // 8 groups per indexer-key row
    constexpr int kSlice4 = kDim / 4;    // projection channels per wave
    const int wg = blockIdx.x;
    if (wg < J.wg_kv) {
        const int64_t t = (int64_t)wg * 256 + threadIdx.x;
        if (t < (int64_t)J.rows * kKv) {
            const int64_t r = t / kKv;
            const int64_t o = dst_row(J.kv_dst, J.dst0, r, J.kv_stride, J.kv_cap);
            if (o >= 0)
                encode_row_group(J.kv_x, r, (int32_t)(t % kKv), kDim, J.cs, J.sn, J.rope_off,
                                 J.rope_dim, J.kv_codes, J.kv_scales, o);
        }
        return;
    }
    if (wg < J.wg_kv + J.wg_idx) {
        const int w = wg - J.wg_kv;
        if (J.idx_x != nullptr) {
            const int64_t t = (int64_t)w * 256 + threadIdx.x;
            if (t < (int64_t)J.rows * kIdx) {
                const int64_t r = t / kIdx;
                const int64_t o = dst_row(J.kv_dst, J.dst0, r, J.idx_stride, J.kv_cap);
                if (o >= 0)
                    encode_row_group(J.idx_x, r, (int32_t)(t % kIdx), kIdxDim, nullptr, nullptr,
                                     0, 0, J.idx_codes, J.idx_scales, o);
            }
            return;
        }
        // projection: one workgroup per row; wave q sums channels [128q, 128q+128) for
        // every output (lane l: outputs 2l, 2l+1), loads one 16-channel step ahead
        __shared__ float part[4][kIdxDim];
        const int lane = threadIdx.x & 63;
        const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int64_t r = w;
        const float4* xr = reinterpret_cast<const float4*>(J.kv_x + r * kDim + kSlice4 * q);
        const uint4* w0 = reinterpret_cast<const uint4*>(J.w_idx + (int64_t)(2 * lane) * kDim +
                                                         kSlice4 * q);
        const uint4* w1 = reinterpret_cast<const uint4*>(J.w_idx + (int64_t)(2 * lane + 1) * kDim +
                                                         kSlice4 * q);
        float p0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, p1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float4 xa[4];
        uint4 wa[2], wb[2];
        auto load = [&](int j) {  // channels 16j .. 16j+15 of the quarter
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xa[i] = xr[4 * j + i];
            wa[0] = w0[2 * j]; wa[1] = w0[2 * j + 1];
            wb[0] = w1[2 * j]; wb[1] = w1[2 * j + 1];
        };
        load(0);
#pragma unroll
        for (int j = 0; j < kSlice4 / 16; ++j) {
            const float xs[16] = {xa[0].x, xa[0].y, xa[0].z, xa[0].w, xa[1].x, xa[1].y, xa[1].z,
                                  xa[1].w, xa[2].x, xa[2].y, xa[2].z, xa[2].w, xa[3].x, xa[3].y,
                                  xa[3].z, xa[3].w};
            const uint32_t da[8] = {wa[0].x, wa[0].y, wa[0].z, wa[0].w, wa[1].x, wa[1].y, wa[1].z, wa[1].w};
            const uint32_t db[8] = {wb[0].x, wb[0].y, wb[0].z, wb[0].w, wb[1].x, wb[1].y, wb[1].z, wb[1].w};
            if (j + 1 < kSlice4 / 16)
                load(j + 1);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float fa = __uint_as_float(i % 2 == 0 ? da[i / 2] << 16 : da[i / 2] & 0xFFFF0000u);
                const float fb = __uint_as_float(i % 2 == 0 ? db[i / 2] << 16 : db[i / 2] & 0xFFFF0000u);
                p0[i % 4] = __builtin_fmaf(xs[i], fa, p0[i % 4]);
                p1[i % 4] = __builtin_fmaf(xs[i], fb, p1[i % 4]);
            }
        }
        part[q][2 * lane] = __fadd_rn(__fadd_rn(p0[0], p0[1]), __fadd_rn(p0[2], p0[3]));
        part[q][2 * lane + 1] = __fadd_rn(__fadd_rn(p1[0], p1[1]), __fadd_rn(p1[2], p1[3]));
        __syncthreads();
        if (q != 0)
            return;
        const float y0 = __fadd_rn(__fadd_rn(part[0][2 * lane], part[1][2 * lane]),
                                   __fadd_rn(part[2][2 * lane], part[3][2 * lane]));
        const float y1 = __fadd_rn(__fadd_rn(part[0][2 * lane + 1], part[1][2 * lane + 1]),
                                   __fadd_rn(part[2][2 * lane + 1], part[3][2 * lane + 1]));
        if (J.idx_y != nullptr)
            *reinterpret_cast<float2*>(J.idx_y + r * kIdxDim + 2 * lane) = make_float2(y0, y1);
        // group of 16 channels = lanes 8g .. 8g+7
        const float amax = max8_lanes(fmaxf(fabsf(y0), fabsf(y1)));
        const uint32_t sb = group_scale(amax);
        const float sv = e4m3_value(sb);
        const int64_t orow = dst_row(J.kv_dst, J.dst0, r, J.idx_stride, J.kv_cap);
        if (orow < 0)
            return;
        J.idx_codes[key_code_offset(orow, lane)] =
            (uint8_t)(e2m1_nibble(y0, sv) | (e2m1_nibble(y1, sv) << 4));
        if ((lane & 7) == 0)
            J.idx_scales[orow * kIdx + lane / 8] = (uint8_t)sb;
        return;
    }
    const int64_t t = (int64_t)(wg - J.wg_kv - J.wg_idx) * 256 + threadIdx.x;
    if (4 * t >= (int64_t)J.swa_rows * kDim)
        return;
    const uint32_t word = fp8_word(reinterpret_cast<const float4*>(J.swa_x)[t]);
    const int64_t r = 4 * t / kDim, c = 4 * t % kDim;
    const int64_t o = dst_row(J.swa_dst, 0, r, J.swa_stride, J.swa_cap);
    if (o >= 0)
        *reinterpret_cast<uint32_t*>(J.swa_out + o * kDim + c) = word;
}

}  // namespace

namespace {

// Workgroups of the encoding launches (256 threads each): one thread per
// 16-channel MXFP4 group, per 4 window bytes, and for the one-launch encoder
// the sum of its three parts.
int64_t quantize_kv_workgroups(int64_t rows, int32_t channels)
{
    return (rows * (channels / 16) + 255) / 256;
}

int64_t quantize_swa_workgroups(int64_t n)
{
    return (n / 4 + 255) / 256;
}

struct EntryGrid {
    int64_t kv, idx, swa;
};

EntryGrid encode_entries_grid(int32_t rows, bool idx_rows_given, int32_t swa_rows)
{
    return {((int64_t)rows * (kDim / 16) + 255) / 256,
            idx_rows_given ? ((int64_t)rows * (kIdxDim / 16) + 255) / 256 : (int64_t)rows,
            ((int64_t)swa_rows * (kDim / 4) + 255) / 256};
}

}  // namespace

bool quantize_kv_fits(int64_t rows, int32_t channels)
{
    // rows first: the product of a larger count would overflow
    return rows <= kMaxWorkItems && grid_fits(quantize_kv_workgroups(rows, channels), 256);
}

bool quantize_swa_fits(int64_t n)
{
    return grid_fits(quantize_swa_workgroups(n), 256);
}

bool encode_entries_fits(int32_t rows, bool idx_rows_given, int32_t swa_rows)
{
    const EntryGrid g = encode_entries_grid(rows, idx_rows_given, swa_rows);
    return grid_fits(g.kv + g.idx + g.swa, 256);
}

hipError_t launch_quantize_kv(const float* x, int64_t rows, int32_t channels, const float* cs,
                              const float* sn, int32_t rope_off, int32_t rope_dim, uint8_t* codes,
                              uint8_t* scales, int64_t dst_row, int64_t dst_stride,
                              hipStream_t stream)
{
    if (!quantize_kv_fits(rows, channels))
        return hipErrorInvalidConfiguration;
    const int64_t grid = quantize_kv_workgroups(rows, channels);
    if (grid == 0)
        return hipSuccess;
    quantize_kv_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(
        x, rows, channels, cs, sn, rope_off, rope_dim, codes, scales, dst_row, dst_stride);
    return hipGetLastError();
}

hipError_t launch_quantize_swa(const float* x, int64_t n, int32_t row_len, uint8_t* out,
                               int64_t dst_stride, hipStream_t stream)
{
    const int64_t grid = quantize_swa_workgroups(n);
    if (grid == 0)
        return hipSuccess;
    if (!grid_fits(grid, 256))
        return hipErrorInvalidConfiguration;
    quantize_swa_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(x, n, row_len, out,
                                                                        dst_stride);
    return hipGetLastError();
}


hipError_t launch_encode_entries(int32_t rows, const float* kv_x, const float* cs, const float* sn,
                                 int32_t rope_off, int32_t rope_dim, uint8_t* kv_codes,
                                 uint8_t* kv_scales, int64_t kv_stride, const int64_t* kv_dst,
                                 int64_t dst_row, int64_t kv_cap, const float* idx_x,
                                 const uint16_t* w_idx, uint8_t* idx_codes, uint8_t* idx_scales,
                                 int64_t idx_stride, float* idx_y, const float* swa_x,
                                 int32_t swa_rows, uint8_t* swa_out, int64_t swa_stride,
                                 const int64_t* swa_dst, int64_t swa_cap, hipStream_t stream)
{
    EntryJob J{rows, kv_x, cs, sn, rope_off, rope_dim, kv_codes, kv_scales, kv_stride, kv_dst,
               dst_row, kv_cap, idx_x, w_idx, idx_codes, idx_scales, idx_stride, idx_y,
               swa_x, swa_rows, swa_out, swa_stride, swa_dst, swa_cap, 0, 0};
    const EntryGrid eg = encode_entries_grid(rows, idx_x != nullptr, swa_rows);
    const int64_t grid = eg.kv + eg.idx + eg.swa;
    if (grid == 0)
        return hipSuccess;
    if (!grid_fits(grid, 256))
        return hipErrorInvalidConfiguration;
    J.wg_kv = (int32_t)eg.kv;
    J.wg_idx = (int32_t)eg.idx;
    encode_entries_kernel<<<dim3((uint32_t)grid), dim3(256), 0, stream>>>(J);
    return hipGetLastError();
}

}  // namespace csa2
