// Sparse MLA attention over the selected MXFP4 main-KV entries plus the FP8
// sliding window ([N] 1 of the DeepSeek-V4.1 reading notes: 64 query heads x
// 512; [S] "DeepSeek-V4 model structure (7)": K = V single-head MQA on the
// 512-dim latent, top-k compressed entries plus 128 window entries).  One
// joint softmax over both key sets; no de-duplication; no sink.
//
// One decomposition.  A workgroup of eight waves serves one query row and a
// group of 16, 32 or 64 heads (more heads for more rows); K = V is one latent
// shared by every head, so a key is fetched and dequantised once per group
// (once per row with 64 heads).  Wave w owns the channels [64w, 64w+64) of
// the latent.  Keys go in tiles of 32 (64 with 32 heads).  Per tile:
//   1. every wave dequantises its 64 channels of the tile's keys exactly to fp16,
//      straight into the MFMA operand, stores them row-major to its own LDS
//      V tile and forms the partial S^T over its channels for all the
//      group's heads (v_mfma_f32_16x16x32_f16, Q^T held in registers);
//   2. the eight partials meet in LDS (barrier); each wave owns the softmax
//      of one eighth of the heads: it adds the partials in wave order, runs
//      the online softmax in the log2 domain and writes P, split into two
//      fp16 terms (hi + lo, so P V keeps ~22 bits of P), and each head's
//      rescale factor (barrier);
//   3. every wave rescales its output accumulators and adds V^T P^T for its
//      64 dims of all the group's heads, V^T read from its own LDS tile with
//      the gfx950 transposing read.
// A head's arithmetic depends on the tile size only, so the 16- and 64-head
// forms give bit-identical outputs.  For few rows (decode) the keys are also
// split over workgroups and a second, short kernel merges the splits.
//
// Channel order inside the MFMAs: lane group G = l/16 of wave w holds the
// channels [64w + 16G, +16) (one scale block of the MXFP4 entry); k-step t
// takes the eight channels 64w + 16G + 8t .. +8, for the keys (A operand) and
// the query (B operand) alike.
//   S^T accumulator (kb, hb): lane l holds head 16hb + l%16 and the keys
//     16kb + 4G + r (r < 4) of the tile;
//   P^T operand (B of O^T = V^T P^T), k-step ks of 32 keys: MFMA k-index
//     8G + i <-> key 32ks + 16(i/4) + 4G + i%4, head l%16;
//   V^T[16 dims x 32 keys] (A operand): from the row-major LDS tile with
//     ds_read_b64_tr_b16 (within each 16-lane group, lane 4a + j receives
//     element j of lanes a, a+4, a+8, a+12), two reads per MFMA, in the same
//     key order;
//   loads are unconditional (clamped inside the list or pointed at the query
//     row, masked afterwards), so the load counter stays exact; the top-k
//     indices are loaded ahead of the keys they address.
// The running maximum of each head moves lazily (kMaxSlack below), so a tile
// whose keys do not raise any head's maximum much costs no rescale.
#include "device_common.h"
#include "launch.h"

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((vector_size(8)));  // operand type of the LDS transposing read
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int kTile = 32;                       // keys per MFMA k-step of P V (two blocks of 16)
constexpr int kHg = 16;                         // heads per record of the split partials
constexpr int kGroups = kHeads / kHg;           // 4 such records per row
constexpr int kWaves = 8;                       // waves per workgroup
constexpr int kCh = kDim / kWaves;              // 64 channels / output dims per wave
constexpr int kVRow = kCh + 8;                  // halves per LDS row of a V tile (144 B)
constexpr int kPRow = 17;                       // 16-byte slots per LDS row of partials / P
constexpr int kXcds = 8;                        // MI355X dies: workgroups go round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// A head's running maximum (log2 domain) moves only when a tile's maximum
// exceeds it by more than this; P then stays <= 2^8, well inside fp16.  Any
// reference point gives the same softmax, and a head whose maximum did not
// move keeps its accumulators untouched (its rescale factor is exactly 1).
constexpr float kMaxSlack = 8.0f;

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int kCtrl>
__device__ __forceinline__ int dpp_i32(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

// Combines v over the lanes whose index differs only in bits [0, log2 kC),
// as a butterfly: level 1 pairs lanes that differ in bit 0, level 2 the pairs
// that differ in bit 1, and so on (the mirror patterns stand in for the xor
// partner once each lower group holds one value; the last level takes both
// 16-lane rows of a pair from v_permlane16_swap), so every lane ends with the
// same result and the order of a sum is fixed by the lane bits.
template <int kC, typename T, typename Op>
__device__ __forceinline__ T lane_reduce(T v, Op op)
{
    if constexpr (kC >= 2)
        v = op(v, dpp_i32<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (kC >= 4)
        v = op(v, dpp_i32<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (kC >= 8)
        v = op(v, dpp_i32<0x141>(v));   // row_half_mirror: the other quad of the 8
    if constexpr (kC >= 16)
        v = op(v, dpp_i32<0x140>(v));   // row_mirror: the other 8 of the row
    if constexpr (kC >= 32) {           // rows 2r and 2r+1 swapped: (row 2r, row 2r+1)
        const auto r = __builtin_amdgcn_permlane16_swap((int)v, (int)v, false, false);
        v = op((int)r[0], (int)r[1]);
    }
    static_assert(kC <= 32, "reductions span at most 32 lanes");
    return v;
}

// Maximum and sum of a float over the lanes of lane_reduce.  The maximum runs
// on order-preserving integer keys (a float's bits with the magnitude bits
// flipped when negative), so each level is one integer max with its DPP
// source; the sum adds the floats' bit patterns moved as integers.
template <int kC>
__device__ __forceinline__ float lane_max(float v)
{
    int x = __float_as_int(v);
    x ^= (x >> 31) & 0x7FFFFFFF;
    x = lane_reduce<kC>(x, [](int a, int b) { return max(a, b); });
    x ^= (x >> 31) & 0x7FFFFFFF;
    return __int_as_float(x);
}

template <int kC>
__device__ __forceinline__ float lane_sum(float v)
{
    const int x = lane_reduce<kC>(__float_as_int(v), [](int a, int b) {
        return __float_as_int(__int_as_float(a) + __int_as_float(b));
    });
    return __int_as_float(x);
}

// Where the output goes: fp32 as computed, or (kRopeBf16) inverse rotary on
// the rotary channels followed by a bf16 cast.
struct AttnOut {
    float* out;            // fp32 [rows, 64, 512] (kRopeBf16 = false)
    uint16_t* out_bf16;    // bf16 [rows, 64, 512] (kRopeBf16 = true)
    const float* cs;       // [rows, rope_dim/2]: the query position's angles
    const float* sn;
    int32_t rope_off, rope_dim;
};

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}


// ============================================================= the kernel

#ifndef CSA2_ATTN_DEPTH
#define CSA2_ATTN_DEPTH 2
#endif
constexpr int kDepth = CSA2_ATTN_DEPTH;          // tiles in flight per wave
#ifndef CSA2_ATTN_SPLIT_WGS
#define CSA2_ATTN_SPLIT_WGS 256
#endif
constexpr int64_t kSplitWgs = CSA2_ATTN_SPLIT_WGS;  // workgroup budget of the key splits
constexpr int kMaxSplits = 8;                   // key splits per (row, head group)
#ifndef CSA2_ATTN_MIN_SPLIT_TILES
#define CSA2_ATTN_MIN_SPLIT_TILES 2
#endif
constexpr int kMinSplitTiles = CSA2_ATTN_MIN_SPLIT_TILES;  // fewest 32-key tiles per split
constexpr int kPartFloats = kHg * kDim + 2 * kHg;  // one split's O [16][512], max, sum

// Who owns which scores in the softmax step, for kHW heads per workgroup and
// tiles of kKB blocks of 16 keys: wave w owns heads w*kHpw + hl (hl < kHpw);
// lane l = c + kC*hl takes kNv consecutive keys of its head,
// c = rl + kR*(G' + 4kb) naming the keys 16kb + 4G' + kNv*rl + e (e < kNv).
// The lane bits of c order the key index bits from r upwards, so the sum
// over a head's keys adds them in the same tree for every kHW of a tile size.
template <int kHW, int kKB>
struct Owner {
    static constexpr int kHB = kHW / 16;          // MFMA head blocks
    static constexpr int kHpw = kHW / kWaves;     // heads per wave: 2, 4, 8
    static constexpr int kNv = kKB * kHW / 32;    // keys per lane
    static constexpr int kC = kWave / kHpw;       // lanes per head: 32, 16, 8
    static constexpr int kR = 4 / kNv;            // lanes per 4 keys
    static_assert(kNv >= 1 && kNv <= 4 && kR * 4 * kKB == kC, "owner layout");
};

template <int kHW, int kKB>
struct Smem {
    _Float16 v[kWaves][16 * kKB][kVRow];          // each wave's V tile (its 64 dims)
    // partial S^T: [wave][head block][4kb + G][head%16 (+1 pad slot)][4 keys];
    // a lane's 16-byte store is contiguous with its neighbours', and the
    // owners' reads of one head spread over the padded rows
    f32x4 part[kWaves][kHW / 16][4 * kKB][kPRow];
    // P^T operand, hi and lo: [k-step of 32 keys][hb][G][head%16 (+pad)][8 keys
    // in MFMA k-order]
    half8 p[2][kKB / 2][kHW / 16][4][kPRow];
    float alpha[kHW];                             // each head's rescale factor of the tile
    float lsum[kHW];                              // each head's final sum
    float qmax[kWaves][kHW];                      // largest |q| of each head over each wave's channels
};

// Raw bytes of one tile for the calling lane, for key l%16 of block kb: top-k
// tile: a = the 8 code bytes of channels [64w + 16G, +16), s = the 8 scale
// bytes 8(w/2) .. +8 of the entry (byte 4(w%2) + G is this lane's); window
// tile: a, s = the 16 E4M3 bytes of those channels.
template <int kKB>
struct TileRaw {
    uint2 a[kKB], s[kKB];
    uint32_t valid;  // bit kb: key of block kb is valid
};

// Partial S^T of one tile over the wave's 64 channels (s[kb][hb]); the
// dequantised keys also go to the wave's LDS tile.  kMain: MXFP4 top-k keys,
// else E4M3 window rows.
template <bool kMain, int kHB, int kKB>
__device__ __forceinline__ void tile_scores(const TileRaw<kKB>& R, const half8 (&qop)[kHB][2],
                                            _Float16* __restrict__ vtile, int wave, int G,
                                            int key16, f32x4 (&s)[kKB][kHB])
{
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
        const bool ok = (R.valid >> kb) & 1u;
        half8 a[2];
        if (kMain) {
            const uint32_t sdw = (wave & 1) ? R.s[kb].y : R.s[kb].x;
            const _Float16 sc = e4m3_byte_to_f16(ok ? sdw >> (8 * G) : 0u, 0);
            a[0] = dequant8_fp4(ok ? R.a[kb].x : 0u, sc);
            a[1] = dequant8_fp4(ok ? R.a[kb].y : 0u, sc);
        } else {
            const uint32_t w0 = ok ? R.a[kb].x : 0u, w1 = ok ? R.a[kb].y : 0u;
            const uint32_t w2 = ok ? R.s[kb].x : 0u, w3 = ok ? R.s[kb].y : 0u;
            const half4v x0 = e4m3x4_to_f16(w0), x1 = e4m3x4_to_f16(w1);
            const half4v x2 = e4m3x4_to_f16(w2), x3 = e4m3x4_to_f16(w3);
            a[0] = half8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            a[1] = half8{x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
        }
        f32x4 acc[kHB];
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb)
            acc[hb] = f32x4{};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int hb = 0; hb < kHB; ++hb)
                acc[hb] = mfma16(a[t], qop[hb][t], acc[hb]);
            *reinterpret_cast<half8*>(vtile + (16 * kb + key16) * kVRow + 16 * G + 8 * t) = a[t];
        }
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb)
            s[kb][hb] = acc[hb];
    }
}

// Writes this lane's outputs (head `head`, dims 64*wave + 16db + 4G + r) as
// o * inv, through the epilogue of kRopeBf16.
template <bool kRopeBf16>
__device__ __forceinline__ void emit(const f32x4 (&o)[kCh / 16], float inv, int64_t qrow,
                                     int head, int wave, int G, const AttnOut& dst)
{
    const int64_t base = (qrow * kHeads + head) * kDim + kCh * wave + 4 * G;
#pragma unroll
    for (int db = 0; db < kCh / 16; ++db) {
        float res[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            res[r] = o[db][r] * inv;
        if (!kRopeBf16) {
            *reinterpret_cast<float4*>(dst.out + base + 16 * db) =
                make_float4(res[0], res[1], res[2], res[3]);
        } else {
            // rotate each rotary pair (a, b) back by the query's angle:
            // a' = a*c + b*s, b' = b*c - a*s, every product and sum rounded to fp32
            const int half = dst.rope_dim / 2;
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const int d = kCh * wave + 16 * db + 4 * G + i;
                if (d >= dst.rope_off && d < dst.rope_off + dst.rope_dim) {
                    const int pi = (d - dst.rope_off) / 2;
                    const float c = dst.cs[qrow * half + pi];
                    const float sn = dst.sn[qrow * half + pi];
                    const float a = res[i], bb = res[i + 1];
                    res[i] = __fadd_rn(__fmul_rn(a, c), __fmul_rn(bb, sn));
                    res[i + 1] = __fsub_rn(__fmul_rn(bb, c), __fmul_rn(a, sn));
                }
            }
            const uint32_t p0 = (uint32_t)bf16_rne(res[0]) | ((uint32_t)bf16_rne(res[1]) << 16);
            const uint32_t p1 = (uint32_t)bf16_rne(res[2]) | ((uint32_t)bf16_rne(res[3]) << 16);
            *reinterpret_cast<uint2*>(dst.out_bf16 + base + 16 * db) = make_uint2(p0, p1);
        }
    }
}

constexpr int kSlice = 128;                     // dims per merge workgroup
constexpr int kSlices = kDim / kSlice;          // 4 merge workgroups per 16 heads

constexpr int kBufferConfig = 0x00020000;  // raw (untyped) buffer, 32-bit data
constexpr int kCachePolicy = 0;            // plain loads (the partials of the previous kernel)
constexpr int kWriteThrough = 17;          // sc0 | sc1 stores: written through to memory

// The key-split partials of (row, head group): splits x kPartFloats floats.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* part, int64_t qrow, int hg,
                                                            int32_t splits)
{
    return __builtin_amdgcn_make_buffer_rsrc(part + (qrow * kGroups + hg) * splits * kPartFloats,
                                             0, splits * kPartFloats * 4, kBufferConfig);
}

// Merge of the key splits of one (row, head group) over one 128-dim slice, by
// 256 threads: thread t takes head t/16 and the 8 dims 8*(t%16) .. +8 of the
// slice.  Every split's (max, sum, 8 outputs) is loaded first (slots past
// `splits` repeat the last split and are ignored), then they are combined in
// split order (deterministic) and written through the epilogue.
template <bool kRopeBf16>
__device__ __forceinline__ void merge_slice(__amdgpu_buffer_rsrc_t rs, int32_t splits,
                                            int64_t qrow, int hg, int slice, int t,
                                            const AttnOut& dst, float* __restrict__ lse)
{
    const int h = t / 16;
    const int d0 = kSlice * slice + 8 * (t % 16);
    float ms[kMaxSplits], ls[kMaxSplits];
    u32x4 va[kMaxSplits], vb[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        const int32_t ps = (s < splits ? s : splits - 1) * kPartFloats;
        ms[s] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (ps + kHg * kDim + h), 0, kCachePolicy));
        ls[s] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rs, 4 * (ps + kHg * kDim + kHg + h), 0, kCachePolicy));
        va[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (ps + h * kDim + d0), 0, kCachePolicy);
        vb[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (ps + h * kDim + d0 + 4), 0,
                                                      kCachePolicy);
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        M = s < splits ? fmaxf(M, ms[s]) : M;
    float den = 0.0f;
    float num[8] = {};
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        if (s < splits) {
            const float f = ms[s] == -INFINITY ? 0.0f : exp2f(ms[s] - M);
            den += f * ls[s];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                num[i] += f * __uint_as_float(va[s][i]);
                num[4 + i] += f * __uint_as_float(vb[s][i]);
            }
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    float res[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        res[i] = num[i] * inv;
    const int head = kHg * hg + h;
    const int64_t o0 = (qrow * kHeads + head) * kDim + d0;
    if (!kRopeBf16) {
        float4* o = reinterpret_cast<float4*>(dst.out + o0);
        o[0] = make_float4(res[0], res[1], res[2], res[3]);
        o[1] = make_float4(res[4], res[5], res[6], res[7]);
    } else {
        // rotate each rotary pair (a, b) back by the query's angle:
        // a' = a*c + b*s, b' = b*c - a*s, every product and sum rounded to fp32
        const int half = dst.rope_dim / 2;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const int d = d0 + i;
            if (d >= dst.rope_off && d < dst.rope_off + dst.rope_dim) {
                const int pi = (d - dst.rope_off) / 2;
                const float c = dst.cs[qrow * half + pi];
                const float sn = dst.sn[qrow * half + pi];
                const float a = res[i], bb = res[i + 1];
                res[i] = __fadd_rn(__fmul_rn(a, c), __fmul_rn(bb, sn));
                res[i + 1] = __fsub_rn(__fmul_rn(bb, c), __fmul_rn(a, sn));
            }
        }
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = (uint32_t)bf16_rne(res[2 * i]) | ((uint32_t)bf16_rne(res[2 * i + 1]) << 16);
        uint2* o = reinterpret_cast<uint2*>(dst.out_bf16 + o0);
        o[0] = make_uint2(w[0], w[1]);
        o[1] = make_uint2(w[2], w[3]);
    }
    if (lse != nullptr && slice == 0 && t % 16 == 0)
        lse[qrow * kHeads + head] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}


#ifndef CSA2_ATTN_WAVES_PER_EU
#define CSA2_ATTN_WAVES_PER_EU 2
#endif
// Query rows from which a workgroup takes 64 heads (one per row) or 32 heads:
// below them, fewer, larger workgroups would leave CUs idle.
#ifndef CSA2_ATTN_HW64_MIN_ROWS
#define CSA2_ATTN_HW64_MIN_ROWS 256
#endif
#ifndef CSA2_ATTN_HW32_MIN_ROWS
#define CSA2_ATTN_HW32_MIN_ROWS 128
#endif
constexpr int32_t kHw64MinRows = CSA2_ATTN_HW64_MIN_ROWS;
constexpr int32_t kHw32MinRows = CSA2_ATTN_HW32_MIN_ROWS;
// Blocks of 16 keys per tile.  64-key tiles halve the barriers and
// reductions per key: with 32 heads (128 to 255 rows) they measured faster;
// with 16 heads the key splits of few rows then get too few tiles each, and
// with 64 heads only 32-key tiles fit the LDS.
#ifndef CSA2_ATTN_KB16
#define CSA2_ATTN_KB16 2
#endif
#ifndef CSA2_ATTN_KB32
#define CSA2_ATTN_KB32 4
#endif
template <int kHW>
constexpr int kKbOf = kHW == 16 ? CSA2_ATTN_KB16 : (kHW == 32 ? CSA2_ATTN_KB32 : 2);

// One workgroup per (query row, group of kHW heads, key split); tiles of kKB
// blocks of 16 keys.
template <bool kRopeBf16, int kHW, int kKB>
__global__ void __launch_bounds__(kWaves * kWave)
__attribute__((amdgpu_waves_per_eu(CSA2_ATTN_WAVES_PER_EU)))
attn_kernel(const uint16_t* __restrict__ q, int32_t queries,
            const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales,
            int64_t n_cap, int32_t nq, const int32_t* __restrict__ topk, int32_t k,
            const uint8_t* __restrict__ swa, int32_t swa_cap,
            const int32_t* __restrict__ swa_end, int32_t n_win, float scale_log2,
            int32_t splits, float* __restrict__ part, AttnOut dst_spec,
            float* __restrict__ lse)
{
    using O = Owner<kHW, kKB>;
    constexpr int kHB = O::kHB;
    constexpr int kT = 16 * kKB;      // keys per tile
    __shared__ Smem<kHW, kKB> sm;
    const int lane = threadIdx.x & 63;
    // the wave index as a scalar: everything derived from it (pointers,
    // offsets) stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = lane >> 4;
    const int key16 = lane & 15;

    // the workgroups of a query row (head groups x splits) share one die (and
    // its L2, which then serves the keys to every group): with round-robin
    // dispatch, workgroup x runs on die x % 8
    constexpr int kWgGroups = kHeads / kHW;  // workgroups per row and split
    const int wg_per_row = kWgGroups * splits;
    const int64_t x = blockIdx.x;
    const int64_t rest = x / kXcds;
    const int64_t qrow = kXcds * (rest / wg_per_row) + x % kXcds;
    const int head0 = ((int)(rest % wg_per_row) % kWgGroups) * kHW;  // first head of the group
    const int split = (int)(rest % wg_per_row) / kWgGroups;
    if (qrow >= queries)
        return;
    const int64_t b = qrow / nq;

    // this lane's softmax share: head hw (of the group), keys 16kb + 4Gs + kNv*rl + e
    const int c = lane % O::kC;
    const int hw = wave * O::kHpw + lane / O::kC;
    const int rl = c % O::kR;
    const int Gs = (c / O::kR) & 3;
    const int kbs = c / (4 * O::kR);

    // tile list: top-k tiles [0, t_main), then window tiles; this workgroup
    // takes the list positions split + splits * j
    const int t_main = n_cap > 0 ? (k + kT - 1) / kT : 0;
    auto pos = [&](int j) { return split + splits * j; };

    // loads with no data to fetch read the query row (64 KiB, always valid)
    // and are masked, so every load is unconditional
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(q + qrow * kHeads * kDim);
    const uint8_t* kc = t_main > 0 ? kv_codes + b * n_cap * (kDim / 2) : dummy;
    const uint8_t* ks = t_main > 0 ? kv_scales + b * n_cap * (kDim / 16) : dummy;
    const int32_t* tk = t_main > 0 ? topk + qrow * k : reinterpret_cast<const int32_t*>(dummy);

    // top-k index of this lane's key in block kb of tile p (any valid slot
    // when p is not a top-k tile)
    auto load_idx = [&](int p, int32_t (&e)[kKB]) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const int slot = p * kT + 16 * kb + key16;
            e[kb] = tk[t_main > 0 ? (uint32_t)min(slot, k - 1) : 0u];
        }
    };
    int32_t eidx[kDepth][kKB];
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
        load_idx(pos(u), eidx[u]);
    // Q^T operand: head head0 + 16hb + l%16, channels 64w + 16G + 8t .. +8 (bf16)
    uint4 qraw[kHB][2];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
        const uint4* src = reinterpret_cast<const uint4*>(
            q + (qrow * kHeads + head0 + 16 * hb + key16) * kDim + kCh * wave + 16 * G);
        qraw[hb][0] = src[0];
        qraw[hb][1] = src[1];
    }

    // window rows [lo, hi)
    const int end = swa_end[qrow];
    const int lo = max(end - n_win, 0);
    const int hi = max(min(end, swa_cap), lo);
    const int n_sw = hi - lo;
    const int t_sw = (n_sw + kT - 1) / kT;
    const uint8_t* sw = n_sw > 0 ? swa + b * (int64_t)swa_cap * kDim : dummy;
    const int n_tiles = t_main + t_sw;
    const int n_j = split < n_tiles ? (n_tiles - split + splits - 1) / splits : 0;

    // raw bytes of tile p; tiles past the list load valid rows and are
    // masked.  The tile kind picks a base (the same for the whole wave) and
    // a row stride; each lane adds a 32-bit offset (entry ids are below
    // n_cap <= 2^24, so id * 256 fits), so the loads stay outside any branch.
    const uint8_t* const kc_w = kc + 32 * wave;  // the wave's code bytes of entry 0
    const uint8_t* const ks_w = ks + 8 * (wave >> 1);
    const uint8_t* const sw_w = sw + kCh * wave;
    const uint32_t lane_code = 8 * G, lane_win = 16 * G;
    const uint32_t win_row0 = n_sw > 0 ? (uint32_t)lo : 0u;  // a valid row
    auto load_tile = [&](int p, const int32_t (&e)[kKB], TileRaw<kKB>& R) {
        const bool is_main = p < t_main;
        const int tw = p - t_main;
        const uint8_t* ba = is_main ? kc_w : sw_w;
        const uint8_t* bs = is_main ? ks_w : sw_w + 8;
        const uint32_t stride_a = is_main ? kDim / 2 : kDim;
        const uint32_t stride_s = is_main ? kDim / 16 : kDim;
        const uint32_t lane_a = is_main ? lane_code : lane_win;
        const uint32_t lane_s = is_main ? 0u : lane_win;
        R.valid = 0;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
            const int slot = p * kT + 16 * kb + key16;
            const bool ok_m = slot < k && (uint32_t)e[kb] < (uint32_t)n_cap;
            const int r = lo + tw * kT + 16 * kb + key16;
            const bool ok_w = tw >= 0 && tw < t_sw && r < hi;
            const bool ok = is_main ? ok_m : ok_w;
            const uint32_t row = ok ? (is_main ? (uint32_t)e[kb] : (uint32_t)r)
                                    : (is_main ? 0u : win_row0);
            R.a[kb] = *reinterpret_cast<const uint2*>(ba + (row * stride_a + lane_a));
            R.s[kb] = *reinterpret_cast<const uint2*>(bs + (row * stride_s + lane_s));
            R.valid |= ok ? (1u << kb) : 0u;
        }
    };

    TileRaw<kKB> ring[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
        load_tile(pos(u), eidx[u], ring[u]);
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
        load_idx(pos(u + kDepth), eidx[u]);

    // Each head's query is scaled by a power of two bringing its largest |q| into
    // [2^14, 2^15), so the bf16 -> fp16 cast is exact for every value within 2^28 of
    // it and never overflows; the head's score scale takes the inverse power.  A
    // power of two scales every product and partial sum exactly, so the scores are
    // those of the unscaled query.  The largest |q| of a head spans the eight
    // waves' channels: one exchange through LDS.
    auto shift_of = [&](int h) {
        float m = sm.qmax[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            m = fmaxf(m, sm.qmax[w][h]);
        int sh = 0;  // 0 for an all-zero head
        if (m > 0.0f && !__builtin_isinf(m) && !__builtin_isnan(m)) {
            sh = 14 - ((int)((__float_as_uint(m) >> 23) & 0xFF) - 127);
            sh = sh < -100 ? -100 : (sh > 100 ? 100 : sh);
        }
        return sh;
    };
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t d[4] = {qraw[hb][t].x, qraw[hb][t].y, qraw[hb][t].z, qraw[hb][t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                m = fmaxf(m, fabsf(__uint_as_float(d[i] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(d[i] & 0xFFFF0000u)));
            }
        }
        m = fmaxf(m, __shfl_xor(m, 16, kWave));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        if (lane < 16)
            sm.qmax[wave][16 * hb + lane] = m;
    }
    __syncthreads();
    half8 qop[kHB][2];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
        const int sh = shift_of(16 * hb + key16);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t d[4] = {qraw[hb][t].x, qraw[hb][t].y, qraw[hb][t].z, qraw[hb][t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qop[hb][t][2 * i] = (_Float16)ldexpf(__uint_as_float(d[i] << 16), sh);
                qop[hb][t][2 * i + 1] = (_Float16)ldexpf(__uint_as_float(d[i] & 0xFFFF0000u), sh);
            }
        }
    }
    // the owned head's score scale (scale_log2 * 2^-shift)
    const float own_scale = ldexpf(scale_log2, -shift_of(hw));
    float own_m = -INFINITY, own_l = 0.0f;  // the owned head's running max and sum

    f32x4 o[kHB][kCh / 16];  // O^T: head 16hb + l%16, dims 64w + 16db + 4G + r
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
        for (int db = 0; db < kCh / 16; ++db)
            o[hb][db] = f32x4{};
    _Float16* vtile = &sm.v[wave][0][0];
    const float* own_part =
        reinterpret_cast<const float*>(&sm.part[0][hw / 16][4 * kbs + Gs][hw % 16]) + O::kNv * rl;
    constexpr int kPartWaveFloats = kHB * 4 * kKB * kPRow * 4;  // floats per wave of partials
    // P slot of the owned keys: k-step kbs/2, keys 4(kbs%2) + kNv*rl .. of the lane's 8
    _Float16* own_p = reinterpret_cast<_Float16*>(&sm.p[0][kbs / 2][hw / 16][Gs][hw % 16]) +
                      4 * (kbs % 2) + O::kNv * rl;
    constexpr int kPHalves = (kKB / 2) * kHB * 4 * kPRow * 8;  // halves from hi to lo

    // slot u of the ring holds the tile of step j0 + u; after use it is refilled
    // with the tile of step j + kDepth, and its index slot with the indices of
    // step j + 2*kDepth
    for (int j0 = 0; j0 < n_j; j0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int j = j0 + u;
            const int p = pos(j);
            if (j < n_j) {  // the same for every wave: the barriers below are uniform
                // 1. partial scores over this wave's channels
                f32x4 s[kKB][kHB];
                if (p < t_main)
                    tile_scores<true, kHB, kKB>(ring[u], qop, vtile, wave, G, key16, s);
                else
                    tile_scores<false, kHB, kKB>(ring[u], qop, vtile, wave, G, key16, s);
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
                    for (int hb = 0; hb < kHB; ++hb)
                        sm.part[wave][hb][4 * kb + G][key16] = s[kb][hb];
                // the tile's valid keys (bit 16kb + i), the same in every wave
                uint64_t vmask = 0;
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb)
                    vmask |= (__ballot(((ring[u].valid >> kb) & 1u) != 0u) & 0xFFFFull) << (16 * kb);
                __syncthreads();

                // 2. the owned head's scores: partials added in wave order
                // (in wave order: a tree here measured 20 % slower with 64 heads)
                float sc[O::kNv];
#pragma unroll
                for (int e = 0; e < O::kNv; ++e)
                    sc[e] = own_part[e];
#pragma unroll
                for (int w = 1; w < kWaves; ++w)
#pragma unroll
                    for (int e = 0; e < O::kNv; ++e)
                        sc[e] += own_part[w * kPartWaveFloats + e];
                float tmax = -INFINITY;
#pragma unroll
                for (int e = 0; e < O::kNv; ++e) {
                    const int key = 16 * kbs + 4 * Gs + O::kNv * rl + e;
                    sc[e] = ((vmask >> key) & 1ull) ? sc[e] * own_scale : -INFINITY;
                    tmax = fmaxf(tmax, sc[e]);
                }
                tmax = lane_max<O::kC>(tmax);
                const float m_new = tmax > own_m + kMaxSlack ? tmax : own_m;
                const float alpha = m_new == own_m ? 1.0f : __builtin_amdgcn_exp2f(own_m - m_new);
                float pr[O::kNv];
#pragma unroll
                for (int e = 0; e < O::kNv; ++e)
                    // the hardware exp2 (no subnormal range fix-up): an argument is
                    // at most kMaxSlack, and a result below 2^-126 is lost next to
                    // the head's largest term (at least 1) in every sum and rounds to
                    // zero in the fp16 P pair
                    pr[e] = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[e] - m_new);
                float psum = pr[0];
                if constexpr (O::kNv == 2)
                    psum = pr[0] + pr[1];
                if constexpr (O::kNv == 4)
                    psum = (pr[0] + pr[1]) + (pr[2] + pr[3]);
                psum = lane_sum<O::kC>(psum);
                own_l = own_l * alpha + psum;
                own_m = m_new;
                _Float16 phi[O::kNv], plo[O::kNv];
#pragma unroll
                for (int e = 0; e < O::kNv; ++e) {
                    phi[e] = (_Float16)pr[e];
                    plo[e] = (_Float16)(pr[e] - (float)phi[e]);
                }
                if constexpr (O::kNv == 4) {
                    *reinterpret_cast<half4v*>(own_p) = half4v{phi[0], phi[1], phi[2], phi[3]};
                    *reinterpret_cast<half4v*>(own_p + kPHalves) = half4v{plo[0], plo[1], plo[2], plo[3]};
                } else if constexpr (O::kNv == 2) {
                    *reinterpret_cast<half2v*>(own_p) = half2v{phi[0], phi[1]};
                    *reinterpret_cast<half2v*>(own_p + kPHalves) = half2v{plo[0], plo[1]};
                } else {
                    own_p[0] = phi[0];
                    own_p[kPHalves] = plo[0];
                }
                if (c == 0)
                    sm.alpha[hw] = alpha;
                __syncthreads();

                // 3. rescale and accumulate V^T P^T over this wave's dims, one
                // MFMA k-step per 32 keys
#pragma unroll
                for (int hb = 0; hb < kHB; ++hb) {
                    const float al = sm.alpha[16 * hb + key16];
                    if (__ballot(al != 1.0f) != 0ull) {
#pragma unroll
                        for (int db = 0; db < kCh / 16; ++db)
                            o[hb][db] *= al;
                    }
                }
#pragma unroll
                for (int ks = 0; ks < kKB / 2; ++ks) {
                    half8 va[kCh / 16];
                    // source lane 16G + 4i' + a points at key 32ks + 4G + i' (block 0)
                    // or 32ks + 16 + 4G + i' (block 1), dims 16db + 4a .. +4 of the
                    // wave's 64
                    const int src_key = kTile * ks + 4 * G + (key16 >> 2);
                    const int src_dim = 4 * (lane & 3);
#pragma unroll
                    for (int db = 0; db < kCh / 16; ++db) {
                        const _Float16* p0 = vtile + src_key * kVRow + 16 * db + src_dim;
                        const _Float16* p1 = p0 + 16 * kVRow;
                        const half4v lo4 = __builtin_bit_cast(
                            half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p0));
                        const half4v hi4 = __builtin_bit_cast(
                            half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p1));
                        va[db] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
#pragma unroll
                    for (int hb = 0; hb < kHB; ++hb) {
                        const half8 ph = sm.p[0][ks][hb][G][key16];
                        const half8 pl = sm.p[1][ks][hb][G][key16];
#pragma unroll
                        for (int db = 0; db < kCh / 16; ++db) {
                            o[hb][db] = mfma16(va[db], ph, o[hb][db]);
                            o[hb][db] = mfma16(va[db], pl, o[hb][db]);
                        }
                    }
                }
            }
            load_tile(pos(j + kDepth), eidx[u], ring[u]);
            load_idx(pos(j + 2 * kDepth), eidx[u]);
        }
    }

    if (splits == 1) {
        if (c == 0) {
            sm.lsum[hw] = own_l;
            if (lse != nullptr)
                lse[qrow * kHeads + head0 + hw] =
                    own_l > 0.0f ? (own_m + log2f(own_l)) * kLn2 : -INFINITY;
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) {
            const float l = sm.lsum[16 * hb + key16];
            emit<kRopeBf16>(o[hb], l > 0.0f ? 1.0f / l : 0.0f, qrow, head0 + 16 * hb + key16,
                            wave, G, dst_spec);
        }
        return;
    }
    // few rows: this split's unnormalised (O, max, sum) for attn_merge_kernel,
    // one record per 16 heads, through one buffer descriptor over this
    // workgroup's records.  The stores write through to memory (sc0 sc1): the
    // merge reads them a kernel later on any die, and stores that leave no
    // dirty L2 lines shorten the kernel boundary's write-back (attention +
    // merge measured 16.1 -> 15.6 us at 16 rows, 30.0 -> 28.8 us at 64 rows;
    // the same bytes).
    const int32_t rstride = splits * kPartFloats;  // floats between head-group records
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
        part + ((qrow * kGroups + head0 / kHg) * splits + split) * kPartFloats, 0,
        ((kHB - 1) * rstride + kPartFloats) * 4, kBufferConfig);
    if (c == 0) {
        const int32_t off = (hw / kHg) * rstride + kHg * kDim + hw % kHg;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(own_m), pr, 4 * off, 0,
                                              kWriteThrough);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(own_l), pr, 4 * (off + kHg), 0,
                                              kWriteThrough);
    }
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
#pragma unroll
        for (int db = 0; db < kCh / 16; ++db) {
            const int32_t off = hb * rstride + key16 * kDim + kCh * wave + 16 * db + 4 * G;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[hb][db]), pr,
                                                   4 * off, 0, kWriteThrough);
        }
    }
}

// Merge of the key splits of attn_kernel: one workgroup per (query row, 16
// heads, 128-dim slice), on the die of the workgroups that wrote the row's
// partials (the kernel boundary orders the partials: merging them inside the
// attention kernel, by the last split to finish, measured slower -- one
// workgroup then reads what 4 read here).
template <bool kRopeBf16>
__global__ void __launch_bounds__(256)
attn_merge_kernel(float* __restrict__ part, int32_t splits, int32_t queries, AttnOut dst,
                  float* __restrict__ lse)
{
    const int64_t x = blockIdx.x;
    const int64_t rest = x / kXcds;
    const int64_t qrow = kXcds * (rest / (kGroups * kSlices)) + x % kXcds;
    const int hg = (int)(rest % (kGroups * kSlices)) / kSlices;
    const int slice = (int)(rest % (kGroups * kSlices)) % kSlices;
    if (qrow >= queries)
        return;
    merge_slice<kRopeBf16>(part_rsrc(part, qrow, hg, splits), splits, qrow, hg, slice,
                           threadIdx.x, dst, lse);
}

int64_t padded_rows(int32_t queries)
{
    return ((int64_t)queries + kXcds - 1) / kXcds * kXcds;
}

// Key splits for few query rows: enough workgroups to cover the CUs once, at
// least two 32-key tiles per split; 1 when the rows alone fill the CUs.  From
// 64 rows the split workgroups take 32 heads (64 rows: 2 splits, 30.1 against
// 32.9 us for 16 heads without splits); below, 16 (16 rows: 4 splits, 15.9
// against 19.1 us for 32 heads in 8 splits, whose splits get too few tiles).
#ifndef CSA2_ATTN_SPLIT32_MIN_ROWS
#define CSA2_ATTN_SPLIT32_MIN_ROWS 64
#endif
constexpr int32_t kSplit32MinRows = CSA2_ATTN_SPLIT32_MIN_ROWS;

struct SplitPlan {
    int heads;       // heads per workgroup
    int32_t splits;  // key splits per (row, head group)
};

SplitPlan split_plan(int32_t queries, int32_t k, int32_t n_win)
{
    const int heads = queries >= kSplit32MinRows ? 32 : 16;
    const int64_t groups = padded_rows(queries) * (kHeads / heads);
    const int64_t tiles = ((int64_t)k + kTile - 1) / kTile + ((int64_t)n_win + kTile - 1) / kTile;
    int32_t s = 1;
    while (s < kMaxSplits && groups * s * 2 <= kSplitWgs && tiles >= kMinSplitTiles * 2 * s)
        s *= 2;
    return {heads, s};
}

template <int kHW>
hipError_t launch_heads(const uint16_t* q, int32_t queries, int32_t nq,
                        const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                        const int32_t* topk, int32_t k, const uint8_t* swa, int32_t swa_cap,
                        const int32_t* swa_end, int32_t n_win, float scale_log2,
                        int32_t splits, float* part, const AttnOut& spec, bool bf16_out,
                        float* lse, hipStream_t stream)
{
    const int64_t wgs = padded_rows(queries) * (kHeads / kHW) * splits;
    if (!grid_fits(wgs, kWaves * kWave))
        return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)wgs);
    const dim3 block(kWaves * kWave);
    // the split form writes unnormalised partials; the merge applies the epilogue
    if (bf16_out && splits == 1)
        attn_kernel<true, kHW, kKbOf<kHW>><<<grid, block, 0, stream>>>(
            q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end, n_win,
            scale_log2, splits, part, spec, lse);
    else
        attn_kernel<false, kHW, kKbOf<kHW>><<<grid, block, 0, stream>>>(
            q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end, n_win,
            scale_log2, splits, part, spec, lse);
    return hipGetLastError();
}

}  // namespace

// The key-split form launches at most kSplitWgs workgroups (and its merge 16
// per row of the few rows it serves), so the largest grid is the one-launch
// form's: one workgroup per row and head group.
bool sparse_attn_fits(int32_t queries)
{
    const int hw = queries >= kHw64MinRows ? 64 : (queries >= kHw32MinRows ? 32 : 16);
    return grid_fits(padded_rows(queries) * (kHeads / hw), kWaves * kWave);
}

size_t attn_workspace(int32_t queries, int32_t k, int32_t n_win)
{
    const int32_t s = split_plan(queries, k, n_win).splits;
    // one partial record per (row, 16 heads, split)
    return s > 1 ? (size_t)padded_rows(queries) * kGroups * s * kPartFloats * sizeof(float) : 0;
}

hipError_t launch_sparse_attn(const uint16_t* q, int32_t queries, int32_t nq,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                              const int32_t* topk, int32_t k, const uint8_t* swa,
                              int32_t swa_cap, const int32_t* swa_end, int32_t n_win,
                              float softmax_scale, float* out, uint16_t* out_bf16,
                              const float* rope_cos, const float* rope_sin, int32_t rope_off,
                              int32_t rope_dim, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream)
{
    if (queries == 0)
        return hipSuccess;
    const AttnOut spec{out, out_bf16, rope_cos, rope_sin, rope_off, rope_dim};
    const float scale_log2 = softmax_scale * kLog2e;
    const bool bf16_out = out_bf16 != nullptr;
    const size_t need = attn_workspace(queries, k, n_win);
    if (need > 0 && ws != nullptr && ws_bytes >= need) {
        // few rows: each row's keys split over workgroups, then the merge of
        // the splits (a second launch: the kernel boundary orders the partials)
        const SplitPlan sp = split_plan(queries, k, n_win);
        const int32_t splits = sp.splits;
        float* part = static_cast<float*>(ws);
        const hipError_t e =
            sp.heads == 32
                ? launch_heads<32>(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k, swa,
                                   swa_cap, swa_end, n_win, scale_log2, splits, part, spec,
                                   bf16_out, nullptr, stream)
                : launch_heads<16>(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k, swa,
                                   swa_cap, swa_end, n_win, scale_log2, splits, part, spec,
                                   bf16_out, nullptr, stream);
        if (e != hipSuccess)
            return e;
        const dim3 mgrid((uint32_t)(padded_rows(queries) * kGroups * kSlices)), mblock(256);
        if (!bf16_out)
            attn_merge_kernel<false><<<mgrid, mblock, 0, stream>>>(part, splits, queries, spec, lse);
        else
            attn_merge_kernel<true><<<mgrid, mblock, 0, stream>>>(part, splits, queries, spec, lse);
        return hipGetLastError();
    }
    // one workgroup per (row, head group) over every key (also the few-row form
    // when no workspace is given); the group grows with the rows
    if (queries >= kHw64MinRows)
        return launch_heads<64>(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k, swa,
                                swa_cap, swa_end, n_win, scale_log2, 1, nullptr, spec, bf16_out,
                                lse, stream);
    if (queries >= kHw32MinRows)
        return launch_heads<32>(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k, swa,
                                swa_cap, swa_end, n_win, scale_log2, 1, nullptr, spec, bf16_out,
                                lse, stream);
    return launch_heads<16>(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k, swa, swa_cap,
                            swa_end, n_win, scale_log2, 1, nullptr, spec, bf16_out, lse, stream);
}

}  // namespace csa2
