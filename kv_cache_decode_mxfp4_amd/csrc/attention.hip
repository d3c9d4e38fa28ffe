// Sparse MLA attention over the selected MXFP4 main-KV entries plus the FP8
// sliding window ([N] 1 of the DeepSeek-V4.1 reading notes: 64 query heads x
// 512; [S] "DeepSeek-V4 model structure (7)": K = V single-head MQA on the
// 512-dim latent, top-k compressed entries plus 128 window entries).  One
// joint softmax over both key sets; no de-duplication; no sink.
//
// The computation runs in one decomposition (tiles of 32 keys, MFMA
// v_mfma_f32_16x16x32_f16, keys dequantised exactly to fp16 straight into the
// MFMA operand and stored row-major to an LDS tile (K = V), online softmax in
// the log2 domain, P split into two fp16 terms (hi + lo) so P V keeps ~22
// bits of P): one workgroup per (query row, group of 16 heads), 4 workgroups
// per row -- for few rows (decode) also split over the keys, the splits merged
// by a second, short kernel; for many rows, two head groups per workgroup from
// 512 rows.  The four waves of a workgroup walk the same tiles and wave w
// owns the channels [128w, 128w+128): it dequantises only those channels of
// each key, forms the partial scores over them and accumulates the output for
// those 128 dims, so each key is dequantised once per head group and no score
// or output is computed twice.
//   partial S^T over the wave's channels: lane l holds key l%16 and the 32
//     channels [128w + 32G, +32) (k-step t: 128w + 32G + 8t .. +8; the Q^T
//     operand stays in registers); the four partials meet in LDS (one barrier
//     per tile) and every wave adds them in wave order, so all four hold
//     bit-identical scores and softmax state.
//
// Operand layouts:
//   P^T: the S^T accumulator of lane l holds keys 4G + r (r < 4) of both
//     blocks for head l%16, which is the B-operand layout of P^T for
//     O^T = V^T P^T once the 32 keys of a tile take MFMA k-index 8G + i <->
//     key 16*(i/4) + 4G + i%4;
//   V^T[16 dims x 32 keys]: read from the row-major LDS tile with the gfx950
//     transposing read ds_read_b64_tr_b16 (within each 16-lane group, lane
//     4a + j receives element j of lanes a, a+4, a+8, a+12), two reads per
//     MFMA, in the same key order;
//   loads are unconditional (clamped inside the list or pointed at the query
//     row, masked afterwards), so the load counter stays exact; the top-k
//     indices are loaded ahead of the keys they address.
#include "device_common.h"
#include "launch.h"

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4 __attribute__((vector_size(8)));  // operand type of the LDS transposing read
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int kTile = 32;                       // keys per tile (two MFMA blocks of 16)
constexpr int kHg = 16;                         // heads per workgroup
constexpr int kGroups = kHeads / kHg;           // 4 head groups
constexpr int kSlice = 128;                     // channels / output dims per slice
constexpr int kSlices = kDim / kSlice;          // 4 slices
constexpr int kVRow = kSlice + 16;              // halves per LDS row of V (288 B)
constexpr int kXcds = 8;                        // MI355X dies: workgroups go round-robin
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Online-softmax state of one wave: lane l tracks head l%16 (replicated over
// the four lane groups, which always agree bit for bit).
struct Online {
    float m = -INFINITY;   // running max (log2 domain)
    float l = 0.0f;        // running sum
    f32x4 o[kSlice / 16];  // O^T: dims 16*db + 4G + r of the wave's slice, head l%16
};

// Folds one tile's S^T (already scaled, -inf for invalid keys) into the state
// and accumulates P V over the wave's LDS tile.
__device__ __forceinline__ void fold_tile(Online& st, const f32x4 (&s)[2],
                                          const _Float16* __restrict__ vtile, int lane)
{
    const int G = lane >> 4;
    float tmax = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            tmax = fmaxf(tmax, s[b][r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(st.m, tmax);
    float p[2][4];
    float psum = 0.0f;
    float alpha = 1.0f;
    if (m_new == -INFINITY) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                p[b][r] = 0.0f;
    } else {
        // the hardware exp2 (no subnormal range fix-up): every argument here is
        // <= 0, and a result below 2^-126 is lost next to the running maximum's
        // term (exactly 1) in every sum and rounds to zero in the fp16 P pair
        alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[b][r] = __builtin_amdgcn_exp2f(s[b][r] - m_new);
                psum += p[b][r];
            }
    }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int db = 0; db < kSlice / 16; ++db)
        st.o[db] *= alpha;

    half8 phi, plo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float pv = p[i / 4][i % 4];
        phi[i] = (_Float16)pv;
        plo[i] = (_Float16)(pv - (float)phi[i]);
    }
    // source lane 16G + 4i' + a points at key 4G + i' (block 0) or 16 + 4G + i'
    // (block 1), dims 16*db + 4a .. +4 of the slice
    const int src_key = 4 * G + ((lane & 15) >> 2);
    const int src_dim = 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < kSlice / 16; ++db) {
        const _Float16* p0 = vtile + src_key * kVRow + 16 * db + src_dim;
        const _Float16* p1 = p0 + 16 * kVRow;
        const half4v lo =
            __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p0));
        const half4v hi =
            __builtin_bit_cast(half4v, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4*)p1));
        const half8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        st.o[db] = mfma16(a, phi, st.o[db]);
        st.o[db] = mfma16(a, plo, st.o[db]);
    }
}

// S^T of one tile to the log2 domain (scale_log2: the softmax scale times
// log2(e), divided by the lane's head's query scaling), -inf for invalid keys
// (bit b of `valid` tells whether this lane's key of block b is valid).
__device__ __forceinline__ void scale_scores(f32x4 (&s)[2], uint32_t valid, float scale_log2,
                                             int G)
{
    const uint64_t vm0 = __ballot((valid & 1u) != 0u);
    const uint64_t vm1 = __ballot((valid & 2u) != 0u);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int kk = 4 * G + r;
        s[0][r] = ((vm0 >> kk) & 1ull) ? s[0][r] * scale_log2 : -INFINITY;
        s[1][r] = ((vm1 >> kk) & 1ull) ? s[1][r] * scale_log2 : -INFINITY;
    }
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

// ============================================================= grouped form

constexpr int kGroupWaves = kSlices;            // one wave per 128-channel slice
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
constexpr int kMinSplitTiles = CSA2_ATTN_MIN_SPLIT_TILES;  // fewest key tiles per split
constexpr int kPartFloats = kHg * kDim + 2 * kHg;  // one split's O [16][512], max, sum

template <int kHgW>
struct GroupSmem {
    _Float16 v[kGroupWaves][kTile][kVRow];          // each wave's V tile (its 128 dims)
    // partial S^T per head group and wave, double-buffered: [buffer][head
    // group][wave][key block][lane], so each lane's 16-byte store and load is
    // contiguous with its neighbours' (a 32-byte lane stride made lanes l and
    // l + 8 share banks)
    f32x4 part[2][kHgW][kGroupWaves][2][kWave];
    float qmax[kHgW][kGroupWaves][kHg];  // largest |q| of each head over each wave's slice
};

// Raw bytes of one tile for the calling lane, for key l%16 of block b:
// top-k tile: a = the 16 code bytes of channels [128w + 32G, +32), s = the 16
// scale bytes that hold this wave's slice; window tile: a, s = the 32 E4M3
// bytes of those channels.
struct TileRaw {
    u32x4 a[2], s[2];
    uint32_t valid;  // bit b: key of block b is valid
};

// Partial S^T of one tile over the wave's 128 channels (block bb in s[bb]);
// the dequantised keys also go to the wave's LDS tile.  kMain: MXFP4 top-k
// keys, else E4M3 window rows.
template <bool kMain, int kHgW>
__device__ __forceinline__ void tile_scores(const TileRaw& R, const half8 (&qop)[kHgW][4],
                                            _Float16* __restrict__ vtile, int slice, int G,
                                            int key16, f32x4 (&s)[kHgW][2])
{
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
        f32x4 acc[kHgW];
#pragma unroll
        for (int h = 0; h < kHgW; ++h)
            acc[h] = f32x4{};
        const bool ok = (R.valid >> bb) & 1u;
        // scale bytes of this lane's 32 channels: dword 2(w%2) + G/2 of the 16
        // loaded, bytes 2(G%2) and 2(G%2)+1
        const uint32_t sdw = (slice & 1) ? (G >= 2 ? R.s[bb][3] : R.s[bb][2])
                                        : (G >= 2 ? R.s[bb][1] : R.s[bb][0]);
        const uint32_t sc = ok ? sdw >> (16 * (G & 1)) : 0u;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            half8 a;
            if (kMain) {
                const uint32_t word = ok ? R.a[bb][t] : 0u;
                a = dequant8_fp4(word, e4m3_byte_to_f16(sc, t / 2));
            } else {
                const u32x4 src = t < 2 ? R.a[bb] : R.s[bb];
                const uint32_t w0 = ok ? src[2 * (t % 2)] : 0u;
                const uint32_t w1 = ok ? src[2 * (t % 2) + 1] : 0u;
                const half4v x0 = e4m3x4_to_f16(w0), x1 = e4m3x4_to_f16(w1);
                a = half8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            }
#pragma unroll
            for (int h = 0; h < kHgW; ++h)
                acc[h] = mfma16(a, qop[h][t], acc[h]);
            *reinterpret_cast<half8*>(vtile + (16 * bb + key16) * kVRow + 32 * G + 8 * t) = a;
        }
#pragma unroll
        for (int h = 0; h < kHgW; ++h)
            s[h][bb] = acc[h];
    }
}

// Writes this lane's outputs (head `head`, dims 128*slice + 16db + 4G + r) as
// o * inv, through the epilogue of kRopeBf16.
template <bool kRopeBf16>
__device__ __forceinline__ void emit(const f32x4 (&o)[kSlice / 16], float inv, int64_t qrow,
                                     int head, int slice, int G, const AttnOut& dst)
{
    const int64_t base = (qrow * kHeads + head) * kDim + kSlice * slice + 4 * G;
#pragma unroll
    for (int db = 0; db < kSlice / 16; ++db) {
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
                const int d = kSlice * slice + 16 * db + 4 * G + i;
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

constexpr int kBufferConfig = 0x00020000;  // raw (untyped) buffer, 32-bit data
constexpr int kCachePolicy = 0;            // plain loads (the partials of the previous kernel)

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
#define CSA2_ATTN_WAVES_PER_EU 3
#endif
// Query rows from which the many-row form takes two head groups per workgroup:
// below it, half as many workgroups leave CUs idle (64 rows: 50 vs 34 us).
#ifndef CSA2_ATTN_HG2_MIN_ROWS
#define CSA2_ATTN_HG2_MIN_ROWS 512
#endif
constexpr int32_t kHg2MinRows = CSA2_ATTN_HG2_MIN_ROWS;

// kHgW head groups per workgroup: 1 for the key-split (few rows) form; 2 for
// many rows, where each dequantised key then serves 32 heads (half the
// dequantisation and key fetches per head) at two waves per SIMD.  Every head
// group runs exactly the one-group sequence of operations, so outputs are
// bit-identical either way.
template <bool kRopeBf16, int kHgW>
__global__ void __launch_bounds__(kGroupWaves * kWave)
__attribute__((amdgpu_waves_per_eu(kHgW == 1 ? CSA2_ATTN_WAVES_PER_EU : 2)))
attn_group_kernel(const uint16_t* __restrict__ q, int32_t queries,
                  const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales,
                  int64_t n_cap, int32_t nq, const int32_t* __restrict__ topk, int32_t k,
                  const uint8_t* __restrict__ swa, int32_t swa_cap,
                  const int32_t* __restrict__ swa_end, int32_t n_win, float scale_log2,
                  int32_t splits, float* __restrict__ part, AttnOut dst_spec,
                  float* __restrict__ lse)
{
    __shared__ GroupSmem<kHgW> sm;
    const int lane = threadIdx.x & 63;
    // the wave's slice as a scalar: everything derived from it (pointers,
    // offsets) stays in scalar registers
    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = lane >> 4;
    const int key16 = lane & 15;

    // the workgroups of a query row (4 head groups x splits) share one die
    // (and its L2, which then serves the keys to every head group): with
    // round-robin dispatch, workgroup x runs on die x % 8
    constexpr int kWgGroups = kGroups / kHgW;  // workgroups per row and split
    const int wg_per_row = kWgGroups * splits;
    const int64_t x = blockIdx.x;
    const int64_t rest = x / kXcds;
    const int64_t qrow = kXcds * (rest / wg_per_row) + x % kXcds;
    const int hg0 = ((int)(rest % wg_per_row) % kWgGroups) * kHgW;  // first head group
    const int split = (int)(rest % wg_per_row) / kWgGroups;
    if (qrow >= queries)
        return;
    const int64_t b = qrow / nq;
    // head of this lane's score column in head group hg0 + h: kHg * (hg0 + h) + key16

    // tile list: top-k tiles [0, t_main), then window tiles; this workgroup
    // takes the list positions split + splits * j
    const int t_main = n_cap > 0 ? (k + kTile - 1) / kTile : 0;
    auto pos = [&](int j) { return split + splits * j; };

    // loads with no data to fetch read the query row (64 KiB, always valid)
    // and are masked, so every load is unconditional
    const uint8_t* dummy = reinterpret_cast<const uint8_t*>(q + qrow * kHeads * kDim);
    const uint8_t* kc = t_main > 0 ? kv_codes + b * n_cap * (kDim / 2) : dummy;
    const uint8_t* ks = t_main > 0 ? kv_scales + b * n_cap * (kDim / 16) : dummy;
    const int32_t* tk = t_main > 0 ? topk + qrow * k : reinterpret_cast<const int32_t*>(dummy);

    // top-k index of this lane's key in block bb of tile p (any valid slot
    // when p is not a top-k tile)
    auto load_idx = [&](int p, int32_t (&e)[2]) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int slot = p * kTile + 16 * bb + key16;
            e[bb] = tk[t_main > 0 ? (slot < k ? slot : k - 1) : 0];
        }
    };

    int32_t eidx[kDepth][2];
#pragma unroll
    for (int u = 0; u < kDepth; ++u)
        load_idx(pos(u), eidx[u]);
    // Q^T operand: head l%16 of each group, channels [128w + 32G, +32), bf16 -> fp16
    uint4 qraw[kHgW][4];
#pragma unroll
    for (int h = 0; h < kHgW; ++h) {
        const uint4* src = reinterpret_cast<const uint4*>(
            q + (qrow * kHeads + kHg * (hg0 + h) + key16) * kDim + kSlice * slice + 32 * G);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            qraw[h][t] = src[t];
    }

    // window rows [lo, hi)
    const int64_t end = swa_end[qrow];
    int64_t lo = end - n_win;
    lo = lo < 0 ? 0 : lo;
    int64_t hi = end < swa_cap ? end : (int64_t)swa_cap;
    hi = hi < lo ? lo : hi;
    const int n_sw = (int)(hi - lo);
    const int t_sw = (n_sw + kTile - 1) / kTile;
    const uint8_t* sw = n_sw > 0 ? swa + b * (int64_t)swa_cap * kDim : dummy;
    const int n_tiles = t_main + t_sw;
    const int n_j = split < n_tiles ? (n_tiles - split + splits - 1) / splits : 0;

    // raw bytes of tile p; tiles past the list load valid rows and are
    // masked.  Both kinds' addresses are formed and one is selected, so the
    // loads stay outside any branch.
    auto load_tile = [&](int p, const int32_t (&e)[2], TileRaw& R) {
        const bool is_main = p < t_main;
        const int tw = p - t_main;
        R.valid = 0;
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
            const int slot = p * kTile + 16 * bb + key16;
            const bool ok_m = slot < k && e[bb] >= 0 && e[bb] < n_cap;
            const int64_t ee = ok_m ? e[bb] : 0;
            const int64_t r = lo + (int64_t)tw * kTile + 16 * bb + key16;
            const bool ok_w = tw >= 0 && tw < t_sw && r < hi;
            const int64_t rr = ok_w ? r : (n_sw > 0 ? lo : 0);
            const uint8_t* pm = kc + ee * (kDim / 2) + 64 * slice + 16 * G;
            const uint8_t* pw = sw + rr * kDim + kSlice * slice + 32 * G;
            const uint8_t* pa = is_main ? pm : pw;
            const uint8_t* ps = is_main ? ks + ee * (kDim / 16) + 16 * (slice / 2) : pw + 16;
            R.a[bb] = *reinterpret_cast<const u32x4*>(pa);
            R.s[bb] = *reinterpret_cast<const u32x4*>(ps);
            R.valid |= (is_main ? ok_m : ok_w) ? (1u << bb) : 0u;
        }
    };

    TileRaw ring[kDepth];
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
    // those of the unscaled query.  The largest |q| of a head spans the four waves'
    // channel slices: one exchange through LDS.
    float head_scale[kHgW];  // scale_log2 * 2^-shift for this lane's head (l % 16)
    int qshift[kHgW];
    {
#pragma unroll
        for (int h = 0; h < kHgW; ++h) {
            float m = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t d[4] = {qraw[h][t].x, qraw[h][t].y, qraw[h][t].z, qraw[h][t].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    m = fmaxf(m, fabsf(__uint_as_float(d[i] << 16)));
                    m = fmaxf(m, fabsf(__uint_as_float(d[i] & 0xFFFF0000u)));
                }
            }
            m = fmaxf(m, __shfl_xor(m, 16, kWave));
            m = fmaxf(m, __shfl_xor(m, 32, kWave));
            if (lane < kHg)
                sm.qmax[h][slice][lane] = m;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < kHgW; ++h) {
            float m = sm.qmax[h][0][key16];
#pragma unroll
            for (int w = 1; w < kGroupWaves; ++w)
                m = fmaxf(m, sm.qmax[h][w][key16]);
            int sh = 0;  // 0 for an all-zero head
            if (m > 0.0f && !__builtin_isinf(m) && !__builtin_isnan(m)) {
                sh = 14 - ((int)((__float_as_uint(m) >> 23) & 0xFF) - 127);
                sh = sh < -100 ? -100 : (sh > 100 ? 100 : sh);
            }
            qshift[h] = sh;
            head_scale[h] = ldexpf(scale_log2, -sh);
        }
    }
    half8 qop[kHgW][4];
#pragma unroll
    for (int h = 0; h < kHgW; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t d[4] = {qraw[h][t].x, qraw[h][t].y, qraw[h][t].z, qraw[h][t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qop[h][t][2 * i] = (_Float16)ldexpf(__uint_as_float(d[i] << 16), qshift[h]);
                qop[h][t][2 * i + 1] = (_Float16)ldexpf(__uint_as_float(d[i] & 0xFFFF0000u),
                                                        qshift[h]);
            }
        }

    Online st[kHgW];
#pragma unroll
    for (int h = 0; h < kHgW; ++h)
#pragma unroll
        for (int db = 0; db < kSlice / 16; ++db)
            st[h].o[db] = f32x4{};
    _Float16* vtile = &sm.v[slice][0][0];

    // slot u of the ring holds the tile of step j0 + u; after use it is refilled
    // with the tile of step j + kDepth, and its index slot with the indices of
    // step j + 2*kDepth
    for (int j0 = 0; j0 < n_j; j0 += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            const int j = j0 + u;
            const int p = pos(j);
            if (j < n_j) {  // the same for every wave: the barrier below is uniform
                f32x4 s[kHgW][2];
                if (p < t_main)
                    tile_scores<true, kHgW>(ring[u], qop, vtile, slice, G, key16, s);
                else
                    tile_scores<false, kHgW>(ring[u], qop, vtile, slice, G, key16, s);
                // the four partial scores of each head group meet in LDS; every
                // wave adds them in wave order (bit-identical in every wave)
#pragma unroll
                for (int h = 0; h < kHgW; ++h) {
                    sm.part[j & 1][h][slice][0][lane] = s[h][0];
                    sm.part[j & 1][h][slice][1][lane] = s[h][1];
                }
                __syncthreads();
#pragma unroll
                for (int h = 0; h < kHgW; ++h) {
                    f32x4 tot0 = sm.part[j & 1][h][0][0][lane];
                    f32x4 tot1 = sm.part[j & 1][h][0][1][lane];
#pragma unroll
                    for (int w = 1; w < kGroupWaves; ++w) {
                        tot0 += sm.part[j & 1][h][w][0][lane];
                        tot1 += sm.part[j & 1][h][w][1][lane];
                    }
                    s[h][0] = tot0;
                    s[h][1] = tot1;
                    scale_scores(s[h], ring[u].valid, head_scale[h], G);
                    fold_tile(st[h], s[h], vtile, lane);
                }
            }
            load_tile(pos(j + kDepth), eidx[u], ring[u]);
            load_idx(pos(j + 2 * kDepth), eidx[u]);
        }
    }

    if (splits == 1) {
#pragma unroll
        for (int h = 0; h < kHgW; ++h) {
            const int head = kHg * (hg0 + h) + key16;
            const float inv = st[h].l > 0.0f ? 1.0f / st[h].l : 0.0f;
            emit<kRopeBf16>(st[h].o, inv, qrow, head, slice, G, dst_spec);
            if (lse != nullptr && slice == 0 && G == 0)
                lse[qrow * kHeads + head] =
                    st[h].l > 0.0f ? (st[h].m + log2f(st[h].l)) * kLn2 : -INFINITY;
        }
        return;
    }
    // few rows: this split's unnormalised (O, max, sum) for attn_merge_kernel
#pragma unroll
    for (int h = 0; h < kHgW; ++h) {
        float* mine = part + ((qrow * kGroups + hg0 + h) * splits + split) * kPartFloats;
#pragma unroll
        for (int db = 0; db < kSlice / 16; ++db)
            *reinterpret_cast<f32x4*>(mine + key16 * kDim + kSlice * slice + 16 * db + 4 * G) =
                st[h].o[db];
        if (slice == 0 && G == 0) {
            mine[kHg * kDim + key16] = st[h].m;
            mine[kHg * kDim + kHg + key16] = st[h].l;
        }
    }
}

// Merge of the key splits of attn_group_kernel: one workgroup per (query row,
// head group, 128-dim slice), on the die of the workgroups that wrote the
// row's partials (the kernel boundary orders the partials: merging them inside
// the attention kernel, by the last split to finish, measured slower -- one
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

// Key splits of the grouped form for few query rows: enough workgroups to
// cover the CUs once, at least two tiles per split; 1 when the rows alone
// fill the CUs.
#ifndef CSA2_ATTN_SPLIT_HG_PER_WG
#define CSA2_ATTN_SPLIT_HG_PER_WG 1
#endif
constexpr int kSplitHgW = CSA2_ATTN_SPLIT_HG_PER_WG;  // head groups per key-split workgroup

int32_t attn_splits(int32_t queries, int32_t k, int32_t n_win)
{
    const int64_t groups = padded_rows(queries) * (kGroups / kSplitHgW);
    const int64_t tiles = ((int64_t)k + kTile - 1) / kTile + ((int64_t)n_win + kTile - 1) / kTile;
    int32_t s = 1;
    while (s < kMaxSplits && groups * s * 2 <= kSplitWgs && tiles >= kMinSplitTiles * 2 * s)
        s *= 2;
    return s;
}

}  // namespace

size_t attn_workspace(int32_t queries, int32_t k, int32_t n_win)
{
    const int32_t s = attn_splits(queries, k, n_win);
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
    // rows padded to a multiple of the die count (padding workgroups exit at once)
    const int64_t rows = padded_rows(queries);
    const AttnOut spec{out, out_bf16, rope_cos, rope_sin, rope_off, rope_dim};
    const float scale_log2 = softmax_scale * kLog2e;
    const size_t need = attn_workspace(queries, k, n_win);
    const dim3 block(kGroupWaves * kWave);
    if (need > 0 && ws != nullptr && ws_bytes >= need) {
        // few rows: each row's keys split over workgroups, then the merge of the
        // splits (a second launch: the kernel boundary orders the partials)
        const int32_t splits = attn_splits(queries, k, n_win);
        float* part = static_cast<float*>(ws);
        const dim3 grid((uint32_t)(rows * (kGroups / kSplitHgW) * splits));
        attn_group_kernel<false, kSplitHgW><<<grid, block, 0, stream>>>(
            q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end, n_win,
            scale_log2, splits, part, spec, lse);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        const dim3 mgrid((uint32_t)(rows * kGroups * kSlices)), mblock(256);
        if (out_bf16 == nullptr)
            attn_merge_kernel<false><<<mgrid, mblock, 0, stream>>>(part, splits, queries, spec, lse);
        else
            attn_merge_kernel<true><<<mgrid, mblock, 0, stream>>>(part, splits, queries, spec, lse);
    } else if (queries >= kHg2MinRows) {
        // many rows: two head groups per workgroup (enough rows to fill the CUs
        // with half as many workgroups)
        const dim3 grid((uint32_t)(rows * (kGroups / 2)));
        if (out_bf16 == nullptr)
            attn_group_kernel<false, 2><<<grid, block, 0, stream>>>(
                q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end,
                n_win, scale_log2, 1, nullptr, spec, lse);
        else
            attn_group_kernel<true, 2><<<grid, block, 0, stream>>>(
                q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end,
                n_win, scale_log2, 1, nullptr, spec, lse);
    } else {
        // one workgroup per (row, head group) over every key (also the few-row form
        // when no workspace is given)
        const dim3 grid((uint32_t)(rows * kGroups));
        if (out_bf16 == nullptr)
            attn_group_kernel<false, 1><<<grid, block, 0, stream>>>(
                q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end,
                n_win, scale_log2, 1, nullptr, spec, lse);
        else
            attn_group_kernel<true, 1><<<grid, block, 0, stream>>>(
                q, queries, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end,
                n_win, scale_log2, 1, nullptr, spec, lse);
    }
    return hipGetLastError();
}

}  // namespace csa2
