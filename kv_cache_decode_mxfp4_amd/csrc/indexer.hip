// Indexer kernels of the hierarchical sparse indexer ([N] 2.2 and [A] 3.4 of
// the DeepSeek-V4.1 pages: the first Full layer scores the whole visible range
// and ranks blocks of 8 positions by their largest score; Reindex layers score
// only the pool of selected blocks).
//
// Every kernel here scores with score.h's score function (its MFMA mapping and
// the reading of the score formula are described there), so a position's
// score is bit-identical whether it comes from the full scan or a pool scan.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "score.h"
#include "select.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kTileEntries = 32;    // entries per MFMA tile
#ifndef CSA2_SCAN_PREFETCH
#define CSA2_SCAN_PREFETCH 4
#endif
constexpr int kPrefetch = CSA2_SCAN_PREFETCH;  // key tiles in flight per wave
constexpr int kStep = kTileEntries * kWaves;   // entries between a wave's tiles
constexpr int kGroupEntries = kPrefetch * kStep;  // entries per prefetch round
// Entries per scan workgroup: a multiple of kGroupEntries chosen at launch,
// the largest (up to kMaxChunk) that still gives kScanTargetWorkgroups
// workgroups (256 CUs x 4 resident workgroups), so each workgroup loads its
// query once and keeps its prefetch ring running over a long range.
#ifndef CSA2_SCAN_MAX_CHUNK
#define CSA2_SCAN_MAX_CHUNK 16384
#endif
#ifndef CSA2_SCAN_TARGET_WGS
#define CSA2_SCAN_TARGET_WGS 1024
#endif
constexpr int kMaxChunk = CSA2_SCAN_MAX_CHUNK;
constexpr int64_t kScanTargetWorkgroups = CSA2_SCAN_TARGET_WGS;
// Query rows per sequence from which the scan pairs rows (prefill shapes);
// decode (one row per sequence) streams its keys from HBM, one row each.
#ifndef CSA2_SCAN_PAIR_MIN_ROWS
#define CSA2_SCAN_PAIR_MIN_ROWS 2
#endif
constexpr int32_t kPairMinRows = CSA2_SCAN_PAIR_MIN_ROWS;

// Keys of one chunk, read with raw buffer loads: the descriptors hold the
// chunk's base addresses and sizes in bytes (scalar registers), a lane keeps
// one 32-bit offset per array, and the hardware range check turns every load
// past the size into zeros.  The scale descriptor ends at the last visible
// entry; the code descriptor starts at the key tile holding the chunk's first
// entry f0 and ends with the tile holding its last visible entry (entries of
// that tile past the visible end are read and masked).  Tile offsets are
// added to the vector offset, which the range check covers.  Loads are
// non-temporal (the keys are streamed once).
struct ChunkKeys {
    __amdgpu_buffer_rsrc_t codes, scales;
    int32_t vc, vs;  // byte offsets of the lane's entry and half in tile 0
};

constexpr int kBufferConfig = 0x00020000;  // raw (untyped) buffer, 32-bit data
constexpr int kNonTemporal = 2;

// f0: flat index of the chunk's first entry; entries: visible entries of the
// chunk; entry: the lane's entry relative to f0 in tile 0 (32 * wave plus
// lane % 32).
__device__ __forceinline__ ChunkKeys chunk_keys(const uint8_t* codes, const uint8_t* scales,
                                                int64_t f0, int32_t entries, int entry,
                                                int half)
{
    ChunkKeys C;
    const int64_t t0 = f0 >> 5;                                // key tile of f0
    const int64_t t_end = (f0 + entries + kKeyTile - 1) >> 5;  // past the last visible tile
    C.codes = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes + t0 * kKeyTileBytes), 0,
        (int32_t)((t_end - t0) * kKeyTileBytes), kBufferConfig);
    C.scales = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + f0 * (kIdxDim / 16)), 0, entries * (kIdxDim / 16),
        kBufferConfig);
    const int e = (int)(f0 & 31) + entry;  // the lane's entry counted from tile t0's first
    C.vc = (e >> 5) * kKeyTileBytes + 2 * half * kKeyPlane + (e & 31) * 16;
    C.vs = entry * (kIdxDim / 16) + 4 * half;
    return C;
}

// Tile whose entries start `first_entry` (a multiple of 32) entries after the
// lane's tile-0 entry.
__device__ __forceinline__ void load_key(const ChunkKeys& C, int32_t first_entry, KeyTile& K)
{
    const int32_t oc = C.vc + first_entry * (kIdxDim / 2);
    const int32_t os = C.vs + first_entry * (kIdxDim / 16);
    K.c0 = __builtin_amdgcn_raw_buffer_load_b128(C.codes, oc, 0, kNonTemporal);
    K.c1 = __builtin_amdgcn_raw_buffer_load_b128(C.codes, oc + kKeyPlane, 0, kNonTemporal);
    K.sc = __builtin_amdgcn_raw_buffer_load_b32(C.scales, os, 0, kNonTemporal);
}

// Scores of the lane's entry for two queries: the key is dequantised once and
// feeds both MFMA chains; each chain is the one score_entry runs (same operands,
// same order), so both scores are bit-identical to score_entry's.
__device__ __forceinline__ void score_entry2(const QueryOperand& Q0, const QueryOperand& Q1,
                                             const KeyTile& K, float& s0, float& s1)
{
    const uint32_t words[8] = {K.c0[0], K.c0[1], K.c0[2], K.c0[3], K.c1[0], K.c1[1], K.c1[2], K.c1[3]};
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const _Float16 s = e4m3_byte_to_f16(K.sc, t / 2);
        const half8 b = dequant8_fp4(words[t], s);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Q0.a[t], b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(Q1.a[t], b, acc1, 0, 0, 0);
    }
    s0 = head_sum(Q0, acc0);
    s1 = head_sum(Q1, acc1);
}

// Maximum over the 8 lanes of each aligned group of 8 (DPP: swap neighbours,
// swap pairs, then mirror within the half-row of 8).
__device__ __forceinline__ float max8(float s)
{
    float m = fmaxf(s, __uint_as_float(dpp_u32<0xB1>(0u, __float_as_uint(s))));
    m = fmaxf(m, __uint_as_float(dpp_u32<0x4E>(0u, __float_as_uint(m))));
    return fmaxf(m, __uint_as_float(dpp_u32<0x141>(0u, __float_as_uint(m))));
}

// Group keys of one row's chunk for the block select (after the scan loop):
// group t of the chunk -- blocks [t*g, t*g + g) of the chunk, g = 1 << gshift,
// of which [0, nb_here) are visible and held in sblk -- gets the order key of
// its largest non-NaN block maximum, 0 if it has none: what the block
// select's group-maxima pass computes from the block maxima.  Row `row` of
// gkey has ngroups groups; the chunk starts at entry `start` (a multiple of
// 512 entries, so its first group is whole for g <= 64).
__device__ __attribute__((noinline)) void write_group_keys(const float* sblk, int nb_here,
                                                           int64_t row, int64_t start,
                                                           int32_t chunk, int32_t gshift,
                                                           int64_t ngroups,
                                                           uint32_t* __restrict__ gkey)
{
    const int64_t g0 = (start / kBlock) >> gshift;
    const int64_t left = ngroups - g0;
    const int per = (chunk / kBlock) >> gshift;
    const int groups_here = (int)(left < per ? (left < 0 ? 0 : left) : per);
    uint32_t* gk = gkey + row * ngroups + g0;
    const int g = 1 << gshift;
    for (int t = threadIdx.x; t < groups_here; t += kWaves * kWave) {
        uint32_t m = 0u;
        for (int r = 0; r < g; ++r) {
            const int blk = t * g + r;
            if (blk < nb_here) {
                const float f = sblk[blk];
                if (!__builtin_isnan(f))
                    m = max(m, order_key(f));
            }
        }
        gk[t] = m;
    }
}

// Block candidates of one row's chunk for the block select (after the scan
// loop; the chunk's nb_here visible block maxima are in sblk): the kl best
// blocks under the selection order (larger maximum first, lower block first),
// (order key, block id) in block order, (0, -1) padded; full = the chunk had
// more than kl visible blocks.  A NaN maximum has key 0 and is never a
// candidate.  kl <= the chunk's block count, a multiple of 64.
constexpr int kCandThreads = kWaves * kWave;
constexpr int kCandSlots = kMaxChunk / kBlock / kCandThreads;  // blocks per thread

__device__ __attribute__((noinline)) void write_candidates(const float* sblk, int nb_here,
                                                           int64_t blk0, int32_t kl,
                                                           uint32_t* __restrict__ ckey,
                                                           int32_t* __restrict__ cblk,
                                                           int32_t* __restrict__ cfull)
{
    __shared__ sel::Smem<kCandThreads> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    uint32_t key[kCandSlots];
#pragma unroll
    for (int i = 0; i < kCandSlots; ++i) {
        const int b = kCandThreads * i + tid;
        const float f = b < nb_here ? sblk[b] : 0.0f;
        key[i] = b < nb_here && !__builtin_isnan(f) ? order_key(f) : 0u;
    }
    sel::clear_hist(sm, tid);
    const sel::Pick pk = sel::find_threshold<kCandSlots, kCandThreads>(key, (uint32_t)kl, sm, tid,
                                                                       lane, wave);
    bool take[kCandSlots];
    uint32_t off[kCandSlots];
    const uint32_t chosen =
        sel::place<kCandSlots, kCandThreads>(key, pk, take, off, sm, lane, wave);
#pragma unroll
    for (int i = 0; i < kCandSlots; ++i)
        if (take[i] && off[i] < (uint32_t)kl) {
            ckey[off[i]] = key[i];
            cblk[off[i]] = (int32_t)(blk0 + kCandThreads * i + tid);
        }
    for (uint32_t p = chosen + tid; p < (uint32_t)kl; p += kCandThreads) {
        ckey[p] = 0u;
        cblk[p] = -1;
    }
    if (tid == 0)
        *cfull = nb_here > kl ? 1 : 0;
}

// Empty candidate list of a chunk past the row's visible end.
__device__ __forceinline__ void write_no_candidates(int32_t kl, uint32_t* __restrict__ ckey,
                                                    int32_t* __restrict__ cblk,
                                                    int32_t* __restrict__ cfull)
{
    for (int p = threadIdx.x; p < kl; p += kCandThreads) {
        ckey[p] = 0u;
        cblk[p] = -1;
    }
    if (threadIdx.x == 0)
        *cfull = 0;
}

// Full-range scan: one workgroup scans `chunk` entries of one query row and
// writes the maxima of the blocks of 8 it covers (and, with kScores, every
// score).  Wave w scores tiles start + 32*(w + kWaves*i).
//
// The loop has no data-dependent branch and stores nothing to global memory
// (block maxima go to LDS and leave in one coalesced store at the end), so
// the compiler keeps kPrefetch tiles per wave in flight across iterations
// instead of draining the load counter.  The chunk's buffer descriptors end
// at the last visible entry: tiles past it read zeros and their scores are
// masked to -inf, which handles the partial last chunk of a row without a
// second code path.  128 VGPRs: four workgroups per CU.
template <bool kScores>
__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(4)))
index_full_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                  const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t n_cap, const int32_t* __restrict__ n_visible, int32_t nq,
                  int32_t chunk, int32_t chunks_per_query, int64_t nblk_cap,
                  float* __restrict__ block_max, float* __restrict__ scores,
                  uint32_t* __restrict__ gkey, int32_t gshift, int64_t ngroups,
                  uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_blk,
                  int32_t* __restrict__ cand_full, int32_t kl)
{
    __shared__ float sblk[kMaxChunk / kBlock];

    const int64_t row = blockIdx.x / chunks_per_query;  // query row b*nq + i
    const int64_t b = row / nq;
    int64_t n_vis = n_visible[row];
    n_vis = n_vis < 0 ? 0 : (n_vis > n_cap ? n_cap : n_vis);
    const int64_t start = (int64_t)(blockIdx.x % chunks_per_query) * chunk;
    // this chunk's candidate list (block select), when asked for
    const int64_t cslot = (int64_t)blockIdx.x * kl;
    if (start >= n_vis) {
        if (gkey != nullptr)
            write_group_keys(sblk, 0, row, start, chunk, gshift, ngroups, gkey);
        if (cand_key != nullptr)
            write_no_candidates(kl, cand_key + cslot, cand_blk + cslot, cand_full + blockIdx.x);
        return;
    }
    const int32_t n_here = (int32_t)(n_vis - start < chunk ? n_vis - start : chunk);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int entry0 = kTileEntries * wave + (lane & 31);  // lane's entry in tile 0

    const ChunkKeys C = chunk_keys(codes, scales, b * n_cap + start, n_here, entry0, half);
    KeyTile ring[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p)
        load_key(C, p * kStep, ring[p]);
    __builtin_amdgcn_sched_barrier(0);
    QueryOperand Q;  // loaded while the first key tiles are in flight
    load_query(q + row * (kIdxHeads * kIdxDim), w + row * kIdxHeads, lane, Q);

    const bool writer = lane < 32 && (lane & 7) == 0;
    const int blk0 = entry0 / kBlock;  // chunk block of the lane's entry in tile 0
    const int groups = (n_here + kGroupEntries - 1) / kGroupEntries;
    auto finish = [&](int i, float s) {
        const int e = entry0 + i * kStep;
        s = e < n_here ? s : -INFINITY;
        if (kScores && lane < 32 && e < n_here)
            scores[row * n_cap + start + e] = s;
        const float m = max8(s);
        if (writer)
            sblk[blk0 + i * (kStep / kBlock)] = m;
    };
    for (int g = 0; g < groups - 1; ++g) {
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            const int i = g * kPrefetch + p;
            const float s = score_entry(Q, ring[p]);
            load_key(C, (i + kPrefetch) * kStep, ring[p]);
            finish(i, s);
        }
    }
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
        const int i = (groups - 1) * kPrefetch + p;
        finish(i, score_entry(Q, ring[p]));
    }
    __syncthreads();
    const int nb_here = (n_here + kBlock - 1) / kBlock;
    float* dst = block_max + row * nblk_cap + start / kBlock;
    for (int t = threadIdx.x; t < nb_here; t += kWaves * kWave)
        dst[t] = sblk[t];
    if (gkey != nullptr)
        write_group_keys(sblk, nb_here, row, start, chunk, gshift, ngroups, gkey);
    if (cand_key != nullptr)
        write_candidates(sblk, nb_here, start / kBlock, kl, cand_key + cslot, cand_blk + cslot,
                         cand_full + blockIdx.x);
}

// Full-range scan of two query rows of one sequence (rows 2p and 2p + 1 of
// its nq; the second is absent when nq is odd): the many-row (prefill) form.
// Each key tile is loaded and dequantised once for both rows, which halves
// the dequantisation per score, the VALU work that bounds the one-row scan
// when its keys come from the caches rather than HBM.  Same chunking, key
// ring, masking and outputs per row as index_full_kernel; a row whose visible
// range ends before the chunk writes nothing for it.  Two waves per SIMD (the
// two queries' operands and accumulators take twice the registers).
template <bool kScores>
__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
index_full_pair_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                       const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       int64_t n_cap, const int32_t* __restrict__ n_visible, int32_t nq,
                       int32_t pairs_per_seq, int32_t chunk, int32_t chunks_per_pair,
                       int64_t nblk_cap, float* __restrict__ block_max,
                       float* __restrict__ scores, uint32_t* __restrict__ gkey, int32_t gshift,
                       int64_t ngroups)
{
    __shared__ float sblk[2][kMaxChunk / kBlock];

    const int64_t pair = blockIdx.x / chunks_per_pair;
    const int64_t b = pair / pairs_per_seq;
    const int64_t i0 = 2 * (pair % pairs_per_seq);
    const bool two = i0 + 1 < nq;
    const int64_t row0 = b * nq + i0;
    const int64_t row1 = two ? row0 + 1 : row0;
    int64_t nv0 = n_visible[row0];
    nv0 = nv0 < 0 ? 0 : (nv0 > n_cap ? n_cap : nv0);
    int64_t nv1 = two ? (int64_t)n_visible[row1] : 0;
    nv1 = nv1 < 0 ? 0 : (nv1 > n_cap ? n_cap : nv1);
    const int64_t start = (int64_t)(blockIdx.x % chunks_per_pair) * chunk;
    const int64_t nv_max = nv0 > nv1 ? nv0 : nv1;
    if (start >= nv_max) {
        if (gkey != nullptr) {
            write_group_keys(sblk[0], 0, row0, start, chunk, gshift, ngroups, gkey);
            if (two)
                write_group_keys(sblk[1], 0, row1, start, chunk, gshift, ngroups, gkey);
        }
        return;
    }
    auto here = [&](int64_t nv) {
        return (int32_t)(nv <= start ? 0 : (nv - start < chunk ? nv - start : chunk));
    };
    const int32_t n_here0 = here(nv0), n_here1 = here(nv1);
    const int32_t n_here = n_here0 > n_here1 ? n_here0 : n_here1;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int entry0 = kTileEntries * wave + (lane & 31);

    const ChunkKeys C = chunk_keys(codes, scales, b * n_cap + start, n_here, entry0, half);
    KeyTile ring[kPrefetch];
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p)
        load_key(C, p * kStep, ring[p]);
    __builtin_amdgcn_sched_barrier(0);
    QueryOperand Q0, Q1;
    load_query(q + row0 * (kIdxHeads * kIdxDim), w + row0 * kIdxHeads, lane, Q0);
    load_query(q + row1 * (kIdxHeads * kIdxDim), w + row1 * kIdxHeads, lane, Q1);

    const bool writer = lane < 32 && (lane & 7) == 0;
    const int blk0 = entry0 / kBlock;
    const int groups = (n_here + kGroupEntries - 1) / kGroupEntries;
    auto finish = [&](int i, float s0, float s1) {
        const int e = entry0 + i * kStep;
        s0 = e < n_here0 ? s0 : -INFINITY;
        s1 = e < n_here1 ? s1 : -INFINITY;
        if (kScores && lane < 32) {
            if (e < n_here0)
                scores[row0 * n_cap + start + e] = s0;
            if (e < n_here1)
                scores[row1 * n_cap + start + e] = s1;
        }
        const float m0 = max8(s0);
        const float m1 = max8(s1);
        if (writer) {
            sblk[0][blk0 + i * (kStep / kBlock)] = m0;
            sblk[1][blk0 + i * (kStep / kBlock)] = m1;
        }
    };
    for (int g = 0; g < groups - 1; ++g) {
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            const int i = g * kPrefetch + p;
            float s0, s1;
            score_entry2(Q0, Q1, ring[p], s0, s1);
            load_key(C, (i + kPrefetch) * kStep, ring[p]);
            finish(i, s0, s1);
        }
    }
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
        const int i = (groups - 1) * kPrefetch + p;
        float s0, s1;
        score_entry2(Q0, Q1, ring[p], s0, s1);
        finish(i, s0, s1);
    }
    __syncthreads();
    const int nb0 = (n_here0 + kBlock - 1) / kBlock;
    const int nb1 = (n_here1 + kBlock - 1) / kBlock;
    float* dst0 = block_max + row0 * nblk_cap + start / kBlock;
    float* dst1 = block_max + row1 * nblk_cap + start / kBlock;
    for (int t = threadIdx.x; t < nb0; t += kWaves * kWave)
        dst0[t] = sblk[0][t];
    for (int t = threadIdx.x; t < nb1; t += kWaves * kWave)
        dst1[t] = sblk[1][t];
    if (gkey != nullptr) {
        write_group_keys(sblk[0], nb0, row0, start, chunk, gshift, ngroups, gkey);
        if (two)
            write_group_keys(sblk[1], nb1, row1, start, chunk, gshift, ngroups, gkey);
    }
}

// Pool scan: score the positions of a list of blocks (4 blocks per tile).
// 8 tiles per wave: the most gathers in flight that still keep 3 waves per SIMD
// (168 VGPRs); measured 15-22 % faster than 4 on the prefill pool scans and
// equal on the decode one
#ifndef CSA2_POOL_TILES_PER_WAVE
#define CSA2_POOL_TILES_PER_WAVE 8
#endif
constexpr int kPoolTilesPerWave = CSA2_POOL_TILES_PER_WAVE;

__global__ void __launch_bounds__(kWaves * kWave)
index_pool_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                  const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t n_cap, const int32_t* __restrict__ blocks, int32_t n_blocks,
                  const int32_t* __restrict__ n_visible, int32_t nq, int32_t wgs_per_query,
                  float* __restrict__ pool_score, int32_t* __restrict__ pool_idx)
{
    const int64_t row = blockIdx.x / wgs_per_query;
    const int32_t part = blockIdx.x % wgs_per_query;
    const int64_t b = row / nq;
    int64_t n_vis = n_visible[row];
    n_vis = n_vis < 0 ? 0 : (n_vis > n_cap ? n_cap : n_vis);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t slots = (int64_t)n_blocks * kBlock;

    // with nothing visible the loads read the query row instead (8 KiB, always
    // valid: entry 0 of the tiled layout lies in its first 1552 bytes) and are
    // masked: every load below is unconditional, so all of a wave's loads are
    // in flight together
    const uint8_t* qrow_bytes = reinterpret_cast<const uint8_t*>(q + row * (kIdxHeads * kIdxDim));
    const uint8_t* kc = n_vis > 0 ? codes : qrow_bytes;
    const uint8_t* ks = n_vis > 0 ? scales : qrow_bytes;
    const int64_t f_seq = n_vis > 0 ? b * n_cap : 0;  // flat index of the sequence's entry 0
    const int32_t* blk = blocks + row * n_blocks;

    const int64_t first = ((int64_t)part * kWaves + wave) * kPoolTilesPerWave * kTileEntries;
    // every block id of this wave's tiles first, then every key
    int32_t bl[kPoolTilesPerWave];
#pragma unroll
    for (int i = 0; i < kPoolTilesPerWave; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        bl[i] = blk[(slot < slots ? slot : slots - 1) / kBlock];
    }
    int64_t pos[kPoolTilesPerWave];
    KeyTile K[kPoolTilesPerWave];
#pragma unroll
    for (int i = 0; i < kPoolTilesPerWave; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        const int64_t p = (int64_t)bl[i] * kBlock + slot % kBlock;
        pos[i] = (slot < slots && bl[i] >= 0 && p < n_vis) ? p : -1;
        load_key(kc, ks, f_seq + (pos[i] >= 0 ? pos[i] : 0), half, K[i]);
    }
    QueryOperand Q;  // loaded while the gathers are in flight
    load_query(q + row * (kIdxHeads * kIdxDim), w + row * kIdxHeads, lane, Q);
#pragma unroll
    for (int i = 0; i < kPoolTilesPerWave; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        if (slot - (lane & 31) >= slots)
            break;
        const float s = score_entry(Q, K[i]);
        if (lane < 32 && slot < slots) {
            pool_score[row * slots + slot] = pos[i] >= 0 ? s : -INFINITY;
            pool_idx[row * slots + slot] = (int32_t)pos[i];
        }
    }
}

// Pool rescoring and its top-k in one launch ([N] 2.2, [A] 3.4: the pool's
// positions rescored with the layer's own query, then its top-k).  Workgroups
// of 16 waves, kPtT tiles of 32 slots per wave, wgs_per_row workgroups per
// row.  Every workgroup scores its slots exactly as index_pool_kernel (same
// score function: bit-identical scores), stores (score, position) with
// write-through stores (coherent at device scope without a cache flush),
// waits for them, and counts itself in the row's arrival counter; the last
// workgroup to arrive reads the row's slots back (device-coherent loads),
// selects the top-k as csa2_topk does over (pool_score, pool_idx), writes it,
// and returns the counter to zero for the next call.  Nothing waits on
// another workgroup, so the kernel ends whatever the dispatch order.
constexpr int kPtWaves = 16;
constexpr int kPtThreads = kPtWaves * kWave;

__device__ __forceinline__ void store_coherent(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p)
{
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

struct PoolTopkSmem {
    sel::Smem<kPtThreads> sm;
    uint32_t last;
};

template <int kPtT, int P>
__global__ void __launch_bounds__(kPtThreads)
pool_topk_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                 const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                 int64_t n_cap, const int32_t* __restrict__ blocks, int32_t n_blocks,
                 const int32_t* __restrict__ n_visible, int32_t nq, int32_t wgs_per_row,
                 int32_t k, int32_t* __restrict__ out, uint32_t* __restrict__ counters,
                 uint32_t* __restrict__ ws_score, uint32_t* __restrict__ ws_idx)
{
    __shared__ PoolTopkSmem ps;
    const int64_t row = blockIdx.x / wgs_per_row;
    const int32_t part = blockIdx.x % wgs_per_row;
    const int64_t b = row / nq;
    int64_t n_vis = n_visible[row];
    n_vis = n_vis < 0 ? 0 : (n_vis > n_cap ? n_cap : n_vis);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int64_t slots = (int64_t)n_blocks * kBlock;

    // scoring, as index_pool_kernel (loads with nothing visible read the query row)
    const uint8_t* qrow_bytes = reinterpret_cast<const uint8_t*>(q + row * (kIdxHeads * kIdxDim));
    const uint8_t* kc = n_vis > 0 ? codes : qrow_bytes;
    const uint8_t* ks = n_vis > 0 ? scales : qrow_bytes;
    const int64_t f_seq = n_vis > 0 ? b * n_cap : 0;
    const int32_t* blk = blocks + row * n_blocks;
    const int64_t first = ((int64_t)part * kPtWaves + wave) * kPtT * kTileEntries;
    int32_t bl[kPtT];
#pragma unroll
    for (int i = 0; i < kPtT; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        bl[i] = blk[(slot < slots ? slot : slots - 1) / kBlock];
    }
    int64_t pos[kPtT];
    KeyTile K[kPtT];
#pragma unroll
    for (int i = 0; i < kPtT; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        const int64_t p = (int64_t)bl[i] * kBlock + slot % kBlock;
        pos[i] = (slot < slots && bl[i] >= 0 && p < n_vis) ? p : -1;
        load_key(kc, ks, f_seq + (pos[i] >= 0 ? pos[i] : 0), half, K[i]);
    }
    QueryOperand Q;
    load_query(q + row * (kIdxHeads * kIdxDim), w + row * kIdxHeads, lane, Q);
    uint32_t* srow = ws_score + row * slots;
    uint32_t* irow = ws_idx + row * slots;
#pragma unroll
    for (int i = 0; i < kPtT; ++i) {
        const int64_t slot = first + i * kTileEntries + (lane & 31);
        if (slot - (lane & 31) >= slots)
            break;
        const float s = score_entry(Q, K[i]);
        if (lane < 32 && slot < slots) {
            store_coherent(srow + slot, __float_as_uint(pos[i] >= 0 ? s : -INFINITY));
            store_coherent(irow + slot, (uint32_t)(int32_t)pos[i]);
        }
    }
    // every store of this workgroup has completed before it counts itself
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (tid == 0)
        ps.last = __hip_atomic_fetch_add(counters + row, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(wgs_per_row - 1);
    __syncthreads();
    if (ps.last == 0u)
        return;
    if (tid == 0)
        store_coherent(counters + row, 0u);  // every workgroup of the row has arrived
    __asm__ volatile("" ::: "memory");

    // the last workgroup: top-k over the row's slots (csa2_topk's order and output)
    uint32_t key[P];
    int32_t id[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int64_t e = (int64_t)kPtThreads * i + tid;
        const uint32_t sb = e < slots ? load_coherent(srow + e) : 0u;
        const int32_t ix = e < slots ? (int32_t)load_coherent(irow + e) : -1;
        const float f = __uint_as_float(sb);
        id[i] = ix;
        key[i] = ix >= 0 && !__builtin_isnan(f) ? order_key(f) : 0u;
    }
    sel::clear_hist(ps.sm, tid);
    const sel::Pick pk = sel::find_threshold<P, kPtThreads>(key, (uint32_t)k, ps.sm, tid, lane, wave);
    bool take[P];
    uint32_t off[P];
    const uint32_t chosen = sel::place<P, kPtThreads>(key, pk, take, off, ps.sm, lane, wave);
    int32_t* orow = out + row * k;
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (take[i] && off[i] < (uint32_t)k)
            orow[off[i]] = id[i];
    for (uint32_t p = chosen + tid; p < (uint32_t)k; p += kPtThreads)
        orow[p] = -1;
}

template <typename T>
struct same_type {
    using type = T;
};

// Launch of a scan kernel; with timing events, through hipExtLaunchKernel so
// that the dispatch itself records them at the kernel's start and end.
template <typename... P>
hipError_t launch_scan(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                       hipEvent_t ev_start, hipEvent_t ev_stop,
                       typename same_type<P>::type... args)
{
    if (ev_start != nullptr || ev_stop != nullptr) {
        void* a[] = {static_cast<void*>(&args)...};
        return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, a, 0, stream,
                                  ev_start, ev_stop, 0);
    }
    kernel<<<grid, block, 0, stream>>>(args...);
    return hipGetLastError();
}

}  // namespace

ScanShape scan_shape(int64_t n_cap, int32_t B, int32_t nq)
{
    ScanShape sh{0, 0, 0, false};
    if (nq >= kPairMinRows) {
        const int32_t pairs_per_seq = (nq + 1) / 2;
        const int64_t pairs = (int64_t)B * pairs_per_seq;
        int32_t chunk = kMaxChunk;
        while (chunk > kGroupEntries &&
               pairs * ((n_cap + chunk - 1) / chunk) < kScanTargetWorkgroups)
            chunk /= 2;
        sh.chunk = chunk;
        sh.chunks_per_row = (int32_t)((n_cap + chunk - 1) / chunk);
        sh.paired = true;
        sh.max_blocks_per_chunk = chunk / kBlock;
        return sh;
    }
    const int64_t rows = (int64_t)B * nq;
#ifdef CSA2_SCAN_EVEN_CHUNKS
    // chunk = the even share of the target workgroup count, in whole prefetch rounds
    int64_t want = (rows * n_cap + kScanTargetWorkgroups - 1) / kScanTargetWorkgroups;
    want = (want + kGroupEntries - 1) / kGroupEntries * kGroupEntries;
    int32_t chunk = (int32_t)(want < kGroupEntries ? kGroupEntries : (want > kMaxChunk ? kMaxChunk : want));
#else
    int32_t chunk = kMaxChunk;
    while (chunk > kGroupEntries && rows * ((n_cap + chunk - 1) / chunk) < kScanTargetWorkgroups)
        chunk /= 2;
#endif
    sh.chunk = chunk;
    sh.chunks_per_row = (int32_t)((n_cap + chunk - 1) / chunk);
    sh.max_blocks_per_chunk = chunk / kBlock;
    return sh;
}

hipError_t launch_index_full(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* n_visible,
                             int32_t B, int32_t nq, float* block_max, float* scores,
                             uint32_t* group_keys, int32_t group, hipEvent_t ev_start,
                             hipEvent_t ev_stop, hipStream_t stream, uint32_t* cand_key,
                             int32_t* cand_blk, int32_t* cand_full, int32_t kl)
{
    const int64_t nblk_cap = (n_cap + kBlock - 1) / kBlock;
    int32_t gshift = 0;  // group = 1 << gshift (a power of two dividing 64)
    while (group_keys != nullptr && (1 << gshift) < group)
        ++gshift;
    const int64_t ngroups = (nblk_cap + (1 << gshift) - 1) >> gshift;
    if (nq >= kPairMinRows) {
        // many rows per sequence (prefill): two rows per workgroup
        const int32_t pairs_per_seq = (nq + 1) / 2;
        const int64_t pairs = (int64_t)B * pairs_per_seq;
        int32_t chunk = kMaxChunk;
        while (chunk > kGroupEntries &&
               pairs * ((n_cap + chunk - 1) / chunk) < kScanTargetWorkgroups)
            chunk /= 2;
        const int64_t chunks = (n_cap + chunk - 1) / chunk;
        const int64_t grid = pairs * chunks;
        if (grid == 0)
            return hipSuccess;
        return launch_scan(scores != nullptr ? index_full_pair_kernel<true>
                                             : index_full_pair_kernel<false>,
                           dim3((uint32_t)grid), dim3(kWaves * kWave), stream, ev_start, ev_stop,
                           reinterpret_cast<const uint16_t*>(q), w, k_codes, k_scales, n_cap,
                           n_visible, nq, pairs_per_seq, chunk, (int32_t)chunks, nblk_cap,
                           block_max, scores, group_keys, gshift, ngroups);
    }
    const int64_t rows = (int64_t)B * nq;
    const ScanShape sh = scan_shape(n_cap, B, nq);
    const int32_t chunk = sh.chunk;
    const int64_t chunks = sh.chunks_per_row;
    const int64_t grid = rows * chunks;
    if (grid == 0)
        return hipSuccess;
    if (cand_key == nullptr)
        kl = 0;
    return launch_scan(scores != nullptr ? index_full_kernel<true> : index_full_kernel<false>,
                       dim3((uint32_t)grid), dim3(kWaves * kWave), stream, ev_start, ev_stop, q, w,
                       k_codes, k_scales, n_cap, n_visible, nq, chunk, (int32_t)chunks, nblk_cap,
                       block_max, scores, group_keys, gshift, ngroups, cand_key, cand_blk,
                       cand_full, kl);
}

size_t pool_topk_workspace(int32_t rows, int32_t n_blocks)
{
    const size_t slots = (size_t)n_blocks * kBlock;
    const size_t cnt = ((size_t)rows * 4 + 255) / 256 * 256;
    return cnt + 2 * (((size_t)rows * slots * 4 + 255) / 256 * 256);
}

hipError_t launch_pool_topk(const uint16_t* q, const float* w, const uint8_t* k_codes,
                            const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                            int32_t n_blocks, const int32_t* n_visible, int32_t B, int32_t nq,
                            int32_t k, int32_t* out, void* ws, hipStream_t stream)
{
    const int64_t rows = (int64_t)B * nq;
    const int64_t slots = (int64_t)n_blocks * kBlock;
    if (rows == 0)
        return hipSuccess;
    char* base = static_cast<char*>(ws);
    uint32_t* counters = reinterpret_cast<uint32_t*>(base);
    const size_t cnt = ((size_t)rows * 4 + 255) / 256 * 256;
    uint32_t* sc = reinterpret_cast<uint32_t*>(base + cnt);
    uint32_t* ix = reinterpret_cast<uint32_t*>(base + cnt + ((size_t)rows * slots * 4 + 255) / 256 * 256);
    // one tile per wave for the decode pool sizes, two for longer pools
    const int tpw = slots <= 4096 ? 1 : 2;
    const int64_t per_wg = (int64_t)kPtWaves * tpw * kTileEntries;
    const int64_t wgs = slots > 0 ? (slots + per_wg - 1) / per_wg : 1;
    const dim3 grid((uint32_t)(rows * wgs)), block(kPtThreads);
#define CSA2_POOL_TOPK(T, P)                                                                     \
    pool_topk_kernel<T, P><<<grid, block, 0, stream>>>(q, w, k_codes, k_scales, n_cap, blocks,   \
                                                       n_blocks, n_visible, nq, (int32_t)wgs, k, \
                                                       out, counters, sc, ix)
    if (slots <= 4 * kPtThreads)
        CSA2_POOL_TOPK(1, 4);
    else if (slots <= 8 * kPtThreads)
        CSA2_POOL_TOPK(2, 8);
    else
        CSA2_POOL_TOPK(2, 16);
#undef CSA2_POOL_TOPK
    return hipGetLastError();
}

hipError_t launch_index_pool(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                             int32_t n_blocks, const int32_t* n_visible, int32_t B, int32_t nq,
                             float* pool_score, int32_t* pool_idx, hipStream_t stream)
{
    const int64_t slots = (int64_t)n_blocks * kBlock;
    const int64_t per_wg = (int64_t)kWaves * kPoolTilesPerWave * kTileEntries;
    const int64_t wgs = (slots + per_wg - 1) / per_wg;
    const int64_t grid = (int64_t)B * nq * wgs;
    if (grid == 0)
        return hipSuccess;
    index_pool_kernel<<<dim3((uint32_t)grid), dim3(kWaves * kWave), 0, stream>>>(
        q, w, k_codes, k_scales, n_cap, blocks, n_blocks, n_visible, nq, (int32_t)wgs,
        pool_score, pool_idx);
    return hipGetLastError();
}

}  // namespace csa2
