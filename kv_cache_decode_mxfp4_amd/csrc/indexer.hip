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
// Query rows per sequence from which the scan takes several rows per
// workgroup (prefill shapes); decode (one row per sequence) streams its keys
// from HBM, one row each.
#ifndef CSA2_SCAN_MULTI_MIN_ROWS
#define CSA2_SCAN_MULTI_MIN_ROWS 2
#endif
constexpr int32_t kMultiMinRows = CSA2_SCAN_MULTI_MIN_ROWS;

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

// Keys of one sequence for the pool gathers: buffer descriptors over the key
// tiles and scale rows of its visible entries, addressed with 32-bit offsets
// from the tile holding its entry 0 (the boundary keeps a gathering call's
// sequences at 2^24 entries or fewer, so every offset is below 2^31).  A
// position past the visible end, and every position of a sequence with
// nothing visible, reads zeros.  The loads go through the caches: in
// prefill every row's pool gathers from the same sequence.
struct SeqKeys {
    __amdgpu_buffer_rsrc_t codes, scales;
    int32_t e0;  // position of the sequence's entry 0 inside its tile
};

__device__ __forceinline__ SeqKeys seq_keys(const uint8_t* codes, const uint8_t* scales,
                                            int64_t f_seq, int32_t n_vis)
{
    SeqKeys S;
    const int64_t t0 = f_seq >> 5;
    const int64_t t_end = (f_seq + n_vis + kKeyTile - 1) >> 5;
    S.codes = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes + t0 * kKeyTileBytes), 0,
        n_vis > 0 ? (int32_t)((t_end - t0) * kKeyTileBytes) : 0, kBufferConfig);
    S.scales = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + f_seq * (kIdxDim / 16)), 0, n_vis * (kIdxDim / 16),
        kBufferConfig);
    S.e0 = (int32_t)(f_seq & 31);
    return S;
}

// Key at position p of the sequence, channel half `half`.
__device__ __forceinline__ void gather_key(const SeqKeys& S, int32_t p, int half, KeyTile& K)
{
    const int32_t e = S.e0 + p;
    const int32_t oc = (e >> 5) * kKeyTileBytes + 2 * half * kKeyPlane + (e & 31) * 16;
    K.c0 = __builtin_amdgcn_raw_buffer_load_b128(S.codes, oc, 0, 0);
    K.c1 = __builtin_amdgcn_raw_buffer_load_b128(S.codes, oc + kKeyPlane, 0, 0);
    K.sc = __builtin_amdgcn_raw_buffer_load_b32(S.scales, p * (kIdxDim / 16) + 4 * half, 0, 0);
}

// Gathers of one wave's kT pool tiles (slots first + 32 t + lane % 32): pos[t]
// = the slot's position in the sequence, -1 for a slot past the pool, a
// negative block id or a position past the visible end; every load is issued
// (masked slots read position 0), so all of them are in flight together.
template <int kT>
__device__ __forceinline__ void gather_pool_tiles(const SeqKeys& S, const int32_t* __restrict__ blk,
                                                  int32_t slots, int32_t n_vis, int32_t first,
                                                  int lane, int half, int32_t (&pos)[kT],
                                                  KeyTile (&K)[kT])
{
    const int32_t nb_vis = (n_vis + kBlock - 1) / kBlock;
    int32_t bl[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        const int32_t slot = first + t * kTileEntries + (lane & 31);
        bl[t] = blk[(slot < slots ? slot : slots - 1) / kBlock];
    }
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        const int32_t slot = first + t * kTileEntries + (lane & 31);
        // only a checked block id (0 <= bl < nb_vis <= 2^21) is multiplied
        const bool in = slot < slots && bl[t] >= 0 && bl[t] < nb_vis;
        const int32_t p = (in ? bl[t] : 0) * kBlock + slot % kBlock;
        pos[t] = in && p < n_vis ? p : -1;
        gather_key(S, pos[t] >= 0 ? pos[t] : 0, half, K[t]);
    }
}

// Maximum over the 8 lanes of each aligned group of 8 (DPP: swap neighbours,
// swap pairs, then mirror within the half-row of 8).  Each level is one
// v_max_f32 with the DPP lane move folded in: written through fmaxf the
// compiler adds a move and a canonicalisation of the moved value per level.
// v_max_f32 returns the other operand for one NaN and NaN for two, as fmaxf.
// The s_nop gives the two wait states a DPP read of a just-written VGPR needs.
#define CSA2_MAX_DPP(m, ctrl) \
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf" : "=v"(m) : "v"(m))
__device__ __forceinline__ float max8(float s)
{
    float m = s;
    CSA2_MAX_DPP(m, "quad_perm:[1,0,3,2]");
    CSA2_MAX_DPP(m, "quad_perm:[2,3,0,1]");
    CSA2_MAX_DPP(m, "row_half_mirror");
    return m;
}
#undef CSA2_MAX_DPP

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
    // every entry of the groups before the last is visible ((groups - 1) *
    // kGroupEntries < n_here), so only the last group masks
    auto finish = [&](int i, float s, bool last_group) {
        const int e = entry0 + i * kStep;
        if (last_group)
            s = e < n_here ? s : -INFINITY;
        if (kScores && lane < 32 && e < n_here)
            scores[row * n_cap + start + e] = s;
        const float m = max8(s);
        if (writer)
            sblk[blk0 + i * (kStep / kBlock)] = m;
    };
    // A CU issues the oldest workgroups' waves first, so on long chunks the
    // youngest fall far behind and the launch ends with few waves left.  Each
    // wave lowers its issue priority at every quarter of its chunk, so a wave
    // that is ahead yields to one that is behind (measured on 16384-entry
    // chunks: 1-3 % faster; on chunks of 8 prefetch rounds or fewer slower,
    // so those keep the default).
    // (a short chunk puts its quarter points out of reach: one priority throughout)
    const int never = groups < 16 ? groups : 0;
    const int q1 = groups / 4 + never, q2 = groups / 2 + never, q3 = 3 * groups / 4 + never;
    __builtin_amdgcn_s_setprio(3);
    for (int g = 0; g < groups - 1; ++g) {
        if (g == q1)
            __builtin_amdgcn_s_setprio(2);
        else if (g == q2)
            __builtin_amdgcn_s_setprio(1);
        else if (g == q3)
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int p = 0; p < kPrefetch; ++p) {
            const int i = g * kPrefetch + p;
            const float s = score_entry(Q, ring[p]);
            load_key(C, (i + kPrefetch) * kStep, ring[p]);
            finish(i, s, false);
        }
    }
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
        const int i = (groups - 1) * kPrefetch + p;
        finish(i, score_entry(Q, ring[p]), true);
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

// Full-range scan of up to kRowGroup query rows of one sequence (the many-row,
// prefill form): each 32-entry key tile is loaded and dequantised once by the
// whole workgroup into an LDS tile, from which every wave takes its MFMA B
// operands for two rows.  The dequantisation is then shared by 8 rows
// (against 2 when each wave dequantised its own tiles for two rows: 23 %
// fewer VALU instructions), leaving the per-row epilogue (the weighted ReLU
// head sum) as the VALU work per score.  Each row's MFMA chain is the one
// score_entry runs (the same A operand, the same exactly dequantised B values,
// the same k-step order), so the scores are bit-identical to the one-row
// scan's.  Tiles are double-buffered: one barrier per tile.  Rows past nq or
// whose visible range ends before the chunk write nothing for it.
constexpr int kRowGroup = 2 * kWaves;              // query rows per workgroup (two per wave)
#ifndef CSA2_ROWS_CHUNK
#define CSA2_ROWS_CHUNK 4096
#endif
constexpr int kRowsChunk = CSA2_ROWS_CHUNK;        // entries per workgroup
// whole groups of group keys (up to 64 blocks per group) per chunk
static_assert(kRowsChunk % 512 == 0, "chunks start on 64-block group boundaries");
constexpr int kTileRow = kIdxDim + 8;              // halves per LDS row of a key tile (272 B)
// Raw key tiles in flight (the prefill keys come from the caches: 2 measured
// 2-5 % faster than 4, 8 no better)
#ifndef CSA2_ROWS_PREFETCH
#define CSA2_ROWS_PREFETCH 2
#endif
constexpr int kRowsPrefetch = CSA2_ROWS_PREFETCH;

template <bool kScores>
__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(2)))
index_full_rows_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                       const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                       int64_t n_cap, const int32_t* __restrict__ n_visible, int32_t nq,
                       int32_t groups_per_seq, int32_t chunks_per_group, int64_t nblk_cap,
                       float* __restrict__ block_max, float* __restrict__ scores,
                       uint32_t* __restrict__ gkey, int32_t gshift, int64_t ngroups)
{
    __shared__ _Float16 tile[2][kTileEntries][kTileRow];
    __shared__ float sblk[kRowGroup][kRowsChunk / kBlock];
    __shared__ float spare[2][kWaves * kWave];  // block-max stores of lanes that own none

    const int64_t grp = blockIdx.x / chunks_per_group;
    const int64_t b = grp / groups_per_seq;
    const int64_t i0 = (int64_t)kRowGroup * (grp % groups_per_seq);
    const int64_t start = (int64_t)(blockIdx.x % chunks_per_group) * kRowsChunk;
    // visible entries of row slot r in this chunk (0 for a slot past nq)
    auto here = [&](int r) -> int32_t {
        if (i0 + r >= nq)
            return 0;
        int64_t nv = n_visible[b * nq + i0 + r];
        nv = nv < 0 ? 0 : (nv > n_cap ? n_cap : nv);
        return (int32_t)(nv <= start ? 0 : (nv - start < kRowsChunk ? nv - start : kRowsChunk));
    };
    int32_t n_max = 0;
#pragma unroll
    for (int r = 0; r < kRowGroup; ++r)
        n_max = max(n_max, here(r));
    if (n_max == 0) {
        if (gkey != nullptr)
            for (int r = 0; r < kRowGroup && i0 + r < nq; ++r)
                write_group_keys(sblk[r], 0, b * nq + i0 + r, start, kRowsChunk, gshift, ngroups,
                                 gkey);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int ent = lane & 31;  // the lane's entry in a tile (MFMA column)

    // key bytes of the chunk (range-checked: loads past the visible end read zeros)
    const int64_t f0 = b * n_cap + start;
    const int64_t t0 = f0 >> 5;
    const int64_t t_end = (f0 + n_max + kKeyTile - 1) >> 5;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(codes + t0 * kKeyTileBytes), 0,
        (int32_t)((t_end - t0) * kKeyTileBytes), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(scales + f0 * (kIdxDim / 16)), 0, n_max * (kIdxDim / 16),
        kBufferConfig);
    // dequantisation share of thread T: entry T % 32 of each tile, channels
    // [16 cg, 16 cg + 16) with cg = T / 32 (code bytes [8 cg, 8 cg + 8), scale byte cg)
    const int de = threadIdx.x & 31;
    const int dcg = threadIdx.x >> 5;
    const int e_in = (int)(f0 & 31) + de;  // the thread's entry counted from tile t0's first
    const int32_t voc = (e_in >> 5) * kKeyTileBytes + (dcg >> 1) * kKeyPlane + (e_in & 31) * 16 +
                        8 * (dcg & 1);
    const int32_t vos = de * (kIdxDim / 16) + (dcg & ~3);
    uint2 raw_c[kRowsPrefetch];
    uint32_t raw_s[kRowsPrefetch];
    // cached loads (no non-temporal hint): the sequence's other row groups read
    // the same keys (measured 0.3-0.5 % faster)
    auto load_raw = [&](int j, int u) {
        const auto c = __builtin_amdgcn_raw_buffer_load_b64(rc, voc + j * kKeyTileBytes, 0, 0);
        raw_c[u] = make_uint2(c[0], c[1]);
        raw_s[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, vos + j * kTileEntries * (kIdxDim / 16),
                                                        0, 0);
    };
    auto dequant_store = [&](int u, int buf) {
        const _Float16 s = e4m3_byte_to_f16(raw_s[u] >> (8 * (dcg & 3)), 0);
        half8* dst = reinterpret_cast<half8*>(&tile[buf][de][16 * dcg]);
        dst[0] = dequant8_fp4(raw_c[u].x, s);
        dst[1] = dequant8_fp4(raw_c[u].y, s);
    };
#pragma unroll
    for (int u = 0; u < kRowsPrefetch; ++u)
        load_raw(u, u);
    __builtin_amdgcn_sched_barrier(0);

    // this wave's two rows (a slot past nq takes the group's first row and writes nothing)
    const int ra = 2 * wave, rb = 2 * wave + 1;
    const bool has_a = i0 + ra < nq, has_b = i0 + rb < nq;
    const int64_t row_a = b * nq + i0 + (has_a ? ra : 0);
    const int64_t row_b = b * nq + i0 + (has_b ? rb : 0);
    const int32_t nh_a = here(ra), nh_b = here(rb);
    QueryOperand Qa, Qb;
    load_query(q + row_a * (kIdxHeads * kIdxDim), w + row_a * kIdxHeads, lane, Qa);
    load_query(q + row_b * (kIdxHeads * kIdxDim), w + row_b * kIdxHeads, lane, Qb);

    const bool writer = lane < 32 && (lane & 7) == 0;
    const int ntiles = (n_max + kTileEntries - 1) / kTileEntries;
    // tile j's products go to accumulator pair j&1 and its epilogue runs in
    // the next body, beside tile j+1's products (the matrix cores then work
    // while the vector units finish the previous tile); pair 1 starts at zero
    // for the first body's epilogue of tile -1
    f32x16 acc_a[2] = {}, acc_b[2] = {};
    auto products = [&](int j) {
        const _Float16* src = &tile[j & 1][ent][64 * half];
        f32x16 xa = {}, xb = {};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const half8 bt = *reinterpret_cast<const half8*>(src + 8 * t);
            xa = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qa.a[t], bt, xa, 0, 0, 0);
            xb = __builtin_amdgcn_mfma_f32_32x32x16_f16(Qb.a[t], bt, xb, 0, 0, 0);
        }
        acc_a[j & 1] = xa;
        acc_b[j & 1] = xb;
    };
    auto epilogue = [&](int j) {  // j = -1: nothing to finish, the stores go to spare
        const int e = kTileEntries * j + ent;
        float sa = head_sum(Qa, acc_a[j & 1]), sb = head_sum(Qb, acc_b[j & 1]);
        sa = e < nh_a ? sa : -INFINITY;
        sb = e < nh_b ? sb : -INFINITY;
        if (kScores && lane < 32 && e >= 0) {
            if (e < nh_a)
                scores[row_a * n_cap + start + e] = sa;
            if (e < nh_b)
                scores[row_b * n_cap + start + e] = sb;
        }
        const float ma = max8(sa), mb = max8(sb);
        // every lane stores, so the body has no branch: a lane that owns no
        // block (or tile -1) stores into a spare slot of its own
        const bool own = writer && j >= 0;
        const int eb = max(e, 0) / kBlock;  // < kRowsChunk / kBlock: e < 32 * padded tiles
        *(own ? &sblk[ra][eb] : &spare[0][threadIdx.x]) = ma;
        *(own ? &sblk[rb][eb] : &spare[1][threadIdx.x]) = mb;
    };

    dequant_store(0, 0);
    load_raw(kRowsPrefetch, 0);
    __syncthreads();
    // slot u of the raw ring holds tile j0 + u; body j stores tile j + 1 into
    // the other LDS buffer (last read before the previous barrier), refills
    // its slot with tile j + 1 + kRowsPrefetch, runs tile j's products and
    // tile j-1's epilogue.  The bodies have no branch, so each is one
    // scheduling region: the tile count is rounded up to whole ring turns (at
    // most kRowsChunk / 32 tiles, so every LDS index stays in its array), and
    // padded tiles read zeros (range-checked loads) and score -inf.
    static_assert((kRowsChunk / kTileEntries) % kRowsPrefetch == 0, "padded tiles fit the chunk");
    const int ntiles_p = (ntiles + kRowsPrefetch - 1) / kRowsPrefetch * kRowsPrefetch;
    for (int j0 = 0; j0 < ntiles_p; j0 += kRowsPrefetch) {
#pragma unroll
        for (int u = 0; u < kRowsPrefetch; ++u) {
            const int j = j0 + u;
            const int next = (u + 1) % kRowsPrefetch;
            dequant_store(next, (j + 1) & 1);
            load_raw(j + 1 + kRowsPrefetch, next);
            products(j);
            epilogue(j - 1);
            // one MFMA, then up to five vector instructions, sixteen times
            // (measured 2-2.5 % faster than the compiler's own interleave)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
            }
            __syncthreads();
        }
    }
    epilogue(ntiles_p - 1);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRowGroup; ++r) {
        if (i0 + r >= nq)
            break;
        const int nb = (here(r) + kBlock - 1) / kBlock;
        float* dst = block_max + (b * nq + i0 + r) * nblk_cap + start / kBlock;
        for (int t = threadIdx.x; t < nb; t += kWaves * kWave)
            dst[t] = sblk[r][t];
        if (gkey != nullptr)
            write_group_keys(sblk[r], nb, b * nq + i0 + r, start, kRowsChunk, gshift, ngroups,
                             gkey);
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

__global__ void __launch_bounds__(kWaves * kWave) __attribute__((amdgpu_waves_per_eu(3)))
index_pool_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                  const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                  int64_t n_cap, const int32_t* __restrict__ blocks, int32_t n_blocks,
                  const int32_t* __restrict__ n_visible, int32_t nq, int32_t wgs_per_query,
                  float* __restrict__ pool_score, int32_t* __restrict__ pool_idx)
{
    const int64_t row = blockIdx.x / wgs_per_query;
    const int32_t part = blockIdx.x % wgs_per_query;
    const int64_t b = row / nq;
    int64_t nv = n_visible[row];
    const int32_t n_vis = (int32_t)(nv < 0 ? 0 : (nv > n_cap ? n_cap : nv));
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int32_t slots = n_blocks * kBlock;
    const int32_t first = (part * kWaves + wave) * kPoolTilesPerWave * kTileEntries;
    // the query first: prepared while the gathers are in flight it would hold
    // its conversion registers beside the gathered tiles (spills at 168 VGPRs)
    __shared__ QueryLds sq;
    QueryOperand Q;
    shared_query(q + row * (kIdxHeads * kIdxDim), w + row * kIdxHeads, lane, wave, sq, Q);
    int32_t pos[kPoolTilesPerWave];
    KeyTile K[kPoolTilesPerWave];
    gather_pool_tiles(seq_keys(codes, scales, b * n_cap, n_vis), blocks + row * n_blocks, slots,
                      n_vis, first, lane, half, pos, K);
    float* srow = pool_score + row * slots;
    int32_t* irow = pool_idx + row * slots;
#pragma unroll
    for (int i = 0; i < kPoolTilesPerWave; ++i) {
        const int32_t slot = first + i * kTileEntries + (lane & 31);
        if (slot - (lane & 31) >= slots)
            break;
        const float s = score_entry(Q, K[i]);
        if (lane < 32 && slot < slots) {
            srow[slot] = pos[i] >= 0 ? s : -INFINITY;
            irow[slot] = pos[i];
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
    QueryLds query;
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
    int64_t nv = n_visible[row];
    const int32_t n_vis = (int32_t)(nv < 0 ? 0 : (nv > n_cap ? n_cap : nv));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int32_t slots = n_blocks * kBlock;

    // scoring, as index_pool_kernel
    const int32_t first = (part * kPtWaves + wave) * kPtT * kTileEntries;
    int32_t pos[kPtT];
    KeyTile K[kPtT];
    gather_pool_tiles(seq_keys(codes, scales, b * n_cap, n_vis), blocks + row * n_blocks, slots,
                      n_vis, first, lane, half, pos, K);
    QueryOperand Q;
    shared_query(q + row * (kIdxHeads * kIdxDim), w + row * kIdxHeads, lane, wave, ps.query, Q);
    uint32_t* srow = ws_score + row * slots;
    uint32_t* irow = ws_idx + row * slots;
#pragma unroll
    for (int i = 0; i < kPtT; ++i) {
        const int32_t slot = first + i * kTileEntries + (lane & 31);
        if (slot - (lane & 31) >= slots)
            break;
        const float s = score_entry(Q, K[i]);
        if (lane < 32 && slot < slots) {
            store_coherent(srow + slot, __float_as_uint(pos[i] >= 0 ? s : -INFINITY));
            store_coherent(irow + slot, (uint32_t)pos[i]);
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
    if (nq >= kMultiMinRows) {
        sh.chunk = kRowsChunk;
        sh.chunks_per_row = (int32_t)((n_cap + kRowsChunk - 1) / kRowsChunk);
        sh.multi_row = true;
        sh.max_blocks_per_chunk = kRowsChunk / kBlock;
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

// Workgroups of the scan launch: one per chunk and row, or per chunk and group
// of 8 rows (multi-row form).
static int64_t scan_workgroups(int64_t n_cap, int32_t B, int32_t nq)
{
    const ScanShape sh = scan_shape(n_cap, B, nq);
    const int64_t row_units = sh.multi_row ? (int64_t)B * ((nq + kRowGroup - 1) / kRowGroup)
                                           : (int64_t)B * nq;
    return row_units * sh.chunks_per_row;
}

bool index_full_fits(int64_t n_cap, int32_t B, int32_t nq)
{
    return grid_fits(scan_workgroups(n_cap, B, nq), kWaves * kWave);
}

hipError_t launch_index_full(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* n_visible,
                             int32_t B, int32_t nq, float* block_max, float* scores,
                             uint32_t* group_keys, int32_t group, hipEvent_t ev_start,
                             hipEvent_t ev_stop, hipStream_t stream, uint32_t* cand_key,
                             int32_t* cand_blk, int32_t* cand_full, int32_t kl)
{
    const int64_t grid = scan_workgroups(n_cap, B, nq);
    if (grid == 0)
        return hipSuccess;
    if (!grid_fits(grid, kWaves * kWave))
        return hipErrorInvalidConfiguration;
    const int64_t nblk_cap = (n_cap + kBlock - 1) / kBlock;
    int32_t gshift = 0;  // group = 1 << gshift (a power of two dividing 64)
    while (group_keys != nullptr && (1 << gshift) < group)
        ++gshift;
    const int64_t ngroups = (nblk_cap + (1 << gshift) - 1) >> gshift;
    if (nq >= kMultiMinRows) {
        // many rows per sequence (prefill): 8 rows per workgroup sharing each
        // dequantised key tile
        const int32_t groups_per_seq = (nq + kRowGroup - 1) / kRowGroup;
        const int64_t chunks = (n_cap + kRowsChunk - 1) / kRowsChunk;
        return launch_scan(scores != nullptr ? index_full_rows_kernel<true>
                                             : index_full_rows_kernel<false>,
                           dim3((uint32_t)grid), dim3(kWaves * kWave), stream, ev_start, ev_stop,
                           reinterpret_cast<const uint16_t*>(q), w, k_codes, k_scales, n_cap,
                           n_visible, nq, groups_per_seq, (int32_t)chunks, nblk_cap, block_max,
                           scores, group_keys, gshift, ngroups);
    }
    const ScanShape sh = scan_shape(n_cap, B, nq);
    const int32_t chunk = sh.chunk;
    const int64_t chunks = sh.chunks_per_row;
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

// Workgroups per row of the fused rescoring: one key tile per wave for the
// decode pool sizes, two for longer pools.
static int64_t pool_topk_wgs_per_row(int64_t slots)
{
    const int tpw = slots <= 4096 ? 1 : 2;
    const int64_t per_wg = (int64_t)kPtWaves * tpw * kTileEntries;
    return slots > 0 ? (slots + per_wg - 1) / per_wg : 1;
}

bool pool_topk_fits(int64_t rows, int32_t n_blocks)
{
    return grid_fits(rows * pool_topk_wgs_per_row((int64_t)n_blocks * kBlock), kPtThreads);
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
    const int64_t wgs = pool_topk_wgs_per_row(slots);
    if (!grid_fits(rows * wgs, kPtThreads))
        return hipErrorInvalidConfiguration;
    char* base = static_cast<char*>(ws);
    uint32_t* counters = reinterpret_cast<uint32_t*>(base);
    const size_t cnt = ((size_t)rows * 4 + 255) / 256 * 256;
    uint32_t* sc = reinterpret_cast<uint32_t*>(base + cnt);
    uint32_t* ix = reinterpret_cast<uint32_t*>(base + cnt + ((size_t)rows * slots * 4 + 255) / 256 * 256);
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

// Workgroups per row of the pool scan (kPoolTilesPerWave key tiles per wave).
static int64_t index_pool_wgs_per_row(int32_t n_blocks)
{
    const int64_t slots = (int64_t)n_blocks * kBlock;
    const int64_t per_wg = (int64_t)kWaves * kPoolTilesPerWave * kTileEntries;
    return (slots + per_wg - 1) / per_wg;
}

bool index_pool_fits(int64_t rows, int32_t n_blocks)
{
    return grid_fits(rows * index_pool_wgs_per_row(n_blocks), kWaves * kWave);
}

hipError_t launch_index_pool(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                             int32_t n_blocks, const int32_t* n_visible, int32_t B, int32_t nq,
                             float* pool_score, int32_t* pool_idx, hipStream_t stream)
{
    const int64_t wgs = index_pool_wgs_per_row(n_blocks);
    const int64_t grid = (int64_t)B * nq * wgs;
    if (grid == 0)
        return hipSuccess;
    if (!grid_fits(grid, kWaves * kWave))
        return hipErrorInvalidConfiguration;
    index_pool_kernel<<<dim3((uint32_t)grid), dim3(kWaves * kWave), 0, stream>>>(
        q, w, k_codes, k_scales, n_cap, blocks, n_blocks, n_visible, nq, (int32_t)wgs,
        pool_score, pool_idx);
    return hipGetLastError();
}

}  // namespace csa2
