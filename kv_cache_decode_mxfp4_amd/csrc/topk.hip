// Deterministic top-k select ([N] 1 of the DeepSeek-V4.1 reading notes: top-k
// 512; [N] 2.2 / [A] 3.4: the top-2048 blocks form the pool).
//
// Order: score descending, then position ascending (the lower index wins a
// tie); -0 equals +0; NaN and masked entries never win.  Output: the chosen
// indices in ascending order, -1 padded.
//
// Core: one workgroup of 1024 threads holds up to 16384 (key, index) pairs in
// registers, P per thread (slot i of thread t is element 1024*i + t, so loads
// are coalesced and position order is slot-major; P = 16, or 4 / 8 for rows of
// at most 4096 / 8192 keys, which skips the empty slots' work).  The k-th largest key is
// found by an adaptive-range radix select: each pass histograms the live key
// range [lo, hi] into at most 2048 equal LDS bins and keeps the bin holding the
// k-th key, shrinking the span by at least 2^11 (three passes at most; 2048
// bins, 2 per thread, keep a pass's prefix step short and the histograms at
// 16 KB — on score-like data 1-5 % faster than 4096 bins on rows of 4096 to
// 16384 keys, equal on the 1M-context block select, and faster than 1024).  Once the chosen bin holds at most 64
// keys (on score-like data, after the first pass) they are gathered into LDS
// and one wave ranks them against each other instead of running another
// pass, whose cost is the same per key however few keys are live.  One
// ballot round then gives every chosen entry its output offset:
//   offset = (#greater before it) + min(#equal before it, #equal to take).
//
// Longer rows:
//   grouped (g = ceil(L/16384) with k*g <= 16384): the row is cut into groups of
//     g consecutive entries; the top-k entries lie in the top-k groups ranked by
//     their largest key (a group ranked above a winner's group holds another
//     winner, also under the lower-position tie-break), so a wide kernel writes
//     the group maxima and one workgroup per row selects k groups, gathers
//     their k*g entries and selects k of those;
//   otherwise exact levels: every segment of 16384 emits its own top-k
//     candidates (the global top-k is a subset of their union, and the
//     candidate lists keep position order) until one segment remains.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "select.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kTopkSegment / kThreads;  // 16

using sel::key_value;
using sel::Pick;
using Smem = sel::Smem<kThreads>;

template <int P>
__device__ __forceinline__ Pick find_threshold(const uint32_t (&key)[P], uint32_t k, Smem& sm,
                                               int tid, int lane, int wave)
{
    return sel::find_threshold<P, kThreads>(key, k, sm, tid, lane, wave);
}

template <int P>
__device__ __forceinline__ uint32_t place(const uint32_t (&key)[P], Pick pk, bool (&take)[P],
                                          uint32_t (&off)[P], Smem& sm, int lane, int wave)
{
    return sel::place<P, kThreads>(key, pk, take, off, sm, lane, wave);
}

template <int P>
__device__ __forceinline__ void write_result(const bool (&take)[P], const uint32_t (&off)[P],
                                             const uint32_t (&key)[P], const int32_t (&id)[P],
                                             uint32_t chosen, int32_t k, int tid,
                                             int32_t* __restrict__ out, float* __restrict__ cs,
                                             int32_t* __restrict__ ci)
{
    if (cs == nullptr) {
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (take[i] && off[i] < (uint32_t)k)
                out[off[i]] = id[i];
        for (uint32_t p = chosen + tid; p < (uint32_t)k; p += kThreads)
            out[p] = -1;
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (take[i] && off[i] < (uint32_t)k) {
                cs[off[i]] = key_value(key[i]);
                ci[off[i]] = id[i];
            }
        for (uint32_t p = chosen + tid; p < (uint32_t)k; p += kThreads) {
            cs[p] = 0.0f;
            ci[p] = -1;
        }
    }
}

// Loads slot i of thread tid = element seg_start + 1024*i + tid (clamped
// inside the row, masked by position < seg_end, index >= 0 and not NaN).
template <int P>
__device__ __forceinline__ void load_slots(const float* __restrict__ srow,
                                           const int32_t* __restrict__ irow, int64_t L,
                                           int64_t seg_start, int64_t seg_end, int tid,
                                           uint32_t (&key)[P], int32_t (&id)[P])
{
    float f[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        int64_t pos = seg_start + (int64_t)kThreads * i + tid;
        pos = pos < L ? pos : L - 1;
        f[i] = srow[pos];
        id[i] = irow != nullptr ? irow[pos] : (int32_t)pos;
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int64_t pos = seg_start + (int64_t)kThreads * i + tid;
        const bool ok = pos < seg_end && id[i] >= 0 && !__builtin_isnan(f[i]);
        key[i] = ok ? order_key(f[i]) : 0u;
    }
}

// Valid prefix of a row: ceil(n_valid[row] / div) clamped to [0, L] (div = 8
// turns a count of visible entries into a count of visible blocks), or L.
__device__ __forceinline__ int64_t valid_prefix(const int32_t* __restrict__ n_valid, int64_t row,
                                                int64_t L, int32_t div)
{
    if (n_valid == nullptr)
        return L;
    int64_t nv = n_valid[row];
    nv = nv < 0 ? 0 : (nv + div - 1) / div;
    return nv > L ? L : nv;
}

// Direct select within segments of up to 1024 * P entries (P slots per
// thread; short rows take a smaller P, which drops the empty slots' ballots,
// histogram adds and scans).  Grid: rows * nseg.
// Final mode (cand_score == nullptr): out[row, 0..k) = ascending indices.
// Candidate mode: cand_score/cand_idx[row, seg, 0..k) = chosen (score, index)
// pairs in position order, padded with index -1.
template <int P>
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ score, const int32_t* __restrict__ idx, int64_t L,
            int64_t seg_len, int32_t nseg, const int32_t* __restrict__ n_valid,
            int32_t valid_div, int32_t k,
            int32_t* __restrict__ out, float* __restrict__ cand_score,
            int32_t* __restrict__ cand_idx)
{
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x / nseg;
    const int64_t seg = blockIdx.x % nseg;
    const int64_t nv = valid_prefix(n_valid, row, L, valid_div);
    const int64_t seg_start = seg * seg_len;
    const int64_t seg_end = seg_start + seg_len < nv ? seg_start + seg_len : nv;
    sel::clear_hist(sm, tid);

    uint32_t key[P];
    int32_t id[P];
    if (L > 0) {
        load_slots(score + row * L, idx != nullptr ? idx + row * L : nullptr, L, seg_start,
                   seg_end, tid, key, id);
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) {
            key[i] = 0u;
            id[i] = -1;
        }
    }
    const Pick pk = find_threshold(key, (uint32_t)k, sm, tid, lane, wave);
    bool take[P];
    uint32_t off[P];
    const uint32_t chosen = place(key, pk, take, off, sm, lane, wave);
    write_result(take, off, key, id, chosen, k, tid, out + row * k,
                 cand_score ? cand_score + (row * nseg + seg) * k : nullptr,
                 cand_idx ? cand_idx + (row * nseg + seg) * k : nullptr);
}

// Group maxima of keys for the grouped path: gkey[row, grp] = largest key of
// entries [grp*g, grp*g + g) of the row (0 if none is valid).  One thread per
// group; grid: rows * ceil(ngroups / 256).
template <int G>
__global__ void __launch_bounds__(256)
group_max_kernel(const float* __restrict__ score, const int32_t* __restrict__ idx, int64_t L,
                 int32_t g_runtime, int64_t ngroups, int32_t wgs_per_row,
                 const int32_t* __restrict__ n_valid, int32_t valid_div,
                 uint32_t* __restrict__ gkey)
{
    const int g = G > 0 ? G : g_runtime;
    const int64_t row = blockIdx.x / wgs_per_row;
    const int64_t grp = (int64_t)(blockIdx.x % wgs_per_row) * 256 + threadIdx.x;
    if (grp >= ngroups)
        return;
    const int64_t nv = valid_prefix(n_valid, row, L, valid_div);
    const float* srow = score + row * L;
    const int32_t* irow = idx != nullptr ? idx + row * L : nullptr;
    uint32_t m = 0u;
    if (G > 0) {
        float f[G > 0 ? G : 1];
        int32_t ii[G > 0 ? G : 1];
#pragma unroll
        for (int r = 0; r < (G > 0 ? G : 1); ++r) {
            int64_t pos = grp * G + r;
            pos = pos < L ? pos : L - 1;
            f[r] = srow[pos];
            ii[r] = irow != nullptr ? irow[pos] : 0;
        }
#pragma unroll
        for (int r = 0; r < (G > 0 ? G : 1); ++r)
            if (grp * G + r < nv && ii[r] >= 0 && !__builtin_isnan(f[r]))
                m = max(m, order_key(f[r]));
    } else {
        for (int r = 0; r < g; ++r) {
            const int64_t pos = grp * g + r;
            if (pos < nv) {
                const float f = srow[pos];
                const int32_t ii = irow != nullptr ? irow[pos] : 0;
                if (ii >= 0 && !__builtin_isnan(f))
                    m = max(m, order_key(f));
            }
        }
    }
    gkey[row * ngroups + grp] = m;
}

// Group maxima for groups of 8 without an index array when rows are float4
// aligned (L % 4 == 0, 16-byte aligned scores): lane t of the grid loads the
// float4 of entries [4t, 4t+4) of the flattened rows, and the two lanes of a
// group combine through a DPP swap, so every load instruction is one
// contiguous 1 KiB.  Grid: ceil(rows * L / 4 / 256).
__global__ void __launch_bounds__(256)
group_max8_vec_kernel(const float* __restrict__ score, int64_t L, int64_t rows,
                      int64_t ngroups, const int32_t* __restrict__ n_valid, int32_t valid_div,
                      uint32_t* __restrict__ gkey)
{
    const int64_t quads_per_row = L / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t tc = t < rows * quads_per_row ? t : rows * quads_per_row - 1;
    const int64_t row = tc / quads_per_row;
    const int64_t pos = 4 * (tc % quads_per_row);
    const int64_t nv = valid_prefix(n_valid, row, L, valid_div);
    const float4 f = reinterpret_cast<const float4*>(score)[tc];
    const float v[4] = {f.x, f.y, f.z, f.w};
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (pos + j < nv && !__builtin_isnan(v[j]))
            m = max(m, order_key(v[j]));
    m = max(m, dpp_u32<0xB1>(0u, m));  // partner lane (xor 1): the other half of the group
    if ((threadIdx.x & 1) == 0 && t < rows * quads_per_row)
        gkey[row * ngroups + pos / 8] = m;
}

struct GroupSmem {
    Smem sm;
    uint32_t chosen_groups[kTopkSegment / 2];  // k <= 16384 / g with g >= 2
};

// The grouped select as an out-of-line call, for the block select's rare
// fallback: its registers then do not weigh on the common path's.
template <int kG>
__device__ __attribute__((noinline)) void grouped_select_row_call(
    const float* __restrict__ srow, int64_t nv, int32_t g_runtime, int64_t ngroups,
    const uint32_t* __restrict__ grow, int32_t k, int32_t* __restrict__ out, GroupSmem& gs);

// Grouped select of one row from its group maxima grow[0..ngroups) (ngroups
// <= 16384, g * k <= 16384) into out[0..k): the k best groups by their
// largest key, then the k best of those groups' g*k entries.  srow / irow:
// the row's keys and indices (irow null = positions), nv its valid prefix.
// kG: the group size when known at compile time (8: L up to 131072 with k <=
// 2048), else 0 (g_runtime).  Expects gs.sm.hist[0] cleared.
template <int kG>
__device__ void grouped_select_row(const float* __restrict__ srow,
                                   const int32_t* __restrict__ irow, int64_t nv,
                                   int32_t g_runtime, int64_t ngroups,
                                   const uint32_t* __restrict__ grow, int32_t k,
                                   int32_t* __restrict__ out, GroupSmem& gs, int tid, int lane,
                                   int wave)
{
    Smem& sm = gs.sm;
    const uint32_t g = kG > 0 ? (uint32_t)kG : (uint32_t)g_runtime;
    uint32_t key[kPer];
    int32_t id[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t grp = (int64_t)kThreads * i + tid;
        key[i] = grp < ngroups ? grow[grp] : 0u;
        id[i] = (int32_t)grp;
    }
    Pick pk = find_threshold(key, (uint32_t)k, sm, tid, lane, wave);
    bool take[kPer];
    uint32_t off[kPer];
    uint32_t chosen = place(key, pk, take, off, sm, lane, wave);
    // chosen group ids, ascending, into LDS
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (take[i] && off[i] < (uint32_t)k)
            gs.chosen_groups[off[i]] = (uint32_t)id[i];
    sel::clear_hist(sm, tid);
    __syncthreads();
    const uint32_t n_chosen = chosen < (uint32_t)k ? chosen : (uint32_t)k;
    // candidate c*g + r is entry r of the c-th chosen group: position order.
    // Every group id is read first, then every score (clamped, masked), so the
    // loads of all 16 slots are in flight together.
    uint32_t cg[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t c = (uint32_t)(kThreads * i + tid) / g;
        cg[i] = gs.chosen_groups[c < n_chosen ? c : 0u];
    }
    float f[kPer];
    int64_t pos[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t e = (uint32_t)(kThreads * i + tid);
        const uint32_t c = e / g;
        const int64_t p = (int64_t)cg[i] * g + (e - c * g);
        pos[i] = c < n_chosen && p < nv ? p : -1;
        f[i] = srow[pos[i] >= 0 ? pos[i] : 0];
    }
    if (irow != nullptr) {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            id[i] = irow[pos[i] >= 0 ? pos[i] : 0];
    } else {
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            id[i] = (int32_t)pos[i];
    }
    // A candidate below v, the k-th largest group key, cannot win: each of the
    // k chosen groups holds an entry >= v, so k entries rank above it.  Dropping
    // those candidates (ties at v stay) narrows the second search's range.
    const uint32_t keep = pk.need > 0u ? pk.T : pk.T + 1u;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const bool ok = pos[i] >= 0 && id[i] >= 0 && !__builtin_isnan(f[i]);
        const uint32_t kk = ok ? order_key(f[i]) : 0u;
        key[i] = kk >= keep ? kk : 0u;
        id[i] = pos[i] >= 0 ? id[i] : -1;
    }
    pk = find_threshold(key, (uint32_t)k, sm, tid, lane, wave);
    chosen = place(key, pk, take, off, sm, lane, wave);
    write_result(take, off, key, id, chosen, k, tid, out, nullptr, nullptr);
}

template <int kG>
__device__ __attribute__((noinline)) void grouped_select_row_call(
    const float* __restrict__ srow, int64_t nv, int32_t g_runtime, int64_t ngroups,
    const uint32_t* __restrict__ grow, int32_t k, int32_t* __restrict__ out, GroupSmem& gs)
{
    const int tid = threadIdx.x;
    grouped_select_row<kG>(srow, nullptr, nv, g_runtime, ngroups, grow, k, out, gs, tid, tid & 63,
                           tid >> 6);
}

// Grouped select for one row from its group maxima gkey[row, 0..ngroups)
// (ngroups <= 16384, g * k <= 16384).  Grid: rows.
template <int kG>
__global__ void __launch_bounds__(kThreads)
topk_grouped_kernel(const float* __restrict__ score, const int32_t* __restrict__ idx, int64_t L,
                    int32_t g_runtime, int64_t ngroups, const uint32_t* __restrict__ gkey,
                    const int32_t* __restrict__ n_valid, int32_t valid_div, int32_t k,
                    int32_t* __restrict__ out)
{
    __shared__ GroupSmem gs;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t nv = valid_prefix(n_valid, row, L, valid_div);
    sel::clear_hist(gs.sm, tid);
    grouped_select_row<kG>(score + row * L, idx != nullptr ? idx + row * L : nullptr, nv,
                           g_runtime, ngroups, gkey + row * ngroups, k, out + row * k, gs, tid,
                           lane, wave);
}

// ------------------------------------------------------------ block select
//
// Pool (top-nb blocks) and top-k blocks of one row in one workgroup ([N] 2.2,
// [A] 3.4: the pool holds the 2048 blocks with the largest block scores; the
// Full layer's top-k entries lie in its top-k blocks).  Keys come either
// straight from the row's block maxima (rows of at most 16384 blocks), or
// from the candidate lists the scan wrote: each scan chunk's kl best blocks
// in block order, plus a flag telling whether the chunk had more than kl
// valid blocks.
//
// The candidates' top-t (t = nb or k) is the row's top-t unless some chunk
// left blocks out that could outrank the t-th chosen candidate.  A chunk's
// left-out blocks all rank below its own lowest-ranked candidate u; if fewer
// than kl of the chunk's candidates are chosen, u is not chosen and so ranks
// below the t-th chosen candidate, as do the left-out blocks.  So the
// selection is exact unless a full chunk has all kl candidates chosen; then
// (rare on score-like data: a chunk holds about t / chunks of the winners,
// kl is at least twice that) the row falls back to the exact grouped select
// over the group maxima the scan also wrote.
struct BlockSelJob {
    const float* block_max;   // [rows, L] block maxima (fp32)
    int64_t L;                // block slots per row
    const int32_t* n_visible; // [rows] visible entries (valid blocks: ceil(n / 8))
    const uint32_t* gkey;     // [rows, ngroups] group maxima (order keys), groups of g
    int64_t ngroups;
    int32_t g;
    const uint32_t* cand_key; // [rows, chunks, kl] or null: the direct form
    const int32_t* cand_blk;
    const int32_t* cand_full; // [rows, chunks]
    int32_t chunks, kl;
    int32_t nb, k;            // targets (0: not wanted)
    int32_t* pool;            // [rows, nb] ascending block ids, -1 padded
    int32_t* sel;             // [rows, k]
    uint32_t* zero_counters;  // [rows] or null: set to zero (by workgroup 2r)
};

struct BlockSelSmem {
    GroupSmem gs;
    uint32_t chunk_taken[kTopkSegment / 64];  // chosen candidates per chunk (kl >= 64)
};

// Top-t of one row's candidate lists (chunks lists of kl, a multiple of 64)
// into out[0..t) -- unless a full chunk had all kl of its candidates chosen:
// then nothing is written and the result is false.
template <int P>
__device__ __forceinline__ bool select_candidates(const uint32_t* __restrict__ ck,
                                                  const int32_t* __restrict__ ci,
                                                  const int32_t* __restrict__ cf, int32_t chunks,
                                                  int32_t kl, int32_t t, int32_t* __restrict__ out,
                                                  BlockSelSmem& bs, int tid, int lane, int wave)
{
    Smem& sm = bs.gs.sm;
    const int64_t n = (int64_t)chunks * kl;
    uint32_t key[P];
    int32_t id[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int64_t e = (int64_t)kThreads * i + tid;
        key[i] = e < n ? ck[e] : 0u;
        id[i] = e < n ? ci[e] : -1;
    }
    const int32_t full = tid < chunks ? cf[tid] : 0;  // chunks <= 256
    if (tid < chunks)
        bs.chunk_taken[tid] = 0u;  // ordered before the counts by find_threshold's barriers
    sel::clear_hist(sm, tid);
    const Pick pk = find_threshold(key, (uint32_t)t, sm, tid, lane, wave);
    bool take[P];
    uint32_t off[P];
    const uint32_t chosen = place(key, pk, take, off, sm, lane, wave);
    // chosen candidates per chunk: the 64 lanes of a wave's slot lie in one chunk
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint64_t bt = __ballot(take[i]);
        if (lane == 0 && bt != 0ull)
            atomicAdd(&bs.chunk_taken[(kThreads * i + 64 * wave) / kl], (uint32_t)__popcll(bt));
    }
    __syncthreads();
    const bool bad = tid < chunks && full != 0 && bs.chunk_taken[tid] >= (uint32_t)kl;
    if (__syncthreads_or(bad ? 1 : 0) != 0)
        return false;
    write_result(take, off, key, id, chosen, t, tid, out, nullptr, nullptr);
    return true;
}

// Direct form: the t best of the row's nvb block maxima into out[0..t).
template <int P>
__device__ __forceinline__ void select_direct(const float* __restrict__ srow, int64_t L,
                                              int64_t nvb, int32_t t, int32_t* __restrict__ out,
                                              Smem& sm, int tid, int lane, int wave)
{
    uint32_t key[P];
    int32_t id[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int64_t e = (int64_t)kThreads * i + tid;
        const float f = L > 0 ? srow[e < nvb ? e : 0] : 0.0f;  // no block maxima when L == 0
        key[i] = e < nvb && !__builtin_isnan(f) ? order_key(f) : 0u;
        id[i] = (int32_t)e;
    }
    sel::clear_hist(sm, tid);
    const Pick pk = find_threshold(key, (uint32_t)t, sm, tid, lane, wave);
    bool take[P];
    uint32_t off[P];
    const uint32_t chosen = place(key, pk, take, off, sm, lane, wave);
    write_result(take, off, key, id, chosen, t, tid, out, nullptr, nullptr);
}

// Grid: rows x passes -- with two passes workgroup 2r selects row r's top-k
// blocks (what the Full layer's own top-k waits for) and 2r + 1 its pool, side
// by side; with one pass (no pool) workgroup r selects the top-k blocks.
// kCand: the candidate form, with its out-of-line grouped fallback; the direct
// form is compiled without it (no scratch memory, 16 KB of LDS).
template <int P, bool kCand>
__global__ void __launch_bounds__(kThreads)
block_select_kernel(BlockSelJob J, int32_t passes)
{
    __shared__ std::conditional_t<kCand, BlockSelSmem, Smem> shm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x / passes;
    const int pass = blockIdx.x % passes;
    if (pass == 0 && J.zero_counters != nullptr && tid == 0)
        J.zero_counters[row] = 0u;
    const int32_t t = pass == 0 ? J.k : J.nb;
    int32_t* out = pass == 0 ? J.sel : J.pool;
    if (t <= 0 || out == nullptr)
        return;
    out += row * t;
    int64_t nvb = J.n_visible[row];
    nvb = nvb < 0 ? 0 : (nvb + kBlock - 1) / kBlock;
    nvb = nvb > J.L ? J.L : nvb;
    if constexpr (kCand) {
        const int64_t n = (int64_t)J.chunks * J.kl;
        if (select_candidates<P>(J.cand_key + row * n, J.cand_blk + row * n,
                                 J.cand_full + row * J.chunks, J.chunks, J.kl, t, out, shm, tid,
                                 lane, wave))
            return;
        // exact: the grouped select over the row's group maxima
        sel::clear_hist(shm.gs.sm, tid);
        if (J.g == 8)
            grouped_select_row_call<8>(J.block_max + row * J.L, nvb, J.g, J.ngroups,
                                       J.gkey + row * J.ngroups, t, out, shm.gs);
        else
            grouped_select_row_call<0>(J.block_max + row * J.L, nvb, J.g, J.ngroups,
                                       J.gkey + row * J.ngroups, t, out, shm.gs);
    } else {
        select_direct<P>(J.block_max + row * J.L, J.L, nvb, t, out, shm, tid, lane, wave);
    }
}

int64_t segments(int64_t L)
{
    return (L + kTopkSegment - 1) / kTopkSegment;
}

// Group size of the grouped path, or 0 when it does not apply.
int32_t group_size(int64_t L, int32_t k)
{
    if (L <= kTopkSegment)
        return 0;
    const int64_t g = (L + kTopkSegment - 1) / kTopkSegment;
    return (g * k <= kTopkSegment) ? (int32_t)g : 0;
}

}  // namespace

size_t topk_workspace(int64_t L, int32_t rows, int32_t k)
{
    if (L <= kTopkSegment)
        return 0;
    const int32_t g = group_size(L, k);
    if (g > 0)  // group maxima
        return (size_t)rows * (size_t)((L + g - 1) / g) * sizeof(uint32_t);
    // two ping-pong candidate buffers of the first (largest) level
    return 2ull * (size_t)rows * (size_t)segments(L) * (size_t)k * (sizeof(float) + sizeof(int32_t));
}

int32_t topk_group_size(int64_t L, int32_t k)
{
    return group_size(L, k);
}

bool block_select_fits(int64_t rows, int32_t passes)
{
    return grid_fits(rows * passes, kThreads);
}

// Every launch of launch_topk: one workgroup per row (the final select or the
// grouped one), the group maxima (counted in the larger of their two forms,
// the vectorised one at one thread per 4 keys) or the first (largest) level of
// segments.
bool topk_fits(int64_t L, int64_t rows, int32_t k)
{
    if (!grid_fits(rows, kThreads))
        return false;
    const int32_t g = group_size(L, k);
    if (g > 0) {
        const int64_t ngroups = (L + g - 1) / g;
        return grid_fits(rows * ((ngroups + 255) / 256), 256) &&
               grid_fits((rows * (L / 4) + 255) / 256, 256);
    }
    return L <= kTopkSegment || grid_fits(rows * segments(L), kThreads);
}

hipError_t launch_block_select(const BlockSelect& S, hipStream_t stream)
{
    if (S.rows == 0)
        return hipSuccess;
    const int32_t g = S.g;
    BlockSelJob J{S.block_max, S.L, S.n_visible, S.gkey, g > 0 ? (S.L + g - 1) / g : 0, g,
                  S.cand_key, S.cand_blk, S.cand_full, S.chunks, S.kl, S.nb, S.k, S.pool, S.sel,
                  S.zero_counters};
    const bool cand = S.cand_key != nullptr;
    const int64_t n = cand ? (int64_t)S.chunks * S.kl : S.L;
    const int32_t passes = S.nb > 0 && S.pool != nullptr ? 2 : 1;
    if (!block_select_fits(S.rows, passes))
        return hipErrorInvalidConfiguration;
    const dim3 grid((uint32_t)(passes * S.rows)), block(kThreads);
#define CSA2_BLOCK_SELECT(PP)                                                            \
    if (cand)                                                                            \
        block_select_kernel<PP, true><<<grid, block, 0, stream>>>(J, passes);           \
    else                                                                                 \
        block_select_kernel<PP, false><<<grid, block, 0, stream>>>(J, passes);
    if (n <= 4 * kThreads) {
        CSA2_BLOCK_SELECT(4)
    } else if (n <= 8 * kThreads) {
        CSA2_BLOCK_SELECT(8)
    } else {
        CSA2_BLOCK_SELECT(kPer)
    }
#undef CSA2_BLOCK_SELECT
    return hipGetLastError();
}

hipError_t launch_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                       const int32_t* n_valid, int32_t valid_div, int32_t k, int32_t* out,
                       void* ws, bool group_keys_ready, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    if (!topk_fits(L, rows, k))
        return hipErrorInvalidConfiguration;
    const int32_t g = group_size(L, k);
    if (g > 0) {
        const int64_t ngroups = (L + g - 1) / g;
        const int32_t per_row = (int32_t)((ngroups + 255) / 256);
        uint32_t* gkey = static_cast<uint32_t*>(ws);
        const dim3 grid((uint32_t)(rows * per_row));
        if (group_keys_ready) {
            // the scan already wrote the group maxima into the workspace
        } else if (g == 8 && idx == nullptr && L % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(score) % 16 == 0) {
            const int64_t quads = (int64_t)rows * (L / 4);
            group_max8_vec_kernel<<<dim3((uint32_t)((quads + 255) / 256)), dim3(256), 0, stream>>>(
                score, L, rows, ngroups, n_valid, valid_div, gkey);
        } else if (g == 8)
            group_max_kernel<8><<<grid, dim3(256), 0, stream>>>(score, idx, L, g, ngroups, per_row,
                                                                n_valid, valid_div, gkey);
        else
            group_max_kernel<0><<<grid, dim3(256), 0, stream>>>(score, idx, L, g, ngroups, per_row,
                                                                n_valid, valid_div, gkey);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        if (g == 8)
            topk_grouped_kernel<8><<<dim3((uint32_t)rows), dim3(kThreads), 0, stream>>>(
                score, idx, L, g, ngroups, gkey, n_valid, valid_div, k, out);
        else
            topk_grouped_kernel<0><<<dim3((uint32_t)rows), dim3(kThreads), 0, stream>>>(
                score, idx, L, g, ngroups, gkey, n_valid, valid_div, k, out);
        return hipGetLastError();
    }
    const size_t half = topk_workspace(L, rows, k) / 2;
    char* bufs[2] = {static_cast<char*>(ws), static_cast<char*>(ws) + half};
    int flip = 0;
    while (L > kTopkSegment) {
        const int64_t nseg = segments(L);
        const size_t n = (size_t)rows * nseg * k;
        float* cs = reinterpret_cast<float*>(bufs[flip]);
        int32_t* ci = reinterpret_cast<int32_t*>(bufs[flip] + n * sizeof(float));
        topk_kernel<kPer><<<dim3((uint32_t)(rows * nseg)), dim3(kThreads), 0, stream>>>(
            score, idx, L, kTopkSegment, (int32_t)nseg, n_valid, valid_div, k, nullptr, cs, ci);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        score = cs;
        idx = ci;
        L = nseg * k;
        n_valid = nullptr;
        flip ^= 1;
    }
    const dim3 grid((uint32_t)rows), block(kThreads);
    if (L <= 4 * kThreads)
        topk_kernel<4><<<grid, block, 0, stream>>>(score, idx, L, L, 1, n_valid, valid_div, k,
                                                   out, nullptr, nullptr);
    else if (L <= 8 * kThreads)
        topk_kernel<8><<<grid, block, 0, stream>>>(score, idx, L, L, 1, n_valid, valid_div, k,
                                                   out, nullptr, nullptr);
    else
        topk_kernel<kPer><<<grid, block, 0, stream>>>(score, idx, L, L, 1, n_valid, valid_div,
                                                      k, out, nullptr, nullptr);
    return hipGetLastError();
}

// ------------------------------------------------------------ static scratch
//
// The workspace of csa2_topk_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  In host code the
// array's name is only a host-side stand-in; the device address of each GPU's
// copy comes from hipGetSymbolAddress, looked up once per device (with that
// device current) and kept here.  Nothing in the top-k paths needs the
// workspace cleared: the group maxima and the candidate lists are written in
// full before they are read.

static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t topk_scratch(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace csa2
