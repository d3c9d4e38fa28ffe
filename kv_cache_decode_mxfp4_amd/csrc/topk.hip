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

#include "device_common.h"
#include "launch.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kTopkSegment / kThreads;  // 16
constexpr int kNumWaves = kThreads / kWave;    // 16
#ifndef CSA2_TOPK_BIN_BITS
#define CSA2_TOPK_BIN_BITS 11
#endif
constexpr int kBinBits = CSA2_TOPK_BIN_BITS;
constexpr int kBins = 1 << kBinBits;           // radix bins per pass
constexpr int kBpt = kBins / kThreads;         // bins per thread

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct Smem {
    uint32_t hist[2][kBins];
    uint32_t part_gt[kPer * kNumWaves];
    uint32_t part_eq[kPer * kNumWaves];
    uint32_t wave_a[3][kNumWaves];
    uint32_t bcast[2][3];
    uint32_t totals[2];
    uint32_t few_n;             // keys appended to few_key
    uint32_t few_key[kWave];    // the keys of a small chosen bin
    uint32_t few_pick[2];       // (threshold, keys equal to it to take)
};

struct Pick {
    uint32_t T;     // threshold key (0 = take every valid key)
    uint32_t need;  // keys equal to T to take, in position order
};

// Threshold of the k largest keys held by the workgroup (key 0 = invalid).
// Expects sm.hist[0] cleared by the caller before the first barrier here.
template <int P>
__device__ Pick find_threshold(const uint32_t (&key)[P], uint32_t k, Smem& sm, int tid,
                               int lane, int wave)
{
    uint32_t cnt = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (key[i] != 0u) {
            ++cnt;
            lo = min(lo, key[i]);
            hi = max(hi, key[i]);
        }
    cnt = wave_sum_u32(cnt, lane);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    if (lane == 0) {
        sm.wave_a[0][wave] = cnt;
        sm.wave_a[1][wave] = lo;
        sm.wave_a[2][wave] = hi;
    }
    if (tid == 0)
        sm.few_n = 0u;
    __syncthreads();
    uint32_t total = 0;
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int i = 0; i < kNumWaves; ++i) {
        total += sm.wave_a[0][i];
        lo = min(lo, sm.wave_a[1][i]);
        hi = max(hi, sm.wave_a[2][i]);
    }
    // no barrier here: wave_a is next written after the first pass's barrier (or
    // in the next call, after place()'s barriers), when every wave has read it
    Pick pk{0u, 0u};
    if (total <= k)
        return pk;
    uint32_t need = k, live = total;  // live: keys inside [lo, hi]
    // invariant: the threshold is the need-th largest key inside [lo, hi]
    for (int pass = 0; pass < 4 && hi != lo; ++pass) {
        const int buf = pass & 1;
        const uint32_t span = hi - lo;
        const int bits = 32 - __builtin_clz(span);
        const int shift = bits > kBinBits ? bits - kBinBits : 0;
        // key - lo wraps above span for keys below lo (the invalid key 0 too)
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t d = key[i] - lo;
            if (d <= span)
                atomicAdd(&sm.hist[buf][d >> shift], 1u);
        }
        __syncthreads();
        // thread t owns bins kBpt*t .. kBpt*t + kBpt - 1
        uint32_t c[kBpt], mine = 0;
#pragma unroll
        for (int j = 0; j < kBpt; ++j) {
            c[j] = sm.hist[buf][kBpt * tid + j];
            mine += c[j];
            sm.hist[buf ^ 1][kBpt * tid + j] = 0u;  // clear the buffer of the next pass
        }
        const uint32_t incl = wave_prefix_sum(mine, lane);
        if (lane == kWave - 1)
            sm.wave_a[0][wave] = incl;
        __syncthreads();
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int i = 0; i < kNumWaves; ++i) {
            const uint32_t v = sm.wave_a[0][i];
            before += i < wave ? v : 0u;
            all += v;
        }
        uint32_t above = all - (before + incl);  // keys in bins above this thread's
#pragma unroll
        for (int j = kBpt - 1; j >= 0; --j) {
            if (above < need && above + c[j] >= need) {
                sm.bcast[buf][0] = (uint32_t)(kBpt * tid + j);
                sm.bcast[buf][1] = above;
                sm.bcast[buf][2] = c[j];
            }
            above += c[j];
        }
        __syncthreads();
        const uint32_t bin = sm.bcast[buf][0];
        const uint32_t in_bin = sm.bcast[buf][2];
        need -= sm.bcast[buf][1];
        live = in_bin;
        lo = lo + (bin << shift);
        const uint64_t top = (uint64_t)lo + ((1ull << shift) - 1ull);
        hi = top < (uint64_t)hi ? (uint32_t)top : hi;
        if (in_bin <= (uint32_t)kWave && hi != lo) {
            // Few keys left in [lo, hi]: gather them and rank them in one wave
            // instead of another histogram pass.
            const uint32_t width = hi - lo;
#pragma unroll
            for (int i = 0; i < P; ++i)
                if (key[i] - lo <= width) {
                    const uint32_t p = atomicAdd(&sm.few_n, 1u);
                    if (p < (uint32_t)kWave)
                        sm.few_key[p] = key[i];
                }
            __syncthreads();
            if (wave == 0) {
                const uint32_t v = lane < (int)in_bin ? sm.few_key[lane] : 0u;
                uint32_t gt = 0, eq = 0;
                for (uint32_t j = 0; j < in_bin; ++j) {
                    const uint32_t u = (uint32_t)__builtin_amdgcn_readlane((int)v, (int)j);
                    gt += u > v ? 1u : 0u;
                    eq += u == v ? 1u : 0u;
                }
                // the need-th largest of the gathered keys: gt < need <= gt + eq
                if (lane < (int)in_bin && gt < need && need <= gt + eq) {
                    // when every key equal to v is taken, "above v - 1" says the same
                    const bool all = need == gt + eq;
                    sm.few_pick[0] = all ? v - 1u : v;
                    sm.few_pick[1] = all ? 0u : need - gt;
                }
            }
            __syncthreads();
            pk.T = sm.few_pick[0];
            pk.need = sm.few_pick[1];
            return pk;
        }
    }
    // every key left equals lo
    pk.T = need == live ? lo - 1u : lo;
    pk.need = need == live ? 0u : need;
    return pk;
}

// Exclusive scan, in position order, of the 16 * P (slot, wave) counts
// part[] in place by one wave (P / 4 per lane); returns the total on every lane.
template <int P>
__device__ __forceinline__ uint32_t scan_parts(uint32_t* part, int lane)
{
    constexpr int kN = P * kNumWaves / kWave;
    static_assert(kN >= 1 && kN * kWave == P * kNumWaves, "slots per thread: a multiple of 4");
    uint32_t c[kN], sum = 0;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        c[j] = part[kN * lane + j];
        sum += c[j];
    }
    const uint32_t incl = wave_prefix_sum(sum, lane);
    uint32_t run = incl - sum;
#pragma unroll
    for (int j = 0; j < kN; ++j) {
        part[kN * lane + j] = run;
        run += c[j];
    }
    return (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
}

// Marks the chosen slots and their output offsets (position order); returns
// how many were chosen.  pk.need == 0 (every key equal to the threshold is
// taken, or there is none) needs only the "above" ballots.
template <int P>
__device__ uint32_t place(const uint32_t (&key)[P], Pick pk, bool (&take)[P],
                          uint32_t (&off)[P], Smem& sm, int lane, int wave)
{
    if (pk.need == 0u) {
        uint32_t gt_below[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint64_t bg = __ballot(key[i] > pk.T);
            gt_below[i] = lanes_below(bg, lane);
            if (lane == 0)
                sm.part_gt[i * kNumWaves + wave] = (uint32_t)__popcll(bg);
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t all = scan_parts<P>(sm.part_gt, lane);
            if (lane == 0)
                sm.totals[0] = all;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            take[i] = key[i] > pk.T;
            off[i] = sm.part_gt[i * kNumWaves + wave] + gt_below[i];
        }
        const uint32_t n_gt = sm.totals[0];
        __syncthreads();
        return n_gt;
    }
    uint32_t gt_below[P], eq_below[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint64_t bg = __ballot(key[i] > pk.T);
        const uint64_t be = __ballot(key[i] == pk.T);
        gt_below[i] = lanes_below(bg, lane);
        eq_below[i] = lanes_below(be, lane);
        if (lane == 0) {
            sm.part_gt[i * kNumWaves + wave] = (uint32_t)__popcll(bg);
            sm.part_eq[i * kNumWaves + wave] = (uint32_t)__popcll(be);
        }
    }
    __syncthreads();
    if (wave < 2) {
        const uint32_t all = scan_parts<P>(wave == 0 ? sm.part_gt : sm.part_eq, lane);
        if (lane == 0)
            sm.totals[wave] = all;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t gt_before = sm.part_gt[i * kNumWaves + wave] + gt_below[i];
        const uint32_t eq_before = sm.part_eq[i * kNumWaves + wave] + eq_below[i];
        take[i] = key[i] > pk.T || (key[i] == pk.T && eq_before < pk.need);
        off[i] = gt_before + (eq_before < pk.need ? eq_before : pk.need);
    }
    const uint32_t n_gt = sm.totals[0], n_eq = sm.totals[1];
    __syncthreads();
    return n_gt + (n_eq < pk.need ? n_eq : pk.need);
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
    for (int b = tid; b < kBins; b += kThreads)
        sm.hist[0][b] = 0u;

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

// Grouped select for one row from its group maxima gkey[row, 0..ngroups)
// (ngroups <= 16384, g * k <= 16384).  Grid: rows.  kG: the group size when
// known at compile time (8: L up to 131072 with k <= 2048), else 0.
template <int kG>
__global__ void __launch_bounds__(kThreads)
topk_grouped_kernel(const float* __restrict__ score, const int32_t* __restrict__ idx, int64_t L,
                    int32_t g_runtime, int64_t ngroups, const uint32_t* __restrict__ gkey,
                    const int32_t* __restrict__ n_valid, int32_t valid_div, int32_t k,
                    int32_t* __restrict__ out)
{
    __shared__ GroupSmem gs;
    Smem& sm = gs.sm;
    const uint32_t g = kG > 0 ? (uint32_t)kG : (uint32_t)g_runtime;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t nv = valid_prefix(n_valid, row, L, valid_div);
    const float* srow = score + row * L;
    const int32_t* irow = idx != nullptr ? idx + row * L : nullptr;
    for (int b = tid; b < kBins; b += kThreads)
        sm.hist[0][b] = 0u;

    uint32_t key[kPer];
    int32_t id[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t grp = (int64_t)kThreads * i + tid;
        key[i] = grp < ngroups ? gkey[row * ngroups + grp] : 0u;
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
    for (int b = tid; b < kBins; b += kThreads)
        sm.hist[0][b] = 0u;
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
    write_result(take, off, key, id, chosen, k, tid, out + row * k, nullptr, nullptr);
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

hipError_t launch_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                       const int32_t* n_valid, int32_t valid_div, int32_t k, int32_t* out,
                       void* ws, bool group_keys_ready, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
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
