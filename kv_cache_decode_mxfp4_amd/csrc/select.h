// Workgroup-wide exact selection primitives shared by the top-k kernels and
// the indexer scan's per-chunk candidate select ([N] 1 of the DeepSeek-V4.1
// reading notes: top-k 512; [N] 2.2 / [A] 3.4: the top-2048 blocks form the
// pool).
//
// Keys are unsigned order keys (order_key: larger score <=> larger key, key 0
// = no entry) held in registers, P per thread: slot i of thread t is element
// kT*i + t of the workgroup's list, so position order is slot-major.  The
// selection order is key descending, then position ascending.
//
// find_threshold: the k-th largest key by an adaptive-range radix select --
// each pass histograms the live key range [lo, hi] into at most 2048 equal
// LDS bins and keeps the bin holding the k-th key (the span shrinks by at
// least 2^11 per pass); once the chosen bin holds at most 64 keys they are
// gathered into LDS and one wave ranks them against each other instead of
// running another pass.
// place: one ballot round gives every chosen slot its output offset in
// position order: offset = (#greater before it) + min(#equal before it,
// #equal to take).
#pragma once

#include "device_common.h"

namespace csa2 {
namespace sel {

constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;  // radix bins per pass
constexpr int kMaxP = 16;             // slots per thread, at most

template <int kT>
struct Smem {
    static constexpr int kWaves = kT / kWave;
    uint32_t hist[2][kBins];
    uint32_t part_gt[kMaxP * kWaves];
    uint32_t part_eq[kMaxP * kWaves];
    uint32_t wave_a[3][kWaves];
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

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Clears the first histogram buffer (before each find_threshold, once every
// thread is done with the previous one's histograms).
template <int kT>
__device__ __forceinline__ void clear_hist(Smem<kT>& sm, int tid)
{
    for (int b = tid; b < kBins; b += kT)
        sm.hist[0][b] = 0u;
}

// Threshold of the k largest keys held by the workgroup (key 0 = invalid).
// Expects sm.hist[0] cleared before the first barrier here (clear_hist); the
// histograms are left dirty, so a later call needs clear_hist again.
template <int P, int kT>
__device__ Pick find_threshold(const uint32_t (&key)[P], uint32_t k, Smem<kT>& sm, int tid,
                               int lane, int wave)
{
    constexpr int kWaves = kT / kWave;
    constexpr int kBpt = kBins / kT;  // bins per thread
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
    for (int i = 0; i < kWaves; ++i) {
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
        for (int i = 0; i < kWaves; ++i) {
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

// Exclusive scan, in position order, of the P * kWaves (slot, wave) counts
// part[] in place by one wave; returns the total on every lane.
template <int P, int kWaves>
__device__ __forceinline__ uint32_t scan_parts(uint32_t* part, int lane)
{
    constexpr int kTot = P * kWaves;
    if constexpr (kTot >= kWave) {
        constexpr int kN = kTot / kWave;
        static_assert(kN * kWave == kTot, "slot and wave counts: a multiple of 64");
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
    } else {
        const uint32_t c = lane < kTot ? part[lane] : 0u;
        const uint32_t incl = wave_prefix_sum(c, lane);
        if (lane < kTot)
            part[lane] = incl - c;
        return (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
    }
}

// Marks the chosen slots and their output offsets (position order); returns
// how many were chosen.  pk.need == 0 (every key equal to the threshold is
// taken, or there is none) needs only the "above" ballots.
template <int P, int kT>
__device__ uint32_t place(const uint32_t (&key)[P], Pick pk, bool (&take)[P],
                          uint32_t (&off)[P], Smem<kT>& sm, int lane, int wave)
{
    constexpr int kWaves = kT / kWave;
    if (pk.need == 0u) {
        uint32_t gt_below[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint64_t bg = __ballot(key[i] > pk.T);
            gt_below[i] = lanes_below(bg, lane);
            if (lane == 0)
                sm.part_gt[i * kWaves + wave] = (uint32_t)__popcll(bg);
        }
        __syncthreads();
        if (wave == 0) {
            const uint32_t all = scan_parts<P, kWaves>(sm.part_gt, lane);
            if (lane == 0)
                sm.totals[0] = all;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            take[i] = key[i] > pk.T;
            off[i] = sm.part_gt[i * kWaves + wave] + gt_below[i];
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
            sm.part_gt[i * kWaves + wave] = (uint32_t)__popcll(bg);
            sm.part_eq[i * kWaves + wave] = (uint32_t)__popcll(be);
        }
    }
    __syncthreads();
    if (wave < 2) {
        const uint32_t all = scan_parts<P, kWaves>(wave == 0 ? sm.part_gt : sm.part_eq, lane);
        if (lane == 0)
            sm.totals[wave] = all;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t gt_before = sm.part_gt[i * kWaves + wave] + gt_below[i];
        const uint32_t eq_before = sm.part_eq[i * kWaves + wave] + eq_below[i];
        take[i] = key[i] > pk.T || (key[i] == pk.T && eq_before < pk.need);
        off[i] = gt_before + (eq_before < pk.need ? eq_before : pk.need);
    }
    const uint32_t n_gt = sm.totals[0], n_eq = sm.totals[1];
    __syncthreads();
    return n_gt + (n_eq < pk.need ? n_eq : pk.need);
}

}  // namespace sel
}  // namespace csa2
