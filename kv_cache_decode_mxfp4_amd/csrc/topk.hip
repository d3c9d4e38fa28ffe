// Deterministic top-k select ([N] 1 of the DeepSeek-V4.1 reading notes: top-k
// 512; [N] 2.2 / [A] 3.4: top-2048 blocks form the pool).
//
// Order: score descending, then position ascending (the lower index wins a
// tie); -0 equals +0; NaN and masked entries never win.  Output: the chosen
// indices in ascending order, -1 padded.
//
// One workgroup of 1024 threads holds a segment of up to 16384 scores in
// registers (16 per thread, thread t owning positions [16t, 16t+16)) and finds
// the k-th largest key with an adaptive-range radix select: every pass
// histograms the live key range [kmin, kmax] into 256 equal bins in LDS and
// keeps the bin that holds the k-th key, so each pass shrinks the range by at
// least 2^8 and at most four passes are needed.  A workgroup-wide prefix sum
// then writes the chosen entries in position order.
//
// Rows longer than one segment are reduced exactly in levels: every segment
// emits its own top-k candidates (the global top-k is a subset of their
// union, and the candidate lists keep position order), until one segment
// remains.
#include "device_common.h"

namespace csa2 {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = kTopkSegment / kThreads;  // 16
constexpr int kNumWaves = kThreads / kWave;    // 16

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u)
        u = 0u;  // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct Smem {
    uint32_t hist[256];
    uint32_t wave_a[kNumWaves];
    uint32_t wave_b[kNumWaves];
    uint32_t bcast[4];
};

// Workgroup sum of one value per thread.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, Smem& sm, int lane, int wave)
{
    v = wave_sum(v);
    if (lane == 0)
        sm.wave_a[wave] = v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kNumWaves; ++i)
        t += sm.wave_a[i];
    __syncthreads();
    return t;
}

// Workgroup min and max of one key per thread (inactive threads pass
// min = 0xFFFFFFFF, max = 0).
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, Smem& sm, int lane,
                                             int wave)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
    }
    if (lane == 0) {
        sm.wave_a[wave] = mn;
        sm.wave_b[wave] = mx;
    }
    __syncthreads();
    mn = 0xFFFFFFFFu;
    mx = 0u;
#pragma unroll
    for (int i = 0; i < kNumWaves; ++i) {
        mn = min(mn, sm.wave_a[i]);
        mx = max(mx, sm.wave_b[i]);
    }
    __syncthreads();
}

// Exclusive prefix sum over the workgroup in thread order.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, Smem& sm, int lane, int wave)
{
    const uint32_t inc = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1)
        sm.wave_a[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < wave; ++i)
        before += sm.wave_a[i];
    __syncthreads();
    return before + inc - v;
}

// Selects within rows of up to kTopkSegment entries.  Grid: rows * nseg
// workgroups; workgroup (row, seg) covers positions [seg*seg_len, +seg_len).
// Final mode (cand_score == nullptr): out[row, 0..k) = ascending indices.
// Candidate mode: cand_score/cand_idx[row, seg, 0..k) = chosen (score, index)
// pairs in position order, padded with index -1.
__global__ void __launch_bounds__(kThreads)
topk_kernel(const float* __restrict__ score, const int32_t* __restrict__ idx, int64_t L,
            int64_t seg_len, int32_t nseg, const int32_t* __restrict__ n_valid, int32_t k,
            int32_t* __restrict__ out, float* __restrict__ cand_score,
            int32_t* __restrict__ cand_idx)
{
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t row = blockIdx.x / nseg;
    const int64_t seg = blockIdx.x % nseg;
    int64_t nv = L;
    if (n_valid != nullptr) {
        nv = n_valid[row];
        nv = nv < 0 ? 0 : (nv > L ? L : nv);
    }
    const int64_t seg_start = seg * seg_len;
    int64_t seg_end = seg_start + seg_len;
    seg_end = seg_end < nv ? seg_end : nv;

    uint32_t key[kPer];
    int32_t id[kPer];
    uint32_t n_mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t pos = seg_start + (int64_t)kPer * tid + i;
        uint32_t kk = 0u;
        int32_t ii = -1;
        if (pos < seg_end) {
            const float f = score[row * L + pos];
            ii = idx != nullptr ? idx[row * L + pos] : (int32_t)pos;
            if (ii >= 0 && !__builtin_isnan(f))
                kk = order_key(f);
        }
        key[i] = kk;
        id[i] = ii;
        n_mine += kk != 0u;
    }
    const uint32_t n_total = block_sum(n_mine, sm, lane, wave);

    // threshold key T and the number of keys equal to T to take
    uint32_t T = 0u;
    uint32_t need = 0u;
    if (n_total > (uint32_t)k) {
        uint32_t lo = 1u, hi = 0xFFFFFFFFu;
        need = (uint32_t)k;
        // each pass drops at least 8 bits of the live range: 4 passes narrow a
        // 32-bit range to one key, the 5th sees kmin == kmax; 6 bounds the loop
        for (int pass = 0; pass < 6; ++pass) {
            uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                if (key[i] >= lo && key[i] <= hi) {
                    mn = min(mn, key[i]);
                    mx = max(mx, key[i]);
                }
            block_minmax(mn, mx, sm, lane, wave);
            T = mn;
            if (mn == mx)
                break;
            const uint32_t span = mx - mn;
            const int bits = 32 - __builtin_clz(span);
            const int shift = bits > 8 ? bits - 8 : 0;
            if (tid < 256)
                sm.hist[tid] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kPer; ++i)
                if (key[i] >= mn && key[i] <= mx)
                    atomicAdd(&sm.hist[(key[i] - mn) >> shift], 1u);
            __syncthreads();
            if (wave == 0) {
                // lane owns bins 4*lane .. 4*lane+3; count of keys in bins above
                uint32_t c[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    c[j] = sm.hist[4 * lane + j];
                const uint32_t mine = c[0] + c[1] + c[2] + c[3];
                // suffix sum over lanes: keys in bins of lanes > lane
                uint32_t incl = mine;
#pragma unroll
                for (int o = 1; o < kWave; o <<= 1) {
                    const uint32_t t = __shfl_down(incl, o, kWave);
                    if (lane + o < kWave)
                        incl += t;
                }
                uint32_t above = incl - mine;  // bins of higher lanes
#pragma unroll
                for (int j = 3; j >= 0; --j) {
                    if (above < need && above + c[j] >= need) {
                        sm.bcast[0] = (uint32_t)(4 * lane + j);
                        sm.bcast[1] = above;
                    }
                    above += c[j];
                }
            }
            __syncthreads();
            const uint32_t bin = sm.bcast[0];
            const uint32_t above = sm.bcast[1];
            __syncthreads();
            need -= above;
            lo = mn + (bin << shift);
            const uint64_t top = (uint64_t)lo + ((1ull << shift) - 1ull);
            hi = top < (uint64_t)mx ? (uint32_t)top : mx;
        }
    }

    // counts per thread, then positions in the output
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        gt += key[i] > T;
        eq += (T != 0u) && key[i] == T;
    }
    const uint32_t eq_before = block_exclusive_scan(eq, sm, lane, wave);
    uint32_t take_eq = need > eq_before ? need - eq_before : 0u;
    take_eq = take_eq < eq ? take_eq : eq;
    const uint32_t mine = gt + take_eq;
    uint32_t o = block_exclusive_scan(mine, sm, lane, wave);
    const uint32_t selected = n_total < (uint32_t)k ? n_total : (uint32_t)k;
    uint32_t eq_seen = 0;
    if (cand_score == nullptr) {
        int32_t* dst = out + row * k;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            bool take = key[i] > T;
            if (T != 0u && key[i] == T) {
                take = eq_seen < take_eq;
                ++eq_seen;
            }
            if (take && o < (uint32_t)k)
                dst[o++] = id[i];
        }
        for (uint32_t p = selected + tid; p < (uint32_t)k; p += kThreads)
            dst[p] = -1;
    } else {
        float* ds = cand_score + (row * nseg + seg) * k;
        int32_t* di = cand_idx + (row * nseg + seg) * k;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            bool take = key[i] > T;
            if (T != 0u && key[i] == T) {
                take = eq_seen < take_eq;
                ++eq_seen;
            }
            if (take && o < (uint32_t)k) {
                ds[o] = key_value(key[i]);
                di[o] = id[i];
                ++o;
            }
        }
        for (uint32_t p = selected + tid; p < (uint32_t)k; p += kThreads) {
            ds[p] = 0.0f;
            di[p] = -1;
        }
    }
}

int64_t segments(int64_t L)
{
    return (L + kTopkSegment - 1) / kTopkSegment;
}

}  // namespace

size_t topk_workspace(int64_t L, int32_t rows, int32_t k)
{
    if (L <= kTopkSegment)
        return 0;
    // two ping-pong candidate buffers of the first (largest) level
    return 2ull * (size_t)rows * (size_t)segments(L) * (size_t)k * (sizeof(float) + sizeof(int32_t));
}

hipError_t launch_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                       const int32_t* n_valid, int32_t k, int32_t* out, void* ws,
                       hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    const size_t half = topk_workspace(L, rows, k) / 2;
    char* bufs[2] = {static_cast<char*>(ws), static_cast<char*>(ws) + half};
    int flip = 0;
    while (L > kTopkSegment) {
        const int64_t nseg = segments(L);
        const size_t n = (size_t)rows * nseg * k;
        float* cs = reinterpret_cast<float*>(bufs[flip]);
        int32_t* ci = reinterpret_cast<int32_t*>(bufs[flip] + n * sizeof(float));
        topk_kernel<<<dim3((uint32_t)(rows * nseg)), dim3(kThreads), 0, stream>>>(
            score, idx, L, kTopkSegment, (int32_t)nseg, n_valid, k, nullptr, cs, ci);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        score = cs;
        idx = ci;
        L = nseg * k;
        n_valid = nullptr;
        flip ^= 1;
    }
    topk_kernel<<<dim3((uint32_t)rows), dim3(kThreads), 0, stream>>>(
        score, idx, L, L, 1, n_valid, k, out, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace csa2
