// Sparse MLA attention over the selected MXFP4 main-KV entries plus the FP8
// sliding window ([N] 1 of the DeepSeek-V4.1 reading notes: 64 query heads x
// 512; [S] "DeepSeek-V4 model structure (7)": K = V single-head MQA on the
// 512-dim latent, top-k compressed entries plus 128 window entries).  One
// joint softmax over both key sets; no de-duplication; no sink.
//
// Workgroup = 4 waves = (query row, group of 32 heads, split of the key list).
// The key list is the k top-k slots followed by the window rows, cut into
// tiles of 32 keys.  Per tile:
//   1. every lane gathers its key's 128-channel slice (wave w owns channels
//      [128w, 128w+128)), dequantises it in registers (exact in fp16) and
//      stores it transposed to LDS (it is also V: K = V);
//   2. S^T = K Q^T over the wave's channels (v_mfma_f32_32x32x16_f16,
//      keys x heads); the four waves' partial sums meet in LDS and are added
//      in a fixed order;
//   3. online softmax per head in fp32 (exp2 domain); P is split into two
//      fp16 terms (hi + lo) so P V keeps ~22 bits of P;
//   4. O += P V with O = 32 heads x the wave's 128 dims in fp32 registers.
// The S^T accumulator layout already is the A-operand layout of P for the
// P V product once the 32 keys of a tile are taken in the order
//   k-step u, lane half g, slot i  ->  key 16u + 8(i/4) + 4g + i%4,
// which the B operand (V^T rows in LDS) follows.
// With more than one split, partial (O, m, l) go to the workspace and a
// combine kernel merges them in split order (deterministic).
#include "device_common.h"

namespace csa2 {
namespace {

constexpr int kAttnWaves = 4;
constexpr int kTile = 32;
constexpr int kVtStride = 36;  // halves per V^T row: 32 keys + pad (bank spread, 8-byte aligned)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnSmem {
    _Float16 vt[kDim * kVtStride];
    float sx[kAttnWaves][16][kWave];
};

__global__ void __launch_bounds__(kAttnWaves * kWave)
sparse_attn_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_codes,
                   const uint8_t* __restrict__ kv_scales, int64_t n_cap, int32_t nq,
                   const int32_t* __restrict__ topk, int32_t k, const uint8_t* __restrict__ swa,
                   int32_t swa_cap, const int32_t* __restrict__ swa_end, int32_t n_win,
                   float scale_log2, int32_t splits, float* __restrict__ out,
                   float* __restrict__ lse, float* __restrict__ ws_o, float* __restrict__ ws_m,
                   float* __restrict__ ws_l)
{
    __shared__ AttnSmem sm;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 5;
    const int col = lane & 31;
    const int64_t qrow = blockIdx.x / (2 * splits);
    const int hg = (blockIdx.x / splits) % 2;
    const int sp = blockIdx.x % splits;
    const int64_t b = qrow / nq;

    int64_t end = swa_end[qrow];
    int64_t lo = end - n_win;
    lo = lo < 0 ? 0 : lo;
    int64_t hi = end < swa_cap ? end : (int64_t)swa_cap;
    hi = hi < lo ? lo : hi;
    const int64_t n_sw = hi - lo;
    const int64_t t_main = (k + kTile - 1) / kTile;
    const int64_t t_all = t_main + (n_sw + kTile - 1) / kTile;
    const int64_t t0 = sp * t_all / splits;
    const int64_t t1 = (sp + 1) * t_all / splits;

    // B operand of S^T = K Q^T: head 32*hg + col, dims 128*wave + 64*g + 8t + i
    half8 qb[8];
    {
        const uint4* src = reinterpret_cast<const uint4*>(
            q + (qrow * kHeads + 32 * hg + col) * kDim + 128 * wave + 64 * g);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const uint4 v = src[t];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qb[t][2 * i] = bf16_to_f16((uint16_t)(d[i] & 0xFFFFu));
                qb[t][2 * i + 1] = bf16_to_f16((uint16_t)(d[i] >> 16));
            }
        }
    }

    const uint8_t* kc = kv_codes + b * n_cap * (kDim / 2);
    const uint8_t* ks = kv_scales + b * n_cap * (kDim / 16);
    const uint8_t* sw = swa + b * (int64_t)swa_cap * kDim;
    const int32_t* tk = topk + qrow * k;

    float m_run = -INFINITY;  // per head col (log2 domain)
    float l_run = 0.0f;
    f32x16 o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        o[c] = f32x16{};

    for (int64_t tile = t0; tile < t1; ++tile) {
        // ---- gather + dequantise this lane's key slice
        half8 kv[8];
        bool valid = false;
        const int64_t slot = tile * kTile + col;
        if (tile < t_main) {
            int64_t e = slot < k ? (int64_t)tk[slot] : -1;
            valid = e >= 0 && e < n_cap;
            if (valid) {
                const uint4* c = reinterpret_cast<const uint4*>(kc + e * (kDim / 2) + 64 * wave + 32 * g);
                const uint4 c0 = c[0], c1 = c[1];
                const uint32_t sc =
                    *reinterpret_cast<const uint32_t*>(ks + e * (kDim / 16) + 8 * wave + 4 * g);
                const uint32_t words[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    kv[t] = dequant8_fp4(words[t], e4m3_byte_to_f16(sc, t / 2));
            }
        } else {
            const int64_t r = lo + (slot - t_main * kTile);
            valid = r < hi;
            if (valid) {
                const uint4* c = reinterpret_cast<const uint4*>(sw + r * kDim + 128 * wave + 64 * g);
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    const uint4 v = c[t4];
                    const half4v a0 = e4m3x4_to_f16(v.x), a1 = e4m3x4_to_f16(v.y);
                    const half4v a2 = e4m3x4_to_f16(v.z), a3 = e4m3x4_to_f16(v.w);
                    kv[2 * t4] = half8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    kv[2 * t4 + 1] = half8{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
                }
            }
        }
        if (!valid) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                kv[t] = half8{};
        }
        const uint64_t vmask = __ballot(valid);

        // ---- S^T partial over this wave's channels; V^T to LDS
        f32x16 acc = {};
#pragma unroll
        for (int t = 0; t < 8; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kv[t], qb[t], acc, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d0 = 128 * wave + 64 * g + 8 * t;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sm.vt[(d0 + i) * kVtStride + col] = kv[t][i];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sm.sx[wave][r][lane] = acc[r];
        __syncthreads();

        // ---- full S^T (fixed order over waves), online softmax per head col
        float s[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float v = ((sm.sx[0][r][lane] + sm.sx[1][r][lane]) + sm.sx[2][r][lane]) +
                            sm.sx[3][r][lane];
            const int kr = 8 * (r / 4) + 4 * g + (r % 4);
            s[r] = ((vmask >> kr) & 1ull) ? v * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.0f;
        float psum = 0.0f;
        float p[16];
        if (m_new == -INFINITY) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                p[r] = 0.0f;
        } else {
            alpha = exp2f(m_run - m_new);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = exp2f(s[r] - m_new);
                psum += p[r];
            }
        }
        psum = psum + __shfl_xor(psum, 32, kWave);
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // ---- rescale O rows (heads) and accumulate P V
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float ar = __shfl(alpha, 8 * (r / 4) + 4 * g + (r % 4), kWave);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c][r] *= ar;
        }
        half8 phi[2], plo[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float pv = p[8 * u + i];
                const _Float16 h = (_Float16)pv;
                phi[u][i] = h;
                plo[u][i] = (_Float16)(pv - (float)h);
            }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int dim = 128 * wave + 32 * c + col;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const _Float16* rowp = sm.vt + dim * kVtStride + 16 * u + 4 * g;
                const half4v v0 = *reinterpret_cast<const half4v*>(rowp);
                const half4v v1 = *reinterpret_cast<const half4v*>(rowp + 8);
                const half8 vb = half8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                o[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(phi[u], vb, o[c], 0, 0, 0);
                o[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(plo[u], vb, o[c], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: rows of O are heads 8(r/4) + 4g + r%4 of the group
    const int64_t head0 = qrow * kHeads + 32 * hg;
    if (splits == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int hr = 8 * (r / 4) + 4 * g + (r % 4);
            const float lr = __shfl(l_run, hr, kWave);
            const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                out[(head0 + hr) * kDim + 128 * wave + 32 * c + col] = o[c][r] * inv;
        }
        if (lse != nullptr && wave == 0 && lane < 32)
            lse[head0 + col] = l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    } else {
        const int64_t part = (qrow * 2 + hg) * splits + sp;  // [Q, 2, splits] x 32 heads
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int hr = 8 * (r / 4) + 4 * g + (r % 4);
#pragma unroll
            for (int c = 0; c < 4; ++c)
                ws_o[(part * 32 + hr) * kDim + 128 * wave + 32 * c + col] = o[c][r];
        }
        if (wave == 0 && lane < 32) {
            ws_m[part * 32 + col] = m_run;
            ws_l[part * 32 + col] = l_run;
        }
    }
}

// Merge the per-split partials of one (query row, head): thread per output dim.
__global__ void __launch_bounds__(256)
attn_combine_kernel(int64_t total, int32_t splits, const float* __restrict__ ws_o,
                    const float* __restrict__ ws_m, const float* __restrict__ ws_l,
                    float* __restrict__ out, float* __restrict__ lse)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total)
        return;
    const int64_t head = t / kDim;           // qrow * 64 + h
    const int dim = (int)(t % kDim);
    const int64_t qrow = head / kHeads;
    const int h = (int)(head % kHeads);
    const int hg = h / 32, hl = h % 32;
    const int64_t base = (qrow * 2 + hg) * splits;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s)
        M = fmaxf(M, ws_m[(base + s) * 32 + hl]);
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < splits; ++s) {
            const float ms = ws_m[(base + s) * 32 + hl];
            const float f = ms == -INFINITY ? 0.0f : exp2f(ms - M);
            num += f * ws_o[((base + s) * 32 + hl) * kDim + dim];
            den += f * ws_l[(base + s) * 32 + hl];
        }
    }
    out[t] = den > 0.0f ? num / den : 0.0f;
    if (lse != nullptr && dim == 0)
        lse[head] = den > 0.0f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

}  // namespace

int32_t attn_splits(int32_t queries, int32_t k, int32_t n_win)
{
    const int64_t tiles = (int64_t)(k + kTile - 1) / kTile + (n_win + kTile - 1) / kTile;
    const int64_t wgs = 2ll * queries;
    int64_t s = (512 + wgs - 1) / wgs;  // aim for >= 512 workgroups
    const int64_t cap = (tiles + 1) / 2;  // at least two tiles per split
    s = s > cap ? cap : s;
    return (int32_t)(s < 1 ? 1 : s);
}

size_t attn_workspace(int32_t queries, int32_t k, int32_t n_win)
{
    const int32_t s = attn_splits(queries, k, n_win);
    if (s <= 1)
        return 0;
    return (size_t)queries * 2 * s * 32 * (kDim + 2) * sizeof(float);
}

hipError_t launch_sparse_attn(const uint16_t* q, int32_t queries, int32_t nq,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                              const int32_t* topk, int32_t k, const uint8_t* swa,
                              int32_t swa_cap, const int32_t* swa_end, int32_t n_win,
                              float softmax_scale, float* out, float* lse, void* ws,
                              int32_t splits, hipStream_t stream)
{
    if (queries == 0)
        return hipSuccess;
    float* ws_o = nullptr;
    float* ws_m = nullptr;
    float* ws_l = nullptr;
    if (splits > 1) {
        const size_t parts = (size_t)queries * 2 * splits * 32;
        ws_o = static_cast<float*>(ws);
        ws_m = ws_o + parts * kDim;
        ws_l = ws_m + parts;
    }
    const int64_t grid = (int64_t)queries * 2 * splits;
    sparse_attn_kernel<<<dim3((uint32_t)grid), dim3(kAttnWaves * kWave), 0, stream>>>(
        q, kv_codes, kv_scales, n_cap, nq, topk, k, swa, swa_cap, swa_end, n_win,
        softmax_scale * kLog2e, splits, out, lse, ws_o, ws_m, ws_l);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    const int64_t total = (int64_t)queries * kHeads * kDim;
    attn_combine_kernel<<<dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream>>>(
        total, splits, ws_o, ws_m, ws_l, out, lse);
    return hipGetLastError();
}

}  // namespace csa2
