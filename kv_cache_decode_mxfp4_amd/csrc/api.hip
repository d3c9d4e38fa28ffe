// C ABI of libcsa2 (declared in include/csa2.h): host-side validation, then
// one launcher per call.  Nothing is enqueued when validation fails.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/csa2.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool debug_sync()
{
    static const bool on = [] {
        const char* v = getenv("CSA2_DEBUG_SYNC");
        return v != nullptr && v[0] == '1';
    }();
    return on;
}

csa2_status finish(hipError_t e, hipStream_t stream, const char* what)
{
    if (e == hipSuccess && debug_sync())
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(CSA2_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    g_err[0] = '\0';
    return CSA2_OK;
}

#define REQUIRE(cond, st, ...)                 \
    do {                                       \
        if (!(cond))                           \
            return fail((st), __VA_ARGS__);    \
    } while (0)

// Query rows (B * nq) a call takes; the workspace queries return 0 beyond it.
constexpr int64_t kMaxRows = 1ll << 24;

// A call whose launch would exceed one dispatch's 2^32 - 1 work-items.
constexpr const char* kTooLarge = "%s: a launch would need more than 2^32 - 1 work-items";

inline bool aligned(const void* p, size_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

}  // namespace

extern "C" {

const char* csa2_last_error(void)
{
    return g_err;
}

int32_t csa2_version(void)
{
    return 107;
}

csa2_status csa2_quantize_kv(const float* x, int64_t rows, int32_t channels,
                             const float* rope_cos, const float* rope_sin, int32_t rope_offset,
                             int32_t rope_dim, uint8_t* codes, uint8_t* scales,
                             int64_t dst_row, int64_t dst_stride, void* stream)
{
    REQUIRE(rows >= 0, CSA2_ERR_INVALID_ARG, "quantize_kv: rows < 0");
    REQUIRE(dst_row >= 0, CSA2_ERR_INVALID_ARG, "quantize_kv: dst_row < 0");
    REQUIRE(channels > 0 && channels % 16 == 0 && channels <= 4096, CSA2_ERR_UNSUPPORTED,
            "quantize_kv: channels must be a positive multiple of 16 up to 4096 (got %d)",
            channels);
    REQUIRE(dst_stride >= 1, CSA2_ERR_INVALID_ARG, "quantize_kv: dst_stride < 1");
    REQUIRE(rope_dim >= 0 && rope_dim % 2 == 0 && rope_offset >= 0 && rope_offset % 2 == 0 &&
                rope_offset + rope_dim <= channels,
            CSA2_ERR_INVALID_ARG, "quantize_kv: rotary range [%d, %d) not even / inside %d",
            rope_offset, rope_offset + rope_dim, channels);
    if (rows == 0)
        return CSA2_OK;
    REQUIRE(x && codes && scales, CSA2_ERR_INVALID_ARG, "quantize_kv: null pointer");
    REQUIRE(rope_dim == 0 || (rope_cos && rope_sin), CSA2_ERR_INVALID_ARG,
            "quantize_kv: rope_dim > 0 needs cos/sin tables");
    REQUIRE(aligned(x, 16) && aligned(codes, 8), CSA2_ERR_INVALID_ARG,
            "quantize_kv: x must be 16-byte and codes 8-byte aligned");
    REQUIRE(csa2::quantize_kv_fits(rows, channels), CSA2_ERR_UNSUPPORTED, kTooLarge, "quantize_kv");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_quantize_kv(x, rows, channels, rope_cos, rope_sin, rope_offset,
                                           rope_dim, codes, scales, dst_row, dst_stride, s),
                  s, "quantize_kv");
}

csa2_status csa2_quantize_swa(const float* x, int64_t n, int32_t row_len, uint8_t* out,
                              int64_t dst_stride, void* stream)
{
    REQUIRE(n >= 0, CSA2_ERR_INVALID_ARG, "quantize_swa: n < 0");
    REQUIRE(row_len > 0 && row_len % 4 == 0 && n % row_len == 0, CSA2_ERR_INVALID_ARG,
            "quantize_swa: row_len must be a positive multiple of 4 dividing n");
    REQUIRE(dst_stride >= 1, CSA2_ERR_INVALID_ARG, "quantize_swa: dst_stride < 1");
    if (n == 0)
        return CSA2_OK;
    REQUIRE(x && out, CSA2_ERR_INVALID_ARG, "quantize_swa: null pointer");
    REQUIRE(aligned(x, 16) && aligned(out, 4), CSA2_ERR_INVALID_ARG,
            "quantize_swa: x must be 16-byte and out 4-byte aligned");
    REQUIRE(csa2::quantize_swa_fits(n), CSA2_ERR_UNSUPPORTED, kTooLarge, "quantize_swa");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_quantize_swa(x, n, row_len, out, dst_stride, s), s,
                  "quantize_swa");
}

csa2_status csa2_encode_entries(int32_t rows, const float* kv_x, const float* rope_cos,
                                const float* rope_sin, int32_t rope_offset, int32_t rope_dim,
                                uint8_t* kv_codes, uint8_t* kv_scales, int64_t kv_stride,
                                const int64_t* kv_dst, int64_t dst_row, int64_t kv_cap,
                                const float* idx_x, const uint16_t* w_idx, uint8_t* idx_codes,
                                uint8_t* idx_scales, int64_t idx_stride, float* idx_y,
                                const float* swa_x, int32_t swa_rows, uint8_t* swa_out,
                                int64_t swa_stride, const int64_t* swa_dst, int64_t swa_cap,
                                void* stream)
{
    REQUIRE(rows >= 0 && swa_rows >= 0, CSA2_ERR_INVALID_ARG, "encode_entries: negative rows");
    REQUIRE(dst_row >= 0, CSA2_ERR_INVALID_ARG, "encode_entries: dst_row < 0");
    REQUIRE(kv_stride >= 1 && idx_stride >= 1 && swa_stride >= 1, CSA2_ERR_INVALID_ARG,
            "encode_entries: strides must be >= 1");
    REQUIRE(kv_cap >= 0 && swa_cap >= 0, CSA2_ERR_INVALID_ARG, "encode_entries: negative capacity");
    REQUIRE(aligned(kv_dst, 8) && aligned(swa_dst, 8), CSA2_ERR_INVALID_ARG,
            "encode_entries: misaligned destination index array");
    REQUIRE(rope_dim >= 0 && rope_dim % 2 == 0 && rope_offset >= 0 && rope_offset % 2 == 0 &&
                rope_offset + rope_dim <= csa2::kDim,
            CSA2_ERR_INVALID_ARG, "encode_entries: rotary range [%d, %d) not even / inside 512",
            rope_offset, rope_offset + rope_dim);
    if (rows == 0 && swa_rows == 0)
        return CSA2_OK;
    if (rows > 0) {
        REQUIRE(kv_x && kv_codes && kv_scales && idx_codes && idx_scales, CSA2_ERR_INVALID_ARG,
                "encode_entries: null main-KV or indexer-key pointer");
        REQUIRE(idx_x != nullptr || w_idx != nullptr, CSA2_ERR_INVALID_ARG,
                "encode_entries: indexer keys need their own rows or a projection matrix");
        REQUIRE(rope_dim == 0 || (rope_cos && rope_sin), CSA2_ERR_INVALID_ARG,
                "encode_entries: rope_dim > 0 needs cos/sin tables");
        REQUIRE(aligned(kv_x, 16) && aligned(idx_x, 16) && aligned(w_idx, 16) &&
                    aligned(kv_codes, 8) && aligned(idx_codes, 8) && aligned(idx_y, 8),
                CSA2_ERR_INVALID_ARG, "encode_entries: misaligned pointer");
    }
    if (swa_rows > 0) {
        REQUIRE(swa_x && swa_out, CSA2_ERR_INVALID_ARG, "encode_entries: null window pointer");
        REQUIRE(aligned(swa_x, 16) && aligned(swa_out, 4), CSA2_ERR_INVALID_ARG,
                "encode_entries: misaligned window pointer");
    }
    REQUIRE(csa2::encode_entries_fits(rows, idx_x != nullptr, swa_rows), CSA2_ERR_UNSUPPORTED,
            kTooLarge, "encode_entries");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_encode_entries(rows, kv_x, rope_cos, rope_sin, rope_offset,
                                              rope_dim, kv_codes, kv_scales, kv_stride, kv_dst,
                                              dst_row, kv_cap, idx_x, w_idx, idx_codes, idx_scales,
                                              idx_stride, idx_y, swa_x, swa_rows, swa_out,
                                              swa_stride, swa_dst, swa_cap, s),
                  s, "encode_entries");
}

static csa2_status check_indexer(const char* fn, const uint16_t* q, const float* w,
                                 const uint8_t* k_codes, const uint8_t* k_scales, int64_t n_cap,
                                 const int32_t* n_visible, int32_t B, int32_t nq, int32_t block)
{
    REQUIRE(B >= 0 && nq >= 0 && n_cap >= 0, CSA2_ERR_INVALID_ARG, "%s: negative size", fn);
    REQUIRE(block == csa2::kBlock, CSA2_ERR_UNSUPPORTED, "%s: block must be %d (got %d)", fn,
            csa2::kBlock, block);
    REQUIRE((int64_t)B * nq <= kMaxRows, CSA2_ERR_INVALID_ARG, "%s: too many query rows", fn);
    REQUIRE(n_cap <= (1ll << 30), CSA2_ERR_INVALID_ARG, "%s: n_cap above 2^30", fn);
    if ((int64_t)B * nq == 0)
        return CSA2_OK;
    REQUIRE(q && w && n_visible, CSA2_ERR_INVALID_ARG, "%s: null pointer", fn);
    REQUIRE(n_cap == 0 || (k_codes && k_scales), CSA2_ERR_INVALID_ARG, "%s: null key cache", fn);
    REQUIRE(aligned(q, 16) && aligned(k_codes, 16) && aligned(k_scales, 4), CSA2_ERR_INVALID_ARG,
            "%s: q and k_codes must be 16-byte, k_scales 4-byte aligned", fn);
    return CSA2_OK;
}

// The pool gathers address a sequence's keys with 32-bit offsets.
static csa2_status check_gather_cap(const char* fn, int64_t n_cap)
{
    REQUIRE(n_cap <= (1ll << 24), CSA2_ERR_UNSUPPORTED,
            "%s: more than 2^24 entries per sequence", fn);
    return CSA2_OK;
}

csa2_status csa2_index_full(const uint16_t* q, const float* w, const uint8_t* k_codes,
                            const uint8_t* k_scales, int64_t n_cap, const int32_t* n_visible,
                            int32_t B, int32_t nq, int32_t block, float* block_max,
                            float* scores, void* stream)
{
    csa2_status st = check_indexer("index_full", q, w, k_codes, k_scales, n_cap, n_visible, B,
                                   nq, block);
    if (st != CSA2_OK)
        return st;
    if ((int64_t)B * nq == 0 || n_cap == 0)
        return CSA2_OK;
    REQUIRE(block_max != nullptr, CSA2_ERR_INVALID_ARG, "index_full: null block_max");
    REQUIRE(csa2::index_full_fits(n_cap, B, nq), CSA2_ERR_UNSUPPORTED, kTooLarge, "index_full");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_index_full(q, w, k_codes, k_scales, n_cap, n_visible, B, nq,
                                          block_max, scores, nullptr, 0, nullptr, nullptr, s),
                  s, "index_full");
}

size_t csa2_index_full_pool_workspace(int64_t n_cap, int32_t rows, int32_t nb)
{
    if (n_cap < 0 || rows < 0 || nb < 1 || nb > csa2::kTopkMaxK || rows > kMaxRows)
        return 0;
    return csa2::topk_workspace((n_cap + csa2::kBlock - 1) / csa2::kBlock, rows, nb);
}

csa2_status csa2_index_full_pool(const uint16_t* q, const float* w, const uint8_t* k_codes,
                                 const uint8_t* k_scales, int64_t n_cap,
                                 const int32_t* n_visible, int32_t B, int32_t nq, int32_t block,
                                 int32_t nb, float* block_max, int32_t* pool, void* ws,
                                 size_t ws_bytes, void* scan_start, void* scan_stop,
                                 void* stream)
{
    csa2_status st = check_indexer("index_full_pool", q, w, k_codes, k_scales, n_cap, n_visible,
                                   B, nq, block);
    if (st != CSA2_OK)
        return st;
    REQUIRE(nb >= 1 && nb <= csa2::kTopkMaxK, CSA2_ERR_UNSUPPORTED,
            "index_full_pool: nb must be in [1, %d]", csa2::kTopkMaxK);
    const int64_t rows = (int64_t)B * nq;
    const int64_t L = (n_cap + csa2::kBlock - 1) / csa2::kBlock;
    REQUIRE(rows * ((L + csa2::kTopkSegment - 1) / csa2::kTopkSegment) <= (1ll << 31) - 1,
            CSA2_ERR_INVALID_ARG, "index_full_pool: too many segments");
    if (rows == 0)
        return CSA2_OK;
    // an empty cache has no block maxima to write (block_max may be null); the
    // pool is then all -1
    REQUIRE(pool != nullptr && (n_cap == 0 || block_max != nullptr), CSA2_ERR_INVALID_ARG,
            "index_full_pool: null block_max or pool");
    const size_t need = csa2::topk_workspace(L, (int32_t)rows, nb);
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA2_ERR_WORKSPACE,
            "index_full_pool: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    REQUIRE(aligned(ws, 8), CSA2_ERR_INVALID_ARG,
            "index_full_pool: workspace must be 8-byte aligned");
    REQUIRE(csa2::index_full_fits(n_cap, B, nq) && csa2::topk_fits(L, rows, nb),
            CSA2_ERR_UNSUPPORTED, kTooLarge, "index_full_pool");
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the scan writes the block select's group maxima itself when the groups
    // align with its chunks (group size dividing 64 blocks)
    const int32_t g = csa2::topk_group_size(L, nb);
    const bool fused = g > 0 && 64 % g == 0 && n_cap > 0;  // g in {1, 2, 4, 8, ...}: a power of two
    hipError_t e = hipSuccess;
    if (n_cap > 0)
        e = csa2::launch_index_full(q, w, k_codes, k_scales, n_cap, n_visible, B, nq, block_max,
                                    nullptr, fused ? static_cast<uint32_t*>(ws) : nullptr,
                                    fused ? g : 0, static_cast<hipEvent_t>(scan_start),
                                    static_cast<hipEvent_t>(scan_stop), s);
    if (e == hipSuccess)
        e = csa2::launch_topk(block_max, nullptr, L, (int32_t)rows, n_visible, csa2::kBlock, nb,
                              pool, ws, fused, s);
    return finish(e, s, "index_full_pool");
}

// How csa2_index_full_select runs for a shape.  The pool and the top-k blocks
// come from the direct block select (mode 0: rows of at most 16384 blocks),
// the scan's per-chunk candidates (mode 1: one-row scan, groups of g blocks
// that the scan also writes as the exact fallback), or two csa2_topk calls
// over the block maxima (mode 2).  The top-k entries are the top-k blocks'
// positions rescored: pool rescoring + top-k in one launch (rescore_fused;
// its arrival counters are cleared by the block select), or a pool scan and
// csa2_topk.
// The fused rescoring (pool_topk_kernel) wins while few positions are rescored
// (latency-bound: one launch instead of two); beyond about 32 rows x 4096
// positions the pool scan (8 key tiles per wave in flight) and csa2_topk are
// faster -- measured on the MI355X: 16 x 4096 positions 14.2 vs 18.2 us,
// 64 x 4096 26.1 vs 18.3 us, 128 x 16384 139.4 vs 58.5 us.
constexpr int64_t kFusedRescoreMaxPositions = 32 * 4096;

struct FullSelectPlan {
    int mode;
    int64_t L;            // blocks per row
    int32_t g;            // group size (mode 1)
    int32_t chunks, kl;   // block candidate lists (mode 1)
    bool rescore_fused;
    size_t off_cand_key, off_cand_blk, off_cand_full;
    size_t off_tb;        // top-k blocks [rows, k]
    size_t off_rescore;   // pool_topk workspace (rescore_fused)
    size_t off_pscore, off_pidx, off_topk_ws;
    size_t ws_bytes;
};

static FullSelectPlan full_select_plan(int64_t n_cap, int32_t B, int32_t nq, int32_t nb, int32_t k)
{
    FullSelectPlan P{};
    const int64_t rows = (int64_t)B * nq;
    P.L = (n_cap + csa2::kBlock - 1) / csa2::kBlock;
    const int32_t tmax = nb > k ? nb : k;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) / 256 * 256;
        return o;
    };
    P.mode = P.L <= csa2::kTopkSegment ? 0 : 2;
    if (P.mode == 2) {
        const csa2::ScanShape sh = csa2::scan_shape(n_cap, B, nq);
        const int32_t g = csa2::topk_group_size(P.L, tmax);
        if (!sh.multi_row && g > 0 && 64 % g == 0) {
            // about twice a chunk's share of the winners, at least 64, a power of two
            const int32_t per = (tmax + sh.chunks_per_row - 1) / sh.chunks_per_row;
            int32_t kl = 64;
            while (kl < 2 * per)
                kl *= 2;
            if (kl <= sh.max_blocks_per_chunk && (int64_t)sh.chunks_per_row * kl <= csa2::kTopkSegment) {
                P.mode = 1;
                P.g = g;
                P.chunks = sh.chunks_per_row;
                P.kl = kl;
                const size_t nc = (size_t)rows * P.chunks * kl;
                take((size_t)rows * (size_t)((P.L + g - 1) / g) * 4);  // group keys, at 0
                P.off_cand_key = take(nc * 4);
                P.off_cand_blk = take(nc * 4);
                P.off_cand_full = take((size_t)rows * P.chunks * 4);
            }
        }
    }
    // the top-k blocks, then their positions rescored
    const size_t L8 = (size_t)k * csa2::kBlock;
    if (P.mode == 2) {
        size_t t = csa2::topk_workspace(P.L, (int32_t)rows, nb > 0 ? nb : 1);
        const size_t t2 = csa2::topk_workspace(P.L, (int32_t)rows, k);
        const size_t t3 = csa2::topk_workspace((int64_t)L8, (int32_t)rows, k);
        t = t > t2 ? t : t2;
        P.off_topk_ws = take(t > t3 ? t : t3);
    }
    P.off_tb = take((size_t)rows * k * 4);
    P.rescore_fused = P.mode != 2 && (int64_t)L8 <= csa2::kTopkSegment &&
                      rows * (int64_t)L8 <= kFusedRescoreMaxPositions;
    if (P.rescore_fused) {
        P.off_rescore = take(csa2::pool_topk_workspace((int32_t)rows, k));
    } else {
        const size_t pos_bytes = (size_t)rows * L8 * 4;  // rows x k blocks x 8 positions
        P.off_pscore = take(pos_bytes);
        P.off_pidx = take(pos_bytes);
        if (P.mode != 2)
            P.off_topk_ws = take(csa2::topk_workspace((int64_t)L8, (int32_t)rows, k));
    }
    P.ws_bytes = off;
    return P;
}

size_t csa2_index_full_select_workspace(int64_t n_cap, int32_t B, int32_t nq, int32_t nb,
                                        int32_t k)
{
    if (n_cap < 0 || B < 0 || nq < 0 || nb < 0 || k < 1 || nb > csa2::kTopkMaxK ||
        k > csa2::kTopkMaxK || (int64_t)B * nq > kMaxRows)
        return 0;
    return full_select_plan(n_cap, B, nq, nb, k).ws_bytes;
}

csa2_status csa2_index_full_select(const uint16_t* q, const float* w, const uint8_t* k_codes,
                                   const uint8_t* k_scales, int64_t n_cap,
                                   const int32_t* n_visible, int32_t B, int32_t nq,
                                   int32_t block, int32_t nb, int32_t k, float* block_max,
                                   int32_t* pool, int32_t* topk, void* ws, size_t ws_bytes,
                                   void* scan_start, void* scan_stop, void* stream)
{
    csa2_status st = check_indexer("index_full_select", q, w, k_codes, k_scales, n_cap,
                                   n_visible, B, nq, block);
    if (st != CSA2_OK)
        return st;
    st = check_gather_cap("index_full_select", n_cap);
    if (st != CSA2_OK)
        return st;
    REQUIRE(nb >= 0 && nb <= csa2::kTopkMaxK && k >= 1 && k <= csa2::kTopkMaxK,
            CSA2_ERR_UNSUPPORTED, "index_full_select: nb must be in [0, %d], k in [1, %d]",
            csa2::kTopkMaxK, csa2::kTopkMaxK);
    const int64_t rows = (int64_t)B * nq;
    const int64_t L = (n_cap + csa2::kBlock - 1) / csa2::kBlock;
    REQUIRE(rows * ((L + csa2::kTopkSegment - 1) / csa2::kTopkSegment) <= (1ll << 31) - 1,
            CSA2_ERR_INVALID_ARG, "index_full_select: too many segments");
    REQUIRE(rows * k * csa2::kBlock <= (1ll << 31) - 1, CSA2_ERR_INVALID_ARG,
            "index_full_select: too many rescored positions");
    if (rows == 0)
        return CSA2_OK;
    REQUIRE(topk != nullptr && (nb == 0 || pool != nullptr) &&
                (n_cap == 0 || block_max != nullptr),
            CSA2_ERR_INVALID_ARG, "index_full_select: null block_max, pool or topk");
    const FullSelectPlan P = full_select_plan(n_cap, B, nq, nb, k);
    REQUIRE(ws_bytes >= P.ws_bytes && (P.ws_bytes == 0 || ws != nullptr), CSA2_ERR_WORKSPACE,
            "index_full_select: workspace of %zu bytes needed, %zu given", P.ws_bytes, ws_bytes);
    REQUIRE(aligned(ws, 256), CSA2_ERR_INVALID_ARG,
            "index_full_select: workspace must be 256-byte aligned");
    int32_t* pool_out = nb > 0 ? pool : nullptr;
    {
        // every launch the plan below makes
        const bool select_fits =
            P.mode != 2 ? csa2::block_select_fits(rows, pool_out != nullptr ? 2 : 1)
                        : (nb == 0 || csa2::topk_fits(L, rows, nb)) && csa2::topk_fits(L, rows, k);
        const bool rescore_fits =
            P.rescore_fused ? csa2::pool_topk_fits(rows, k)
                            : csa2::index_pool_fits(rows, k) &&
                                  csa2::topk_fits((int64_t)k * csa2::kBlock, rows, k);
        REQUIRE(csa2::index_full_fits(n_cap, B, nq) && select_fits && rescore_fits,
                CSA2_ERR_UNSUPPORTED, kTooLarge, "index_full_select");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* wsb = static_cast<char*>(ws);
    auto at = [wsb](size_t off) { return static_cast<void*>(wsb + off); };
    int32_t* tb = static_cast<int32_t*>(at(P.off_tb));
    hipError_t e = hipSuccess;
    const hipEvent_t ev0 = static_cast<hipEvent_t>(scan_start);
    const hipEvent_t ev1 = static_cast<hipEvent_t>(scan_stop);

    csa2::BlockSelect S;
    S.block_max = block_max;
    S.L = L;
    S.rows = (int32_t)rows;
    S.n_visible = n_visible;
    S.nb = nb;
    S.k = k;
    S.pool = pool_out;
    S.sel = tb;
    if (P.mode == 1) {
        uint32_t* ck = static_cast<uint32_t*>(at(P.off_cand_key));
        int32_t* cb = static_cast<int32_t*>(at(P.off_cand_blk));
        int32_t* cf = static_cast<int32_t*>(at(P.off_cand_full));
        e = csa2::launch_index_full(q, w, k_codes, k_scales, n_cap, n_visible, B, nq, block_max,
                                    nullptr, static_cast<uint32_t*>(at(0)), P.g, ev0, ev1, s, ck,
                                    cb, cf, P.kl);
        S.gkey = static_cast<const uint32_t*>(at(0));
        S.g = P.g;
        S.cand_key = ck;
        S.cand_blk = cb;
        S.cand_full = cf;
        S.chunks = P.chunks;
        S.kl = P.kl;
    } else if (n_cap > 0) {
        e = csa2::launch_index_full(q, w, k_codes, k_scales, n_cap, n_visible, B, nq, block_max,
                                    nullptr, nullptr, 0, ev0, ev1, s);
    }
    if (P.rescore_fused)
        S.zero_counters = static_cast<uint32_t*>(at(P.off_rescore));  // its arrival counters
    if (e == hipSuccess) {
        if (P.mode != 2) {
            e = csa2::launch_block_select(S, s);
        } else {
            if (nb > 0)
                e = csa2::launch_topk(block_max, nullptr, L, (int32_t)rows, n_visible,
                                      csa2::kBlock, nb, pool_out, at(P.off_topk_ws), false, s);
            if (e == hipSuccess)
                e = csa2::launch_topk(block_max, nullptr, L, (int32_t)rows, n_visible,
                                      csa2::kBlock, k, tb, at(P.off_topk_ws), false, s);
        }
    }
    if (e == hipSuccess) {
        // the top-k entries: the top-k blocks' positions rescored
        if (P.rescore_fused) {
            e = csa2::launch_pool_topk(q, w, k_codes, k_scales, n_cap, tb, k, n_visible, B, nq, k,
                                       topk, at(P.off_rescore), s);
        } else {
            float* ps = static_cast<float*>(at(P.off_pscore));
            int32_t* pi = static_cast<int32_t*>(at(P.off_pidx));
            e = csa2::launch_index_pool(q, w, k_codes, k_scales, n_cap, tb, k, n_visible, B, nq,
                                        ps, pi, s);
            if (e == hipSuccess)
                e = csa2::launch_topk(ps, pi, (int64_t)k * csa2::kBlock, (int32_t)rows, nullptr, 1,
                                      k, topk, at(P.off_topk_ws), false, s);
        }
    }
    return finish(e, s, "index_full_select");
}

csa2_status csa2_index_pool(const uint16_t* q, const float* w, const uint8_t* k_codes,
                            const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                            int32_t n_blocks, int32_t block, const int32_t* n_visible, int32_t B,
                            int32_t nq, float* pool_score, int32_t* pool_idx, void* stream)
{
    csa2_status st = check_indexer("index_pool", q, w, k_codes, k_scales, n_cap, n_visible, B,
                                   nq, block);
    if (st != CSA2_OK)
        return st;
    st = check_gather_cap("index_pool", n_cap);
    if (st != CSA2_OK)
        return st;
    REQUIRE(n_blocks >= 0 && n_blocks <= (1 << 20), CSA2_ERR_INVALID_ARG,
            "index_pool: n_blocks out of range");
    if ((int64_t)B * nq == 0 || n_blocks == 0)
        return CSA2_OK;
    REQUIRE(blocks && pool_score && pool_idx, CSA2_ERR_INVALID_ARG, "index_pool: null pointer");
    REQUIRE(csa2::index_pool_fits((int64_t)B * nq, n_blocks), CSA2_ERR_UNSUPPORTED, kTooLarge,
            "index_pool");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_index_pool(q, w, k_codes, k_scales, n_cap, blocks, n_blocks,
                                          n_visible, B, nq, pool_score, pool_idx, s),
                  s, "index_pool");
}

size_t csa2_index_pool_topk_workspace(int32_t B, int32_t nq, int32_t n_blocks)
{
    if (B < 0 || nq < 0 || n_blocks < 0 || n_blocks > csa2::kTopkSegment / csa2::kBlock ||
        (int64_t)B * nq > kMaxRows)
        return 0;
    return csa2::pool_topk_workspace(B * nq, n_blocks);
}

csa2_status csa2_index_pool_topk(const uint16_t* q, const float* w, const uint8_t* k_codes,
                                 const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                                 int32_t n_blocks, int32_t block, const int32_t* n_visible,
                                 int32_t B, int32_t nq, int32_t k, int32_t* topk, void* ws,
                                 size_t ws_bytes, void* stream)
{
    csa2_status st = check_indexer("index_pool_topk", q, w, k_codes, k_scales, n_cap, n_visible,
                                   B, nq, block);
    if (st != CSA2_OK)
        return st;
    st = check_gather_cap("index_pool_topk", n_cap);
    if (st != CSA2_OK)
        return st;
    REQUIRE(n_blocks >= 0 && n_blocks <= csa2::kTopkSegment / csa2::kBlock, CSA2_ERR_UNSUPPORTED,
            "index_pool_topk: n_blocks must be in [0, %d]", csa2::kTopkSegment / csa2::kBlock);
    REQUIRE(k >= 1 && k <= csa2::kTopkMaxK, CSA2_ERR_UNSUPPORTED,
            "index_pool_topk: k must be in [1, %d]", csa2::kTopkMaxK);
    if ((int64_t)B * nq == 0)
        return CSA2_OK;
    REQUIRE(topk != nullptr && (n_blocks == 0 || blocks != nullptr), CSA2_ERR_INVALID_ARG,
            "index_pool_topk: null pointer");
    const size_t need = csa2::pool_topk_workspace(B * nq, n_blocks);
    REQUIRE(ws != nullptr && ws_bytes >= need, CSA2_ERR_WORKSPACE,
            "index_pool_topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    REQUIRE(aligned(ws, 256), CSA2_ERR_INVALID_ARG,
            "index_pool_topk: workspace must be 256-byte aligned");
    REQUIRE(csa2::pool_topk_fits((int64_t)B * nq, n_blocks), CSA2_ERR_UNSUPPORTED, kTooLarge,
            "index_pool_topk");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_pool_topk(q, w, k_codes, k_scales, n_cap, blocks, n_blocks,
                                         n_visible, B, nq, k, topk, ws, s),
                  s, "index_pool_topk");
}

size_t csa2_topk_workspace(int64_t L, int32_t rows, int32_t k)
{
    if (L < 0 || rows < 0 || k < 1 || k > csa2::kTopkMaxK)
        return 0;
    return csa2::topk_workspace(L, rows, k);
}

csa2_status csa2_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                      const int32_t* n_valid, int32_t k, int32_t* out, void* ws,
                      size_t ws_bytes, void* stream)
{
    REQUIRE(L >= 0 && rows >= 0, CSA2_ERR_INVALID_ARG, "topk: negative size");
    REQUIRE(k >= 1 && k <= csa2::kTopkMaxK, CSA2_ERR_UNSUPPORTED, "topk: k must be in [1, %d]",
            csa2::kTopkMaxK);
    REQUIRE(L <= (1ll << 31) - 1, CSA2_ERR_INVALID_ARG, "topk: L above 2^31-1");
    REQUIRE((int64_t)rows * ((L + csa2::kTopkSegment - 1) / csa2::kTopkSegment) <= (1ll << 31) - 1,
            CSA2_ERR_INVALID_ARG, "topk: too many segments");
    REQUIRE(csa2::topk_fits(L, rows, k), CSA2_ERR_UNSUPPORTED, kTooLarge, "topk");
    if (rows == 0)
        return CSA2_OK;
    REQUIRE(out != nullptr, CSA2_ERR_INVALID_ARG, "topk: null out");
    REQUIRE(L == 0 || score != nullptr, CSA2_ERR_INVALID_ARG, "topk: null score");
    const size_t need = csa2::topk_workspace(L, rows, k);
    REQUIRE(ws_bytes >= need && (need == 0 || ws != nullptr), CSA2_ERR_WORKSPACE,
            "topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
    REQUIRE(aligned(ws, 8), CSA2_ERR_INVALID_ARG, "topk: workspace must be 8-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_topk(score, idx, L, rows, n_valid, 1, k, out, ws, false, s), s,
                  "topk");
}

csa2_status csa2_topk_noalloc(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                              const int32_t* n_valid, int32_t k, int32_t* out, void* stream)
{
    REQUIRE(L >= 0 && rows >= 0, CSA2_ERR_INVALID_ARG, "topk_noalloc: negative size");
    REQUIRE(k >= 1 && k <= csa2::kTopkMaxK, CSA2_ERR_UNSUPPORTED,
            "topk_noalloc: k must be in [1, %d]", csa2::kTopkMaxK);
    REQUIRE(L <= (1ll << 31) - 1, CSA2_ERR_INVALID_ARG, "topk_noalloc: L above 2^31-1");
    REQUIRE((int64_t)rows * ((L + csa2::kTopkSegment - 1) / csa2::kTopkSegment) <= (1ll << 31) - 1,
            CSA2_ERR_INVALID_ARG, "topk_noalloc: too many segments");
    REQUIRE(csa2::topk_fits(L, rows, k), CSA2_ERR_UNSUPPORTED, kTooLarge, "topk_noalloc");
    if (rows == 0)
        return CSA2_OK;
    REQUIRE(out != nullptr, CSA2_ERR_INVALID_ARG, "topk_noalloc: null out");
    REQUIRE(L == 0 || score != nullptr, CSA2_ERR_INVALID_ARG, "topk_noalloc: null score");
    const size_t need = csa2::topk_workspace(L, rows, k);
    REQUIRE(need <= csa2::kTopkScratchBytes, CSA2_ERR_WORKSPACE,
            "topk_noalloc: needs %zu bytes of workspace, above the static %zu", need,
            (size_t)csa2::kTopkScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = csa2::topk_scratch(&ws);
        if (e != hipSuccess)
            return fail(CSA2_ERR_LAUNCH, "topk_noalloc: static workspace address: %s",
                        hipGetErrorString(e));
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_topk(score, idx, L, rows, n_valid, 1, k, out, ws, false, s), s,
                  "topk_noalloc");
}

csa2_status csa2_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t depth,
                             uint32_t* sink, void* stream)
{
    REQUIRE(bytes >= 0 && bytes % 16 == 0, CSA2_ERR_INVALID_ARG,
            "stream_read: bytes must be a non-negative multiple of 16");
    REQUIRE(workgroups >= 1 && workgroups <= (1 << 20), CSA2_ERR_INVALID_ARG,
            "stream_read: workgroups must be in [1, 2^20]");
    REQUIRE(depth == 1 || depth == 2 || depth == 4 || depth == 8, CSA2_ERR_UNSUPPORTED,
            "stream_read: depth must be 1, 2, 4 or 8");
    REQUIRE(bytes / workgroups < (1ll << 30), CSA2_ERR_INVALID_ARG,
            "stream_read: slices above 1 GiB");
    if (bytes == 0)
        return CSA2_OK;
    REQUIRE(src && sink, CSA2_ERR_INVALID_ARG, "stream_read: null pointer");
    REQUIRE(aligned(src, 16), CSA2_ERR_INVALID_ARG, "stream_read: src must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_stream_read(src, bytes, workgroups, depth, sink, s), s,
                  "stream_read");
}

size_t csa2_sparse_attn_workspace(int32_t B, int32_t nq, int32_t k, int32_t n_win)
{
    if (B < 0 || nq < 0 || k < 0 || n_win < 0 || (int64_t)B * nq > kMaxRows)
        return 0;
    return csa2::attn_workspace(B * nq, k, n_win);
}

static csa2_status attn_common(const uint16_t* q, int32_t B, int32_t nq,
                               const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                               const int32_t* topk, int32_t k, const uint8_t* swa,
                               int32_t swa_cap, const int32_t* swa_end, int32_t n_win,
                               float softmax_scale, float* out, uint16_t* out_bf16,
                               const float* rope_cos, const float* rope_sin, int32_t rope_offset,
                               int32_t rope_dim, float* lse, void* ws, size_t ws_bytes,
                               void* stream, const char* name)
{
    REQUIRE(B >= 0 && nq >= 0 && n_cap >= 0 && k >= 0 && swa_cap >= 0 && n_win >= 0,
            CSA2_ERR_INVALID_ARG, "%s: negative size", name);
    REQUIRE((int64_t)B * nq <= kMaxRows, CSA2_ERR_INVALID_ARG, "%s: too many query rows", name);
    REQUIRE(k <= 65536 && n_win <= 65536, CSA2_ERR_UNSUPPORTED, "%s: k or n_win too large", name);
    // the kernels address a sequence's rows with 32-bit byte offsets
    REQUIRE(n_cap <= (1ll << 24) && swa_cap <= (1 << 22), CSA2_ERR_UNSUPPORTED,
            "%s: more than 2^24 main entries or 2^22 window rows per sequence", name);
    const int32_t queries = B * nq;
    if (queries == 0)
        return CSA2_OK;
    REQUIRE(q && (out || out_bf16) && swa_end, CSA2_ERR_INVALID_ARG, "%s: null pointer", name);
    // an empty main cache (n_cap == 0) may come as null pointers: every top-k
    // index is then out of range and skipped, and the kernels never read it
    REQUIRE(k == 0 || (topk && (n_cap == 0 || (kv_codes && kv_scales))), CSA2_ERR_INVALID_ARG,
            "%s: null top-k or KV cache", name);
    REQUIRE(swa_cap == 0 || swa != nullptr, CSA2_ERR_INVALID_ARG, "%s: null window", name);
    REQUIRE(aligned(q, 16) && aligned(kv_codes, 16) && aligned(kv_scales, 4) && aligned(swa, 16) &&
                aligned(out, 16) && aligned(out_bf16, 8),
            CSA2_ERR_INVALID_ARG, "%s: misaligned q / kv / window / out pointer", name);
    if (out_bf16 != nullptr) {
        REQUIRE(rope_dim >= 0 && rope_offset >= 0 && rope_dim % 2 == 0 && rope_offset % 2 == 0 &&
                    rope_offset + rope_dim <= csa2::kDim,
                CSA2_ERR_INVALID_ARG, "%s: rotary range must be even and inside the 512 channels",
                name);
        REQUIRE(rope_dim == 0 || (rope_cos && rope_sin), CSA2_ERR_INVALID_ARG,
                "%s: null rotary table", name);
    }
    REQUIRE(ws == nullptr || aligned(ws, 16), CSA2_ERR_INVALID_ARG, "%s: misaligned workspace",
            name);
    REQUIRE(csa2::sparse_attn_fits(queries), CSA2_ERR_UNSUPPORTED, kTooLarge, name);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(csa2::launch_sparse_attn(q, queries, nq, kv_codes, kv_scales, n_cap, topk, k,
                                           swa, swa_cap, swa_end, n_win, softmax_scale, out,
                                           out_bf16, rope_cos, rope_sin, rope_offset, rope_dim,
                                           lse, ws, ws_bytes, s),
                  s, name);
}

csa2_status csa2_sparse_attn(const uint16_t* q, int32_t B, int32_t nq, const uint8_t* kv_codes,
                             const uint8_t* kv_scales, int64_t n_cap, const int32_t* topk,
                             int32_t k, const uint8_t* swa, int32_t swa_cap,
                             const int32_t* swa_end, int32_t n_win, float softmax_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream)
{
    REQUIRE(out != nullptr || (int64_t)B * nq == 0 || B < 0 || nq < 0, CSA2_ERR_INVALID_ARG,
            "sparse_attn: null pointer");
    return attn_common(q, B, nq, kv_codes, kv_scales, n_cap, topk, k, swa, swa_cap, swa_end,
                       n_win, softmax_scale, out, nullptr, nullptr, nullptr, 0, 0, lse, ws,
                       ws_bytes, stream, "sparse_attn");
}

csa2_status csa2_sparse_attn_rope_bf16(const uint16_t* q, int32_t B, int32_t nq,
                                       const uint8_t* kv_codes, const uint8_t* kv_scales,
                                       int64_t n_cap, const int32_t* topk, int32_t k,
                                       const uint8_t* swa, int32_t swa_cap,
                                       const int32_t* swa_end, int32_t n_win,
                                       float softmax_scale, const float* rope_cos,
                                       const float* rope_sin, int32_t rope_offset,
                                       int32_t rope_dim, uint16_t* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream)
{
    REQUIRE(out != nullptr || (int64_t)B * nq == 0 || B < 0 || nq < 0, CSA2_ERR_INVALID_ARG,
            "sparse_attn_rope_bf16: null pointer");
    return attn_common(q, B, nq, kv_codes, kv_scales, n_cap, topk, k, swa, swa_cap, swa_end,
                       n_win, softmax_scale, nullptr, out, rope_cos, rope_sin, rope_offset,
                       rope_dim, lse, ws, ws_bytes, stream, "sparse_attn_rope_bf16");
}

}  // extern "C"
