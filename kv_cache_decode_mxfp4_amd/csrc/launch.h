// Host-side launchers of the libcsa2 kernels.  The C ABI (api.hip) validates
// arguments and then calls exactly one of these; each enqueues its kernels on
// the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dims.h"

namespace csa2 {

// A dispatch counts its grid in work-items with 32 bits, so one launch holds
// at most 2^32 - 1 work-items.  Each launcher checks its grids against that
// before enqueueing anything (hipErrorInvalidConfiguration otherwise), and the
// *_fits functions below answer the same question for the C ABI's argument
// validation, which rejects an oversized call before any of its launches.
constexpr int64_t kMaxWorkItems = 0xFFFFFFFFll;
inline bool grid_fits(int64_t workgroups, int64_t threads)
{
    return workgroups >= 0 && workgroups <= kMaxWorkItems / threads;
}
bool quantize_kv_fits(int64_t rows, int32_t channels);
bool quantize_swa_fits(int64_t n);
bool encode_entries_fits(int32_t rows, bool idx_rows_given, int32_t swa_rows);
bool index_full_fits(int64_t n_cap, int32_t B, int32_t nq);
bool index_pool_fits(int64_t rows, int32_t n_blocks);
bool pool_topk_fits(int64_t rows, int32_t n_blocks);
bool block_select_fits(int64_t rows, int32_t passes);
bool topk_fits(int64_t L, int64_t rows, int32_t k);
bool sparse_attn_fits(int32_t queries);

hipError_t launch_quantize_kv(const float* x, int64_t rows, int32_t channels, const float* cs,
                              const float* sn, int32_t rope_off, int32_t rope_dim, uint8_t* codes,
                              uint8_t* scales, int64_t dst_row, int64_t dst_stride,
                              hipStream_t stream);

hipError_t launch_quantize_swa(const float* x, int64_t n, int32_t row_len, uint8_t* out,
                               int64_t dst_stride, hipStream_t stream);

// New entries of one step in one launch: main-KV rows (rotary + MXFP4), the
// indexer-key rows (their own fp32 rows idx_x, or projected from kv_x by the
// bf16 [128, 512] matrix w_idx when idx_x is null; idx_y optionally receives
// the fp32 projection), and the FP8 window rows.
hipError_t launch_encode_entries(int32_t rows, const float* kv_x, const float* cs, const float* sn,
                                 int32_t rope_off, int32_t rope_dim, uint8_t* kv_codes,
                                 uint8_t* kv_scales, int64_t kv_stride, const int64_t* kv_dst,
                                 int64_t dst_row, int64_t kv_cap, const float* idx_x,
                                 const uint16_t* w_idx, uint8_t* idx_codes, uint8_t* idx_scales,
                                 int64_t idx_stride, float* idx_y, const float* swa_x,
                                 int32_t swa_rows, uint8_t* swa_out, int64_t swa_stride,
                                 const int64_t* swa_dst, int64_t swa_cap, hipStream_t stream);

// group_keys (or null): also write the selection order key of the maximum of
// every group of `group` consecutive blocks, [B*nq, ceil(ceil(n_cap/8)/group)]
// (0 for groups with no visible block); group must be a power of two <= 64.
// ev_start / ev_stop (or null): HIP events the scan kernel's dispatch records
// at its start and end.
// cand_key / cand_blk / cand_full (or null; one-row scan only): each chunk's
// kl best blocks for the block select, [B*nq, chunks, kl] and [B*nq, chunks]
// (ScanShape::chunks_per_row chunks per row).
hipError_t launch_index_full(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* n_visible,
                             int32_t B, int32_t nq, float* block_max, float* scores,
                             uint32_t* group_keys, int32_t group, hipEvent_t ev_start,
                             hipEvent_t ev_stop, hipStream_t stream,
                             uint32_t* cand_key = nullptr, int32_t* cand_blk = nullptr,
                             int32_t* cand_full = nullptr, int32_t kl = 0);

// How the scan cuts rows into chunks (one workgroup per chunk and row, or per
// chunk and group of 8 rows when `multi_row`).
struct ScanShape {
    int32_t chunk;                 // entries per chunk
    int32_t chunks_per_row;
    int32_t max_blocks_per_chunk;  // chunk / 8
    bool multi_row;
};
ScanShape scan_shape(int64_t n_cap, int32_t B, int32_t nq);

// Pool (top-nb blocks) and top-k blocks of every row in one launch.  Direct
// form (cand_key null): keys are the block maxima, L <= 16384.  Candidate
// form: the scan's per-chunk lists [rows, chunks, kl] (chunks * kl <= 16384,
// kl a multiple of 64), with the exact grouped select over the group maxima
// gkey ([rows, ceil(L/g)], groups of g) as the fallback.  pool / sel may be
// null (target skipped).  zero_counters (or null): [rows] set to zero (the
// arrival counters of a following pool rescoring).
struct BlockSelect {
    const float* block_max = nullptr;
    int64_t L = 0;
    int32_t rows = 0;
    const int32_t* n_visible = nullptr;
    const uint32_t* gkey = nullptr;
    int32_t g = 0;
    const uint32_t* cand_key = nullptr;
    const int32_t* cand_blk = nullptr;
    const int32_t* cand_full = nullptr;
    int32_t chunks = 0, kl = 0;
    int32_t nb = 0, k = 0;
    int32_t* pool = nullptr;
    int32_t* sel = nullptr;
    uint32_t* zero_counters = nullptr;
};
hipError_t launch_block_select(const BlockSelect& S, hipStream_t stream);

hipError_t launch_index_pool(const uint16_t* q, const float* w, const uint8_t* k_codes,
                             const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                             int32_t n_blocks, const int32_t* n_visible, int32_t B, int32_t nq,
                             float* pool_score, int32_t* pool_idx, hipStream_t stream);

// Pool rescoring + top-k in one launch (n_blocks * 8 <= 16384).  ws: rows
// arrival counters (zero before the first use; every call leaves them zero)
// then the slots' scores and positions.
size_t pool_topk_workspace(int32_t rows, int32_t n_blocks);
hipError_t launch_pool_topk(const uint16_t* q, const float* w, const uint8_t* k_codes,
                            const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                            int32_t n_blocks, const int32_t* n_visible, int32_t B, int32_t nq,
                            int32_t k, int32_t* out, void* ws, hipStream_t stream);

size_t topk_workspace(int64_t L, int32_t rows, int32_t k);
// Group size of the grouped select for a row of L keys and k winners (0: the
// direct or segment path); its group maxima live at the front of the workspace
// as uint32 order keys [rows, ceil(L / g)].
int32_t topk_group_size(int64_t L, int32_t k);
// n_valid[row] / valid_div (rounded up) is the row's valid prefix (valid_div 8:
// visible entries -> visible blocks).  group_keys_ready: the workspace already
// holds the group maxima (written by the scan), so they are not recomputed.
// Device address of the calling thread's current GPU's static top-k scratch
// (kTopkScratchBytes), looked up once per device.
hipError_t topk_scratch(void** ptr);
hipError_t launch_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                       const int32_t* n_valid, int32_t valid_div, int32_t k, int32_t* out,
                       void* ws, bool group_keys_ready, hipStream_t stream);

// Bytes of the key-split partials for few query rows (0: no split).
size_t attn_workspace(int32_t queries, int32_t k, int32_t n_win);
// out (fp32) or out_bf16 (inverse rotary on [rope_off, rope_off + rope_dim)
// with the query's rope_cos / rope_sin, then bf16): exactly one is non-null.
hipError_t launch_sparse_attn(const uint16_t* q, int32_t queries, int32_t nq,
                              const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                              const int32_t* topk, int32_t k, const uint8_t* swa,
                              int32_t swa_cap, const int32_t* swa_end, int32_t n_win,
                              float softmax_scale, float* out, uint16_t* out_bf16,
                              const float* rope_cos, const float* rope_sin, int32_t rope_off,
                              int32_t rope_dim, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream);

// Streaming read of `bytes` bytes (calibration): `workgroups` slices, `depth`
// 16-byte loads per lane in flight (1, 2, 4 or 8); sink [workgroups].
hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t depth,
                              uint32_t* sink, hipStream_t stream);

}  // namespace csa2
