/*
 * csa2.h -- C ABI of libcsa2, the MI355X (gfx950) hot path of a CSA2 layer
 * (compressed sparse attention 2) of DeepSeek-V4.1-Flash at decode and in
 * chunked prefill, on one GPU.
 *
 * Sources, by page title:
 *   [N] "DeepSeek V4.1: model architecture and system design, close reading"
 *       section 1 (indexer 32 heads x 128, top-k 512, query 64 heads x 512,
 *       2048 blocks x 8 positions, window 128), section 2.2 (CSA2 Full /
 *       Reindex / Reuse modes, hierarchical sparse indexer), section 2.3 (FP4
 *       main KV: E2M1 with one E4M3 scale per 16 channels, quantised after
 *       RoPE; window KV kept in FP8).
 *   [A] "DeepSeek-V4.1-Flash: pushing KV cache compression to the limit"
 *       (translated abstract) sections 3.3 (CSA2), 3.4 (hierarchical sparse
 *       indexer), 3.6 (FP4 main KV cache).
 *   [S] "DeepSeek-V4 model structure (7): structure decides the system"
 *       (predecessor): attention over the top-k compressed entries plus 128
 *       window entries; K = V single-head MQA on a 512-dim latent.
 *
 * Layer call sequences (one query row per (sequence, query)):
 *   Full     csa2_index_full_select (the scan, the pool of nb blocks and the
 *            top-k entries in one call) -> csa2_sparse_attn.
 *            Step by step: csa2_index_full -> csa2_topk(block maxima, nb) =
 *            pool and csa2_topk(block maxima, k) = top-k blocks ->
 *            csa2_index_pool(own query, top-k blocks) -> csa2_topk(k).
 *   Reindex  csa2_index_pool_topk(own query, Full layer's pool) (or
 *            csa2_index_pool -> csa2_topk(k)) -> csa2_sparse_attn.
 *   Reuse    csa2_sparse_attn with the latest top-k.
 *
 * How the Full layer's top-k is found: the scan keeps no per-entry scores
 * and emits no per-entry candidates; the top-k entries of a row always lie
 * in its k best blocks (a block ranked above a winner's block holds a better
 * entry, also under the lower-index tie-break), so the top-k is selected
 * among those blocks' k * 8 positions, rescored with the scan's own score
 * function (bit-identical scores).  Per-entry candidates from the scan were
 * measured slower on the MI355X than this rescoring.  The scan_start /
 * scan_stop arguments of the fused calls are timing instrumentation (events
 * the scan kernel's dispatch records) and change nothing else.
 *
 * Conventions for every call:
 *   - All tensors are row-major and contiguous, except the indexer-key code
 *     cache (key-tile layout, see csa2_quantize_kv).  Every data pointer is a
 *     DEVICE pointer, allocated and owned by the caller; the library never
 *     allocates, frees or synchronises, and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns.
 *   - Arguments are validated on the host before anything is enqueued; on
 *     any error nothing is enqueued and csa2_last_error() (thread-local)
 *     holds a message.  Device faults surface at the caller's next
 *     synchronisation.  With CSA2_DEBUG_SYNC=1 in the environment every call
 *     synchronises its stream and reports launch/runtime errors.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Supported model dims (CSA2_ERR_UNSUPPORTED otherwise): indexer 32
 *     heads x 128, attention 64 heads x 512, scale group 16, block 8.
 *   - Index inputs that are out of range are skipped (treated as -1), never
 *     dereferenced.
 *   - One kernel launch holds at most 2^32 - 1 work-items (the dispatch
 *     counts its grid in 32 bits).  A call that would need more in any of
 *     its launches fails with CSA2_ERR_UNSUPPORTED before anything is
 *     enqueued.  The limits this sets, by call: csa2_topk about 2^22 rows
 *     (one 1024-thread workgroup per row; fewer for rows whose group maxima
 *     or segments need more threads), as the selects of csa2_index_full_pool;
 *     csa2_index_full_select about 2^21 rows (two such workgroups per row);
 *     the scans rows x ceil(n_cap / 16384)
 *     below 2^24 (decode) or ceil(nq / 8) x ceil(n_cap / 4096) per sequence
 *     (prefill); csa2_sparse_attn below 2^23 query rows.
 *   - The *_workspace queries return 0 for sizes the matching call rejects
 *     (negative sizes, more than 2^24 query rows, k or nb out of range).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape   */
    CSA2_ERR_UNSUPPORTED = 2, /* dims outside the supported set                    */
    CSA2_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace() */
    CSA2_ERR_LAUNCH = 4       /* the HIP runtime refused a launch                  */
} csa2_status;

/* Message of the last failed call on this thread ("" if none). */
const char* csa2_last_error(void);

/* Library ABI version (major * 100 + minor): 107. */
int32_t csa2_version(void);

/*
 * MXFP4 encoder of new cache rows ([N] 2.3, [A] 3.6): rotary (optional) then
 * E2M1 codes with one E4M3FN scale per 16 channels.
 *   x         fp32 [rows, channels], channels % 16 == 0 (512 main KV, 128
 *             indexer key); finite values.
 *   rope_cos, rope_sin  fp32 [rows, rope_dim/2] or NULL when rope_dim == 0.
 *             Row r rotates the pairs (x[rope_offset+2i], x[rope_offset+2i+1])
 *             by (cos[r,i], sin[r,i]): a' = a*c - b*s, b' = a*s + b*c, every
 *             product and sum rounded to fp32 (no fused multiply-add).
 *             rope_offset and rope_dim must be even, rope_offset + rope_dim
 *             <= channels.  Main KV: offset 448, dim 64.
 *   codes     u8 output; row r is written as row d = dst_row + r*dst_stride
 *             of the code array (channel 2j in the low nibble of byte j, 2j+1
 *             in the high one).  channels != 128: row-major, byte j of row d
 *             at codes + d*channels/2 + j.  channels == 128 (indexer keys):
 *             the KEY-TILE LAYOUT of the indexer-key cache, byte j of row d at
 *               codes + (d/32)*2048 + (j/16)*512 + (d%32)*16 + j%16
 *             (tiles of 32 rows, each stored as four 512-byte planes of
 *             16-byte chunks); the array must hold whole tiles.
 *   scales    u8 output, row-major in both cases: row d at scales +
 *             d*channels/16 (byte g scales channels [16g, 16g+16)).
 *   dst_row   >= 0: output row of input row 0.
 *   dst_stride  >= 1: distance in rows between consecutive output rows (1 =
 *             contiguous; n_cap = one new row per sequence of a [B, n_cap]
 *             cache, with dst_row = its position in sequence 0).
 * Encoding per group: scale = E4M3 round-to-nearest-even of max|x|/6,
 * saturating at 448; code = nearest E2M1 value of |x|/scale, ties to the even
 * code, saturating at 6; scale 0 gives code 0; sign only on non-zero codes.
 * Bit-exact, deterministic.
 */
csa2_status csa2_quantize_kv(const float* x, int64_t rows, int32_t channels,
                             const float* rope_cos, const float* rope_sin,
                             int32_t rope_offset, int32_t rope_dim,
                             uint8_t* codes, uint8_t* scales, int64_t dst_row,
                             int64_t dst_stride, void* stream);

/*
 * FP8 encoder of sliding-window KV rows ([N] 2.3: the window KV stays in FP8).
 *   x    fp32 [n] finite values;  out  u8 [n] E4M3FN, round to nearest even,
 *        saturating at +-448, sign kept (a negative value rounding to zero
 *        gives -0).  Elements of row r of a [rows, 512] block go to
 *        out + r*dst_stride*512 when row_len = 512 (row_len divides n).
 */
csa2_status csa2_quantize_swa(const float* x, int64_t n, int32_t row_len, uint8_t* out,
                              int64_t dst_stride, void* stream);

/*
 * New cache entries of one step in one launch ([A] 3.3: a Full layer computes
 * the main KV and projects the indexer key from it; [N] 2.2: indexer K is now
 * projected from the main KV; [N] 2.3: window rows stay FP8).
 *   rows       new compressed entries.
 *   kv_x       fp32 [rows, 512] main latent rows -> rotary (as csa2_quantize_kv,
 *              rope_cos / rope_sin [rows, rope_dim/2]) -> MXFP4 into kv_codes /
 *              kv_scales, row r at cache row d = kv_dst[r] (kv_codes + d*256,
 *              kv_scales + d*32), or d = dst_row + r*kv_stride when kv_dst is
 *              NULL.
 *   kv_dst     int64 [rows] or NULL: per-entry destination rows (each
 *              sequence's own append position: b*n_cap + n_b); rows whose
 *              d is outside [0, kv_cap) are skipped.  The indexer-key row r
 *              goes to the same d.
 *   idx_x      fp32 [rows, 128] indexer-key rows encoded as they are (no
 *              rotary), or NULL: then the keys are projected from the main
 *              latent before its rotary, y = kv_x[r] . w_idx^T with
 *   w_idx      bf16 [128, 512] (row o = output channel o).  Each output
 *              channel is accumulated in fp32: per quarter Q of the 512
 *              channels, four partial sums of fused multiply-adds (channel c
 *              to partial c % 4, in increasing c) added as (p0 + p1) + (p2 + p3);
 *              then the quarters as (Q0 + Q1) + (Q2 + Q3); then encoded.
 *   idx_codes, idx_scales  MXFP4 outputs for row d (d as above, with
 *              idx_stride in place of kv_stride when kv_dst is NULL): codes
 *              in the key-tile layout of csa2_quantize_kv (channels 128),
 *              scales at idx_scales + d*8.  kv_cap counts rows of both
 *              caches; idx_codes must hold ceil(kv_cap/32) tiles of 2048 B.
 *   idx_y      fp32 [rows, 128] receives the projection (NULL: not written;
 *              only used when projecting).
 *   swa_x      fp32 [swa_rows, 512] window rows -> E4M3FN (as
 *              csa2_quantize_swa), row r at swa_out + d*512 with d = swa_dst[r]
 *              (skipped outside [0, swa_cap)) or r*swa_stride; NULL when
 *              swa_rows == 0.  Window ring ([S], state cache: the window
 *              segment of the last 128 tokens is overwritten in place, one per
 *              sequence and layer; [N] 2.4: a miss replays only the last n_win
 *              tokens): token p of sequence b goes to d = b*n_win + p % n_win,
 *              and attention reads the ring with swa_cap = n_win and
 *              swa_end = min(p + 1, n_win) (the joint softmax does not depend
 *              on row order).  Replaying the last n_win tokens of a prompt is
 *              the same call with their rows and ring slots.
 * Reading: the projection takes the latent before rotary (the rotation serves
 * attention positions; the pages say only that the indexer key is projected
 * from the main KV).  The encodings are bit-exact functions of their fp32
 * inputs (the projection itself is fp32 arithmetic).
 */
csa2_status csa2_encode_entries(int32_t rows, const float* kv_x, const float* rope_cos,
                                const float* rope_sin, int32_t rope_offset, int32_t rope_dim,
                                uint8_t* kv_codes, uint8_t* kv_scales, int64_t kv_stride,
                                const int64_t* kv_dst, int64_t dst_row, int64_t kv_cap,
                                const float* idx_x, const uint16_t* w_idx, uint8_t* idx_codes,
                                uint8_t* idx_scales, int64_t idx_stride, float* idx_y,
                                const float* swa_x, int32_t swa_rows, uint8_t* swa_out,
                                int64_t swa_stride, const int64_t* swa_dst, int64_t swa_cap,
                                void* stream);

/*
 * Full-layer indexer scan ([N] 2.2, [A] 3.4: the first Full layer scores the
 * whole causally visible range; a block's score is the largest index score
 * of its positions).
 *   q          bf16 [B, nq, 32, 128] indexer queries.
 *   w          fp32 [B, nq, 32] per-head weights.
 *   k_codes    MXFP4 indexer-key codes of the [B, n_cap] cache in the key-tile
 *              layout (csa2_quantize_kv, channels 128): entry j of sequence b
 *              is row f = b*n_cap + j, in tile f/32; the array holds
 *              ceil(B*n_cap/32) tiles of 2048 B (16-byte aligned).
 *   k_scales   u8 [B, n_cap, 8] row-major scales (shared by every query of a
 *              sequence, like the codes).  n_cap <= 2^30 (CSA2_ERR_INVALID_ARG
 *              above; the calls that gather keys allow 2^24).
 *   n_visible  int32 [B, nq]: query (b, i) sees entries [0, min(n_visible, n_cap)).
 *   block      positions per block (8).
 *   block_max  fp32 [B, nq, ceil(n_cap/block)]: block beta of query (b,i)
 *              receives max over visible j in [beta*block, beta*block+block)
 *              of s_j, for beta < ceil(n_visible/block); later slots are not
 *              written.
 *   scores     fp32 [B, nq, n_cap] or NULL: every s_j, j < n_visible (tests).
 * Score: s_j = sum_h w_h * max(0, q_h . k_j), dot products of the bf16 query
 * with the dequantised key accumulated in fp32 (reading: the pages give the
 * 32 x 128 shape, not the formula; parity unpinned beyond this reading).
 */
csa2_status csa2_index_full(const uint16_t* q, const float* w,
                            const uint8_t* k_codes, const uint8_t* k_scales, int64_t n_cap,
                            const int32_t* n_visible, int32_t B, int32_t nq, int32_t block,
                            float* block_max, float* scores, void* stream);

/*
 * Full-layer scan and pool select in one call ([N] 2.2, [A] 3.4: the Full
 * layer scores the whole visible range and keeps the nb blocks with the
 * largest block scores as the pool).  Same arguments and block_max output as
 * csa2_index_full (no per-entry scores), plus
 *   nb         pool blocks per query row, 1 <= nb <= 8192.
 *   pool       int32 [B, nq, nb]: the chosen block ids in ascending order,
 *              -1 padded -- exactly csa2_topk(block_max, L = ceil(n_cap/8),
 *              rows = B*nq, n_valid = ceil(n_visible/8), k = nb).  With
 *              n_cap == 0 it is all -1 and block_max may be NULL.
 *   ws, ws_bytes  device workspace of at least
 *              csa2_index_full_pool_workspace(n_cap, B*nq, nb) bytes (8-byte
 *              aligned; any contents): the same as that csa2_topk call needs.
 *   scan_start, scan_stop  hipEvent_t (created by the caller) or NULL: the
 *              scan kernel's dispatch records them at its start and end, so
 *              hipEventElapsedTime gives the scan's own duration inside the
 *              call (the benchmark's roofline).  No other effect.
 * When the select groups blocks (rows of more than 16384 blocks) in groups
 * that align with the scan's chunks, the scan writes the group maxima into
 * the workspace itself, which saves the select's pass over the block maxima.
 * Errors as csa2_index_full and csa2_topk (CSA2_ERR_WORKSPACE when ws_bytes
 * is too small).
 */
size_t      csa2_index_full_pool_workspace(int64_t n_cap, int32_t rows, int32_t nb);
csa2_status csa2_index_full_pool(const uint16_t* q, const float* w,
                                 const uint8_t* k_codes, const uint8_t* k_scales, int64_t n_cap,
                                 const int32_t* n_visible, int32_t B, int32_t nq, int32_t block,
                                 int32_t nb, float* block_max, int32_t* pool, void* ws,
                                 size_t ws_bytes, void* scan_start, void* scan_stop,
                                 void* stream);

/*
 * The Full layer's indexer in one call ([N] 2.2, [A] 3.4: the Full layer
 * scores the whole visible range, keeps the nb blocks with the largest block
 * scores as the pool for the Reindex layers, and selects its own top-k
 * entries): scan, pool and top-k.  Same arguments as csa2_index_full_pool,
 * plus
 *   n_cap     at most 2^24 entries per sequence (the rescoring gathers use
 *             32-bit offsets), else CSA2_ERR_UNSUPPORTED.
 *   nb        pool blocks, 0 <= nb <= 8192 (0: no pool, pool may be NULL).
 *   k         1 <= k <= 8192.
 *   pool      int32 [B, nq, nb]: csa2_topk(block_max, ceil(n_cap/8), B*nq,
 *             n_valid = ceil(n_visible/8), nb), bit for bit.
 *   topk      int32 [B, nq, k]: the Full layer's top-k positions, ascending,
 *             -1 padded: the k best visible entries under (score descending,
 *             position ascending), exactly what csa2_topk over every score
 *             of csa2_index_full would select.
 *   ws, ws_bytes  device workspace of csa2_index_full_select_workspace(n_cap,
 *             B, nq, nb, k) bytes, 256-byte aligned, any contents.
 * The scan writes only block maxima (and, for long rows, candidate lists), no
 * per-entry scores.  The top-k entries of a row lie in its k best blocks (a
 * block ranked above a winner's block holds a better entry, also under the
 * lower-index tie-break), so the call selects the pool and the k best blocks
 * (for rows of more than 16384 blocks among the scan's per-chunk candidates
 * -- each chunk's best blocks -- with an exact fallback over group maxima
 * that the scan also writes, for a row where a chunk could hold more winners
 * than it listed), then rescores the k best blocks' k * 8 positions with the
 * scan's own score function (bit-identical scores) and keeps the best k.
 * Every path gives the same result.
 */
size_t      csa2_index_full_select_workspace(int64_t n_cap, int32_t B, int32_t nq, int32_t nb,
                                             int32_t k);
csa2_status csa2_index_full_select(const uint16_t* q, const float* w,
                                   const uint8_t* k_codes, const uint8_t* k_scales,
                                   int64_t n_cap, const int32_t* n_visible, int32_t B,
                                   int32_t nq, int32_t block, int32_t nb, int32_t k,
                                   float* block_max, int32_t* pool, int32_t* topk,
                                   void* ws, size_t ws_bytes, void* scan_start,
                                   void* scan_stop, void* stream);

/*
 * Indexer scoring restricted to a pool of blocks ([N] 2.2, [A] 3.4: Reindex
 * layers score only the Full layer's 2048 x 8 pool with their own query).
 *   q, w, k_codes, k_scales, n_visible, B, nq: as csa2_index_full.
 *   n_cap      as csa2_index_full, at most 2^24 (the gathers use 32-bit
 *              offsets), else CSA2_ERR_UNSUPPORTED.
 *   blocks     int32 [B, nq, n_blocks]: block ids (ascending, -1 padding).
 *   pool_score fp32 [B, nq, n_blocks*block]: slot t*block + r holds the score
 *              of position blocks[t]*block + r, or -inf if that position is
 *              not visible or the block is -1.
 *   pool_idx   int32 [B, nq, n_blocks*block]: the position, or -1.
 * Scores are bit-identical to csa2_index_full's for the same entry and query.
 */
csa2_status csa2_index_pool(const uint16_t* q, const float* w,
                            const uint8_t* k_codes, const uint8_t* k_scales, int64_t n_cap,
                            const int32_t* blocks, int32_t n_blocks, int32_t block,
                            const int32_t* n_visible, int32_t B, int32_t nq,
                            float* pool_score, int32_t* pool_idx, void* stream);

/*
 * Pool rescoring and its top-k in one call ([N] 2.2, [A] 3.4: Reindex layers
 * score only the pool with their own query and keep its top-k; the Full layer
 * does the same over its top-k blocks).  Exactly csa2_index_pool followed by
 * csa2_topk(pool_score, k, idx = pool_idx) into topk [B, nq, k] (ascending
 * positions, -1 padded), bit for bit, without the per-slot scores as an
 * output.  Arguments as csa2_index_pool, plus
 *   n_blocks   0 <= n_blocks <= 2048 (at most 16384 rescored positions).
 *   k          1 <= k <= 8192.
 *   ws, ws_bytes  device workspace of csa2_index_pool_topk_workspace(B, nq,
 *              n_blocks) bytes, 256-byte aligned.  Its first bytes are one
 *              arrival counter per query row: the workspace must be
 *              zero-filled once before its first use (e.g. when it is
 *              allocated); every call leaves the counters zero again, so the
 *              same workspace serves any later call.  Calls that share a
 *              workspace must not overlap in time.
 * One launch: every workgroup scores its slots and stores them to the
 * workspace; the last workgroup of a row to finish selects the row's top-k.
 */
size_t      csa2_index_pool_topk_workspace(int32_t B, int32_t nq, int32_t n_blocks);
csa2_status csa2_index_pool_topk(const uint16_t* q, const float* w, const uint8_t* k_codes,
                                 const uint8_t* k_scales, int64_t n_cap, const int32_t* blocks,
                                 int32_t n_blocks, int32_t block, const int32_t* n_visible,
                                 int32_t B, int32_t nq, int32_t k, int32_t* topk, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Top-k select ([N] 1: top-k 512; [N] 2.2 / [A] 3.4: top-2048 blocks).
 *   score    fp32 [rows, L].
 *   idx      int32 [rows, L] or NULL (= 0..L-1).  Entries with idx < 0, NaN
 *            score, or position >= n_valid[row] are skipped.  Among valid
 *            entries idx must ascend with position (true of csa2_index_pool's
 *            output and of identity indices).
 *   n_valid  int32 [rows] or NULL (= L): valid prefix of each row.
 *   k        1 <= k <= 8192.
 *   out      int32 [rows, k]: the k best under (score descending, index
 *            ascending), -0 equal to +0, written as ascending indices, -1
 *            padding when fewer than k are valid.  Bit-exact, deterministic.
 *   ws       device workspace of csa2_topk_workspace(L, rows, k) bytes (0 for
 *            L <= 16384, where ws may be NULL).
 */
csa2_status csa2_topk(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                      const int32_t* n_valid, int32_t k, int32_t* out,
                      void* ws, size_t ws_bytes, void* stream);
size_t csa2_topk_workspace(int64_t L, int32_t rows, int32_t k);

/*
 * csa2_topk without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * allocation).  Same arguments, selection and output as csa2_topk; the
 * workspace csa2_topk_workspace(L, rows, k) would need comes instead from a
 * static device array of the library (8 MiB per GPU, allocated when the
 * library is loaded and held until the process ends), whose device address
 * is looked up once per GPU on the first call made with that GPU current.
 * Calls whose workspace would exceed 8 MiB fail with CSA2_ERR_WORKSPACE
 * (nothing enqueued).  The call itself allocates nothing.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be ordered by the caller.  No part
 * of the array needs clearing between calls.
 */
csa2_status csa2_topk_noalloc(const float* score, const int32_t* idx, int64_t L, int32_t rows,
                              const int32_t* n_valid, int32_t k, int32_t* out, void* stream);

/*
 * Sparse MLA attention ([N] 1: 64 heads x 512; [S]: K = V single-head MQA on
 * the 512-dim latent, top-k compressed entries plus 128 window entries).
 *   q          bf16 [B, nq, 64, 512], 16-byte aligned.
 *   kv_codes   u8 [B, n_cap, 256], kv_scales u8 [B, n_cap, 32]: MXFP4 main KV
 *              (NULL allowed when n_cap == 0: no compressed entries yet);
 *              n_cap <= 2^24, else CSA2_ERR_UNSUPPORTED.
 *   topk       int32 [B, nq, k]: entry ids; ids outside [0, n_cap) skipped.
 *   swa        u8 [B, swa_cap, 512] E4M3FN window rows, swa_cap <= 2^22; query
 *              (b, i) uses rows [max(0, swa_end[b,i] - n_win),
 *              min(swa_end[b,i], swa_cap)).
 *   softmax_scale  multiplies q . v before the softmax.
 *   out        fp32 [B, nq, 64, 512], 16-byte aligned: o_h = sum_j p_j v_j, p = softmax over the
 *              union of selected entries and window rows (one joint softmax);
 *              0 for an empty key set.
 *   lse        fp32 [B, nq, 64] or NULL: ln sum_j exp(l_j) (-inf if empty).
 *   ws         device workspace, 16-byte aligned, contents arbitrary, or NULL.
 *              With csa2_sparse_attn_workspace(B, nq, k, n_win) bytes (non-zero
 *              only for few query rows) each row's keys are split over several
 *              workgroups whose partial results are merged by a second launch;
 *              with NULL or fewer bytes the call still completes, with one
 *              workgroup per (row, group of heads) over every key.  Each form
 *              is deterministic; the forms differ only in fp32 rounding order.
 * Dequantisation is exact in fp16; products accumulate in fp32.
 */
csa2_status csa2_sparse_attn(const uint16_t* q, int32_t B, int32_t nq,
                             const uint8_t* kv_codes, const uint8_t* kv_scales, int64_t n_cap,
                             const int32_t* topk, int32_t k,
                             const uint8_t* swa, int32_t swa_cap, const int32_t* swa_end,
                             int32_t n_win, float softmax_scale, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);
size_t csa2_sparse_attn_workspace(int32_t B, int32_t nq, int32_t k, int32_t n_win);

/*
 * Sparse MLA attention with the output epilogue of the deployment kernel
 * ([S] "DeepSeek-V4 model structure (7)", sequence dimension: the output is
 * rotated back to restore relative position; [N] 4, inference side: the
 * fused RoPE-attention-RoPE-cast kernel).  Same inputs and attention as
 * csa2_sparse_attn; then, per query row r and head, each pair of output
 * channels (a, b) = (o[off+2i], o[off+2i+1]), i < rope_dim/2, is rotated by
 * minus the query position's angle:
 *     a' = a*c + b*s,  b' = b*c - a*s   (c = rope_cos[r, i], s = rope_sin[r, i],
 *                                        every product and sum rounded to fp32)
 * and every channel is cast to bf16 (round to nearest even).
 *   rope_cos, rope_sin  fp32 [B*nq, rope_dim/2]: the query's own position
 *              (the table the query's rotary part was built with); NULL when
 *              rope_dim == 0.  rope_offset, rope_dim even, offset + dim <= 512
 *              (main latent: 448, 64).
 *   out        bf16 [B, nq, 64, 512] as uint16_t bit patterns, 8-byte aligned.
 *   lse        as csa2_sparse_attn (natural log of the softmax denominator,
 *              the statistic a split-KV combine needs), or NULL.
 */
csa2_status csa2_sparse_attn_rope_bf16(const uint16_t* q, int32_t B, int32_t nq,
                                       const uint8_t* kv_codes, const uint8_t* kv_scales,
                                       int64_t n_cap, const int32_t* topk, int32_t k,
                                       const uint8_t* swa, int32_t swa_cap,
                                       const int32_t* swa_end, int32_t n_win,
                                       float softmax_scale, const float* rope_cos,
                                       const float* rope_sin, int32_t rope_offset,
                                       int32_t rope_dim, uint16_t* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream);

/*
 * Streaming-read calibration (measurement only, no part of a layer): reads
 * `bytes` bytes at `src` (16-byte aligned, bytes % 16 == 0) once with
 * 16-byte loads, `workgroups` workgroups each taking one contiguous slice,
 * `depth` loads per lane in flight (1, 2, 4 or 8).  sink: uint32
 * [workgroups], written only when a workgroup's checksum equals one fixed
 * value (the reads cannot be optimised away; in practice nothing is
 * written).  The fastest setting is the practical read ceiling that the
 * indexer scan's bandwidth is compared with.
 */
csa2_status csa2_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t depth,
                             uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
