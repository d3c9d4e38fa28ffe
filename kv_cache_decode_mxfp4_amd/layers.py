"""CSA2 layer call sequences on top of the C ABI (one GPU, caller's stream).

The three layer modes of the DeepSeek-V4.1 pages ([N] 2.2 of the reading
notes, [A] 3.3-3.4 of the translated abstract):

  Full     scores the whole visible range, selects the pool of `nb` blocks of
           8 (ranked by their largest score) and its own top-k;
  Reindex  rescores only the Full layer's pool with its own indexer query and
           selects its own top-k;
  Reuse    runs attention with the latest top-k.

How the Full layer's top-k is found: its top-k entries always lie in its
top-k blocks (a block ranked above a winner's block holds another winner,
also under the lower-index tie-break), so the scan keeps no per-entry
scores: one call (csa2_index_full_select) scans, selects the pool (top-nb
blocks) and finds the winners among the top-k blocks' positions (from the
scan's per-chunk candidates on long rows, else by rescoring those k * 8
positions).  Every step is a libcsa2 kernel; this module only sequences
calls and owns reusable buffers.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib

BLOCK = 8
FUSED_MAX_BLOCKS = 2048  # csa2_index_pool_topk rescores at most 16384 positions per row
# Beyond about 32 rows x 4096 rescored positions the pool scan (more key gathers in
# flight) and csa2_topk beat the one-launch rescoring + top-k: measured on the MI355X,
# 16 x 4096 positions 14.2 vs 18.2 us, 64 x 4096 26.1 vs 18.3 us, 128 x 16384 139.4 vs
# 58.5 us (the same choice as inside csa2_index_full_select).
FUSED_MAX_POSITIONS = 32 * 4096


def n_valid_blocks(n_visible: torch.Tensor) -> torch.Tensor:
    """Visible blocks per query row, ceil(n_visible / 8), on n_visible's device.

    Host-side input preparation (like n_visible itself), done once per shape."""
    host = ((n_visible.to("cpu").to(torch.int64) + BLOCK - 1) // BLOCK).to(torch.int32)
    return host.to(n_visible.device)


@dataclass
class Buffers:
    """Device buffers reused across steps for one (B, nq, n_cap, k, nb) shape."""
    block_max: torch.Tensor
    pool: torch.Tensor | None
    sel_blocks: torch.Tensor
    pool_score: torch.Tensor
    pool_idx: torch.Tensor
    topk: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    ws_topk: torch.Tensor | None
    ws_attn: torch.Tensor | None
    ws_sel: torch.Tensor | None
    ws_pool_topk: torch.Tensor

    @staticmethod
    def create(B: int, nq: int, n_cap: int, k: int, nb: int, n_win: int,
               device="cuda") -> "Buffers":
        f32, i32 = torch.float32, torch.int32
        nblk = (n_cap + BLOCK - 1) // BLOCK
        pool = torch.empty(B, nq, nb, dtype=i32, device=device) if nb > 0 else None
        nsel = max(nb, k)
        sel = torch.empty(B, nq, k, dtype=i32, device=device)  # the top-k blocks
        ws_t = max(_lib.topk_workspace(nblk, B * nq, nsel), _lib.topk_workspace(nsel * BLOCK, B * nq, k),
                   _lib.topk_workspace(nblk, B * nq, k))
        ws_a = _lib.sparse_attn_workspace(B, nq, k, n_win)
        ws_s = _lib.index_full_select_workspace(n_cap, B, nq, nb, k)
        # arrival counters of the fused pool rescoring + top-k: zeroed once here
        # (sized for the largest pool that takes the fused path at this row count)
        fused_blocks = min(nsel, FUSED_MAX_BLOCKS, FUSED_MAX_POSITIONS // max(B * nq * BLOCK, 1))
        ws_pt = _lib.index_pool_topk_workspace(B, nq, fused_blocks)
        return Buffers(
            block_max=torch.empty(B, nq, nblk, dtype=f32, device=device),
            pool=pool,
            sel_blocks=sel,
            pool_score=torch.empty(B, nq, nsel * BLOCK, dtype=f32, device=device),
            pool_idx=torch.empty(B, nq, nsel * BLOCK, dtype=i32, device=device),
            topk=torch.empty(B, nq, k, dtype=i32, device=device),
            out=torch.empty(B, nq, 64, 512, dtype=f32, device=device),
            lse=torch.empty(B, nq, 64, dtype=f32, device=device),
            ws_topk=torch.empty(ws_t, dtype=torch.uint8, device=device) if ws_t else None,
            ws_attn=torch.empty(ws_a, dtype=torch.uint8, device=device) if ws_a else None,
            ws_sel=torch.empty(ws_s, dtype=torch.uint8, device=device) if ws_s else None,
            ws_pool_topk=torch.zeros(ws_pt, dtype=torch.uint8, device=device),
        )


def select_blocks(buf: Buffers, n_blocks_valid: torch.Tensor, k: int, nb: int, stream=None):
    """Pool (top-nb blocks) and the top-k blocks that hold the top-k entries, as two
    csa2_topk calls over the block maxima."""
    if nb > 0:
        _lib.topk(buf.block_max, nb, buf.pool, n_valid=n_blocks_valid, ws=buf.ws_topk,
                  stream=stream)
    _lib.topk(buf.block_max, k, buf.sel_blocks, n_valid=n_blocks_valid, ws=buf.ws_topk,
              stream=stream)


def full_indexer(buf: Buffers, q_idx, w_idx, k_codes, k_scales, n_visible, n_blocks_valid,
                 k: int, nb: int, scores=None, stream=None, scan_events=None):
    """Full layer indexer: block scan, pool, top-k.  Leaves buf.pool and buf.topk.

    One library call (csa2_index_full_select); with per-entry scores asked for
    (tests), the scan, two csa2_topk calls over the block maxima and the top-k
    blocks' rescoring instead."""
    if scores is None:
        _lib.index_full_select(q_idx, w_idx, k_codes, k_scales, n_visible, buf.block_max,
                               buf.topk, pool=buf.pool, ws=buf.ws_sel, stream=stream,
                               scan_events=scan_events)
        return
    _lib.index_full(q_idx, w_idx, k_codes, k_scales, n_visible, buf.block_max, scores=scores,
                    stream=stream)
    select_blocks(buf, n_blocks_valid, k, nb, stream=stream)
    _pool_topk(buf, q_idx, w_idx, k_codes, k_scales, n_visible, buf.sel_blocks, k, stream)


def _pool_topk(buf: Buffers, q_idx, w_idx, k_codes, k_scales, n_visible, blocks, k: int,
               stream=None):
    """Rescore the positions of `blocks` with this query and select the top-k into buf.topk:
    one fused call for few rescored positions, else the pool scan and csa2_topk."""
    B, nq, nbk = blocks.shape
    if nbk <= FUSED_MAX_BLOCKS and B * nq * nbk * BLOCK <= FUSED_MAX_POSITIONS:
        _lib.index_pool_topk(q_idx, w_idx, k_codes, k_scales, blocks, n_visible, buf.topk,
                             buf.ws_pool_topk, stream=stream)
        return
    score = _slots(buf.pool_score, B, nq, nbk * BLOCK)
    idx = _slots(buf.pool_idx, B, nq, nbk * BLOCK)
    _lib.index_pool(q_idx, w_idx, k_codes, k_scales, blocks, n_visible, score, idx, stream=stream)
    _lib.topk(score, k, buf.topk, idx=idx, ws=buf.ws_topk, stream=stream)


def _slots(t: torch.Tensor, B: int, nq: int, L: int) -> torch.Tensor:
    """Contiguous [B, nq, L] view of the front of a larger buffer."""
    return t.view(-1)[: B * nq * L].view(B, nq, L)


def reindex_indexer(buf: Buffers, q_idx, w_idx, k_codes, k_scales, n_visible, pool, k: int,
                    stream=None):
    """Reindex layer indexer: score the given pool with this layer's query, top-k."""
    _pool_topk(buf, q_idx, w_idx, k_codes, k_scales, n_visible, pool, k, stream)


def attention(buf: Buffers, q, kv_codes, kv_scales, topk, swa, swa_end, n_win: int = 128,
              scale: float = 1.0, stream=None, out_bf16=None, rope_cos=None, rope_sin=None):
    """Sparse MLA attention of one layer (every mode ends with it).  With out_bf16 (and the
    query rows' rope_cos / rope_sin) the output is rotated back and cast to bf16 there
    instead of written as fp32 to buf.out."""
    if out_bf16 is None:
        _lib.sparse_attn(q, kv_codes, kv_scales, topk, swa, swa_end, buf.out, buf.lse,
                         n_win=n_win, softmax_scale=scale, ws=buf.ws_attn, stream=stream)
    else:
        _lib.sparse_attn_rope_bf16(q, kv_codes, kv_scales, topk, swa, swa_end, rope_cos, rope_sin,
                                   out_bf16, buf.lse, n_win=n_win, softmax_scale=scale,
                                   ws=buf.ws_attn, stream=stream)
