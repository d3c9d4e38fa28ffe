"""ctypes binding of libcsa2.so: argument marshalling only.

Each function takes torch tensors that live on the GPU, checks every tensor's
dtype and element count against the shape include/csa2.h documents for it
(inputs and outputs alike, before any pointer is taken), then device and
contiguity, and forwards raw pointers to the C entry point of the same name on
the current torch stream.  An undersized tensor raises here, so the library
never writes past a buffer it was handed.  All computation happens in the
library's HIP kernels; a missing library raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

CSA2_OK = 0
STATUS = {0: "CSA2_OK", 1: "CSA2_ERR_INVALID_ARG", 2: "CSA2_ERR_UNSUPPORTED",
          3: "CSA2_ERR_WORKSPACE", 4: "CSA2_ERR_LAUNCH"}

EXPORTS = ("csa2_last_error", "csa2_version", "csa2_quantize_kv", "csa2_quantize_swa",
           "csa2_index_full", "csa2_index_full_pool", "csa2_index_full_pool_workspace",
           "csa2_index_pool", "csa2_topk", "csa2_topk_workspace",
           "csa2_sparse_attn", "csa2_sparse_attn_workspace", "csa2_sparse_attn_rope_bf16",
           "csa2_encode_entries", "csa2_topk_noalloc", "csa2_stream_read",
           "csa2_index_full_select", "csa2_index_full_select_workspace",
           "csa2_index_pool_topk", "csa2_index_pool_topk_workspace")


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m kv_cache_decode_mxfp4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                             ctypes.c_size_t)
    st = ctypes.c_int
    L.csa2_last_error.restype = ctypes.c_char_p
    L.csa2_last_error.argtypes = []
    L.csa2_version.restype = i32
    L.csa2_version.argtypes = []
    L.csa2_quantize_kv.restype = st
    L.csa2_quantize_kv.argtypes = [vp, i64, i32, vp, vp, i32, i32, vp, vp, i64, i64, vp]
    L.csa2_quantize_swa.restype = st
    L.csa2_quantize_swa.argtypes = [vp, i64, i32, vp, i64, vp]
    L.csa2_index_full.restype = st
    L.csa2_index_full.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, i32, vp, vp, vp]
    L.csa2_index_full_pool.restype = st
    L.csa2_index_full_pool.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, vp, vp, vp, sz,
                                       vp, vp, vp]
    L.csa2_index_full_pool_workspace.restype = sz
    L.csa2_index_full_pool_workspace.argtypes = [i64, i32, i32]
    L.csa2_index_full_select.restype = st
    L.csa2_index_full_select.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp,
                                         vp, vp, sz, vp, vp, vp]
    L.csa2_index_full_select_workspace.restype = sz
    L.csa2_index_full_select_workspace.argtypes = [i64, i32, i32, i32, i32]
    L.csa2_index_pool_topk.restype = st
    L.csa2_index_pool_topk.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, vp, i32, i32, i32, vp,
                                       vp, sz, vp]
    L.csa2_index_pool_topk_workspace.restype = sz
    L.csa2_index_pool_topk_workspace.argtypes = [i32, i32, i32]
    L.csa2_index_pool.restype = st
    L.csa2_index_pool.argtypes = [vp, vp, vp, vp, i64, vp, i32, i32, vp, i32, i32, vp, vp, vp]
    L.csa2_topk.restype = st
    L.csa2_topk.argtypes = [vp, vp, i64, i32, vp, i32, vp, vp, sz, vp]
    L.csa2_topk_noalloc.restype = st
    L.csa2_topk_noalloc.argtypes = [vp, vp, i64, i32, vp, i32, vp, vp]
    L.csa2_stream_read.restype = st
    L.csa2_stream_read.argtypes = [vp, i64, i32, i32, vp, vp]
    L.csa2_topk_workspace.restype = sz
    L.csa2_topk_workspace.argtypes = [i64, i32, i32]
    L.csa2_sparse_attn.restype = st
    L.csa2_sparse_attn.argtypes = [vp, i32, i32, vp, vp, i64, vp, i32, vp, i32, vp, i32, f32,
                                   vp, vp, vp, sz, vp]
    L.csa2_sparse_attn_workspace.restype = sz
    L.csa2_sparse_attn_workspace.argtypes = [i32, i32, i32, i32]
    L.csa2_encode_entries.restype = st
    L.csa2_encode_entries.argtypes = [i32, vp, vp, vp, i32, i32, vp, vp, i64, vp, i64, i64, vp,
                                      vp, vp, vp, i64, vp, vp, i32, vp, i64, vp, i64, vp]
    L.csa2_sparse_attn_rope_bf16.restype = st
    L.csa2_sparse_attn_rope_bf16.argtypes = [vp, i32, i32, vp, vp, i64, vp, i32, vp, i32, vp, i32,
                                             f32, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != CSA2_OK:
        raise Csa2Error(fn, status, load().csa2_last_error().decode())


def _p(t):
    """Device pointer of a CUDA/HIP tensor (None for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _dt(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


_BF16 = (torch.bfloat16, torch.uint16, torch.int16)


def _need(t, dtype, numel, name, optional=False):
    """t must have the dtype (a tuple: any of them) and at least `numel` elements."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
    if not ok:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")


def _bf16_bits(t):
    """bf16 tensors are passed as their bit patterns (uint16 or int16 views accepted)."""
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.uint16, torch.int16):
        return t
    raise TypeError(f"expected bfloat16 (or its uint16 bits), got {t.dtype}")


KEY_TILE = 32            # entries per tile of the indexer-key code cache
KEY_TILE_BYTES = 2048    # 32 entries x 64 code bytes


def key_code_bytes(rows: int) -> int:
    """Bytes of an indexer-key code array holding `rows` entries (whole tiles of 32).

    Layout (include/csa2.h, csa2_quantize_kv with 128 channels): byte j of entry f at
    (f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16."""
    return -(-rows // KEY_TILE) * KEY_TILE_BYTES


def key_codes_empty(rows: int, device="cuda") -> torch.Tensor:
    """Uninitialised indexer-key code array for `rows` entries ([tiles, 2048] uint8)."""
    return torch.empty(key_code_bytes(rows) // KEY_TILE_BYTES, KEY_TILE_BYTES, dtype=torch.uint8,
                       device=device)


def _rows_fit(t, row_bytes, dst_row, dst_stride, rows, name, tiled=False):
    last = dst_row + (rows - 1) * dst_stride + 1 if rows else 0
    need = key_code_bytes(last) if tiled else last * row_bytes
    if dst_row < 0 or need > t.numel():
        raise ValueError(f"{name}: rows do not fit the destination")


def quantize_kv(x, codes, scales, rope_cos=None, rope_sin=None, rope_offset=0, rope_dim=0,
                dst_row=0, dst_stride=1, stream=None):
    """Encode x [rows, C] into rows dst_row + r*dst_stride of the flat code/scale caches
    (C = 128: codes in the key-tile layout of the indexer-key cache)."""
    _dt(x, torch.float32, "x")
    _dt(codes, torch.uint8, "codes")
    _dt(scales, torch.uint8, "scales")
    rows, C = x.shape
    _rows_fit(codes, C // 2, dst_row, dst_stride, rows, "codes", tiled=(C == 128))
    _rows_fit(scales, C // 16, dst_row, dst_stride, rows, "scales")
    _need(rope_cos, torch.float32, rows * (rope_dim // 2), "rope_cos", optional=rope_dim == 0)
    _need(rope_sin, torch.float32, rows * (rope_dim // 2), "rope_sin", optional=rope_dim == 0)
    _check("csa2_quantize_kv", load().csa2_quantize_kv(
        _p(x), rows, C, _p(rope_cos), _p(rope_sin), rope_offset, rope_dim,
        _p(codes), _p(scales), dst_row, dst_stride, _stream(stream)))


def quantize_swa(x, out, row_len=512, dst_row=0, dst_stride=1, stream=None):
    """Encode x [rows, row_len] into rows dst_row + r*dst_stride of the flat window buffer."""
    _dt(x, torch.float32, "x")
    _dt(out, torch.uint8, "out")
    rows = x.numel() // row_len
    _rows_fit(out, row_len, dst_row, dst_stride, rows, "out")
    _check("csa2_quantize_swa", load().csa2_quantize_swa(
        _p(x), x.numel(), row_len, _p(out) + dst_row * row_len, dst_stride, _stream(stream)))


def encode_entries(kv_x, kv_codes, kv_scales, idx_codes, idx_scales, idx_x=None, w_idx=None,
                   rope_cos=None, rope_sin=None, rope_offset=0, rope_dim=0, dst_row=0, dst_stride=1,
                   kv_dst=None, idx_y=None, swa_x=None, swa_out=None, swa_row=0, swa_stride=1,
                   swa_dst=None, stream=None):
    """One launch for a step's new entries: main-KV rows kv_x [rows, 512] and indexer-key
    rows (idx_x [rows, 128], or projected from kv_x by w_idx bf16 [128, 512]) into rows
    dst_row + r*dst_stride of the flat caches (or rows kv_dst[r], int64); window rows
    swa_x [n, 512] into rows swa_row + r*swa_stride of swa_out (or rows swa_dst[r], e.g.
    ring slots)."""
    _dt(kv_x, torch.float32, "kv_x")
    rows = kv_x.shape[0]
    for t_, n_, rb in ((kv_codes, "kv_codes", 256), (kv_scales, "kv_scales", 32),
                       (idx_codes, "idx_codes", 64), (idx_scales, "idx_scales", 8)):
        _dt(t_, torch.uint8, n_)
        if kv_dst is None:
            _rows_fit(t_, rb, dst_row, dst_stride, rows, n_, tiled=(n_ == "idx_codes"))
    kv_cap = min(kv_codes.numel() // 256, kv_scales.numel() // 32,
                 idx_codes.numel() // KEY_TILE_BYTES * KEY_TILE, idx_scales.numel() // 8)
    if kv_dst is not None:
        _need(kv_dst, torch.int64, rows, "kv_dst")
        dst_row = 0
    _need(kv_x, torch.float32, rows * 512, "kv_x")
    _need(rope_cos, torch.float32, rows * (rope_dim // 2), "rope_cos", optional=rope_dim == 0)
    _need(rope_sin, torch.float32, rows * (rope_dim // 2), "rope_sin", optional=rope_dim == 0)
    _need(idx_x, torch.float32, rows * 128, "idx_x", optional=True)
    _need(w_idx, _BF16, 128 * 512, "w_idx", optional=True)
    _need(idx_y, torch.float32, rows * 128, "idx_y", optional=True)
    if w_idx is not None:
        w_idx = _bf16_bits(w_idx)
    n_sw = 0
    if swa_x is not None:
        _dt(swa_x, torch.float32, "swa_x")
        _dt(swa_out, torch.uint8, "swa_out")
        n_sw = swa_x.shape[0]
        _need(swa_x, torch.float32, n_sw * 512, "swa_x")
        if swa_dst is None:
            _rows_fit(swa_out, 512, swa_row, swa_stride, n_sw, "swa_out")
        else:
            _need(swa_dst, torch.int64, n_sw, "swa_dst")
            swa_row = 0
    swa_cap = swa_out.numel() // 512 if swa_out is not None else 0
    _check("csa2_encode_entries", load().csa2_encode_entries(
        rows, _p(kv_x), _p(rope_cos), _p(rope_sin), rope_offset, rope_dim,
        _p(kv_codes), _p(kv_scales), dst_stride, _p(kv_dst), dst_row,
        kv_cap, _p(idx_x), _p(w_idx), _p(idx_codes),
        _p(idx_scales), dst_stride, _p(idx_y), _p(swa_x), n_sw,
        (_p(swa_out) + swa_row * 512) if swa_out is not None else None, swa_stride,
        _p(swa_dst), swa_cap, _stream(stream)))


def _key_cache_rows(k_codes, k_scales, B) -> int:
    """n_cap of a [B, n_cap] indexer-key cache: scales [B, n_cap, 8] row-major, codes in
    whole key tiles for the B * n_cap entries."""
    _dt(k_codes, torch.uint8, "k_codes")
    _dt(k_scales, torch.uint8, "k_scales")
    if k_scales.dim() != 3 or k_scales.shape[0] != B or k_scales.shape[2] != 8:
        raise ValueError(f"k_scales: expected [{B}, n_cap, 8], got {tuple(k_scales.shape)}")
    n_cap = k_scales.shape[1]
    if k_codes.numel() < key_code_bytes(B * n_cap):
        raise ValueError(f"k_codes: {k_codes.numel()} bytes cannot hold {B * n_cap} key entries")
    return n_cap


def _indexer_inputs(q, w, k_codes, k_scales, n_visible):
    """(B, nq, n_cap) of an indexer call after checking q [B, nq, 32, 128] bf16, w
    [B, nq, 32] fp32, n_visible [B, nq] int32 and the key cache."""
    if q.dim() != 4 or q.shape[2:] != (32, 128):
        raise ValueError(f"q: expected [B, nq, 32, 128], got {tuple(q.shape)}")
    B, nq = q.shape[0], q.shape[1]
    _need(q, _BF16, B * nq * 4096, "q")
    _need(w, torch.float32, B * nq * 32, "w")
    _need(n_visible, torch.int32, B * nq, "n_visible")
    return B, nq, _key_cache_rows(k_codes, k_scales, B)


def index_full(q, w, k_codes, k_scales, n_visible, block_max, scores=None, block=8, stream=None):
    B, nq, n_cap = _indexer_inputs(q, w, k_codes, k_scales, n_visible)
    _need(block_max, torch.float32, B * nq * (-(-n_cap // 8)), "block_max", optional=n_cap == 0)
    _need(scores, torch.float32, B * nq * n_cap, "scores", optional=True)
    q = _bf16_bits(q)
    _check("csa2_index_full", load().csa2_index_full(
        _p(q), _p(w), _p(k_codes), _p(k_scales), n_cap, _p(n_visible), B, nq, block,
        _p(block_max), _p(scores), _stream(stream)))


def index_full_pool_workspace(n_cap, rows, nb) -> int:
    return int(load().csa2_index_full_pool_workspace(n_cap, rows, nb))


def index_full_pool(q, w, k_codes, k_scales, n_visible, block_max, pool, ws=None, block=8,
                    scan_events=None, stream=None):
    """Full-layer scan and pool select in one call: block_max as index_full, pool [B, nq, nb]
    = the nb best blocks in ascending order (what topk over block_max returns).
    scan_events: optional (start, stop) torch.cuda.Event pair (timing enabled, already
    created by one record) that the scan kernel's dispatch records."""
    B, nq, n_cap = _indexer_inputs(q, w, k_codes, k_scales, n_visible)
    nb = pool.shape[-1]
    _need(pool, torch.int32, B * nq * nb, "pool")
    _need(block_max, torch.float32, B * nq * (-(-n_cap // 8)), "block_max", optional=n_cap == 0)
    _need(ws, torch.uint8, 0, "ws", optional=True)
    q = _bf16_bits(q)
    _check("csa2_index_full_pool", load().csa2_index_full_pool(
        _p(q), _p(w), _p(k_codes), _p(k_scales), n_cap, _p(n_visible), B, nq, block, nb,
        _p(block_max), _p(pool), _p(ws), ws.numel() if ws is not None else 0,
        scan_events[0].cuda_event if scan_events else None,
        scan_events[1].cuda_event if scan_events else None, _stream(stream)))


def index_full_select_workspace(n_cap, B, nq, nb, k) -> int:
    return int(load().csa2_index_full_select_workspace(n_cap, B, nq, nb, k))


def index_full_select(q, w, k_codes, k_scales, n_visible, block_max, topk, pool=None,
                      ws=None, block=8, scan_events=None, stream=None):
    """The Full layer's indexer in one call: the scan, the pool (top-nb blocks,
    nb = pool.shape[-1], or none) and the top-k positions (k = topk.shape[-1]); ws:
    uint8 device workspace of index_full_select_workspace(...) bytes, 256-byte aligned."""
    B, nq, n_cap = _indexer_inputs(q, w, k_codes, k_scales, n_visible)
    nb = pool.shape[-1] if pool is not None else 0
    k = topk.shape[-1]
    _need(topk, torch.int32, B * nq * k, "topk")
    _need(pool, torch.int32, B * nq * nb, "pool", optional=True)
    _need(block_max, torch.float32, B * nq * (-(-n_cap // 8)), "block_max", optional=n_cap == 0)
    _need(ws, torch.uint8, 0, "ws", optional=True)
    q = _bf16_bits(q)
    _check("csa2_index_full_select", load().csa2_index_full_select(
        _p(q), _p(w), _p(k_codes), _p(k_scales), n_cap, _p(n_visible), B, nq, block, nb, k,
        _p(block_max), _p(pool), _p(topk), _p(ws),
        ws.numel() * ws.element_size() if ws is not None else 0,
        scan_events[0].cuda_event if scan_events else None,
        scan_events[1].cuda_event if scan_events else None, _stream(stream)))


def index_pool(q, w, k_codes, k_scales, blocks, n_visible, pool_score, pool_idx, block=8,
               stream=None):
    B, nq, n_cap = _indexer_inputs(q, w, k_codes, k_scales, n_visible)
    nbk = blocks.shape[-1]
    _need(blocks, torch.int32, B * nq * nbk, "blocks")
    _need(pool_score, torch.float32, B * nq * nbk * block, "pool_score")
    _need(pool_idx, torch.int32, B * nq * nbk * block, "pool_idx")
    q = _bf16_bits(q)
    _check("csa2_index_pool", load().csa2_index_pool(
        _p(q), _p(w), _p(k_codes), _p(k_scales), n_cap, _p(blocks), blocks.shape[-1], block,
        _p(n_visible), B, nq, _p(pool_score), _p(pool_idx), _stream(stream)))


def index_pool_topk_workspace(B, nq, n_blocks) -> int:
    return int(load().csa2_index_pool_topk_workspace(B, nq, n_blocks))


def index_pool_topk(q, w, k_codes, k_scales, blocks, n_visible, out, ws, block=8, stream=None):
    """Pool rescoring and its top-k in one call: out [B, nq, k] = topk(index_pool(blocks)).
    ws: uint8 device workspace of index_pool_topk_workspace(B, nq, n_blocks) bytes, zeroed
    once before its first use (every call leaves its counters zero)."""
    B, nq, n_cap = _indexer_inputs(q, w, k_codes, k_scales, n_visible)
    nbk = blocks.shape[-1]
    k = out.shape[-1]
    _need(blocks, torch.int32, B * nq * nbk, "blocks")
    _need(out, torch.int32, B * nq * k, "out")
    _need(ws, torch.uint8, index_pool_topk_workspace(B, nq, nbk), "ws")
    q = _bf16_bits(q)
    _check("csa2_index_pool_topk", load().csa2_index_pool_topk(
        _p(q), _p(w), _p(k_codes), _p(k_scales), n_cap, _p(blocks), nbk, block, _p(n_visible),
        B, nq, k, _p(out), _p(ws), ws.numel(), _stream(stream)))


def topk_workspace(L, rows, k) -> int:
    return int(load().csa2_topk_workspace(L, rows, k))


def _topk_args(score, k, out, idx, n_valid):
    _dt(score, torch.float32, "score")
    L = score.shape[-1]
    rows = math.prod(score.shape[:-1])  # also for L == 0 (every row then all -1)
    _need(out, torch.int32, rows * k, "out")
    _need(idx, torch.int32, rows * L, "idx", optional=True)
    _need(n_valid, torch.int32, rows, "n_valid", optional=True)
    return L, rows


def topk(score, k, out, idx=None, n_valid=None, ws=None, stream=None):
    L, rows = _topk_args(score, k, out, idx, n_valid)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("csa2_topk", load().csa2_topk(
        _p(score), _p(idx), L, rows, _p(n_valid), k, _p(out), _p(ws), ws_bytes,
        _stream(stream)))


def topk_noalloc(score, k, out, idx=None, n_valid=None, stream=None):
    """csa2_topk with the library's static device workspace (no workspace argument)."""
    L, rows = _topk_args(score, k, out, idx, n_valid)
    _check("csa2_topk_noalloc", load().csa2_topk_noalloc(
        _p(score), _p(idx), L, rows, _p(n_valid), k, _p(out), _stream(stream)))


def stream_read(src, workgroups, depth, sink, stream=None):
    """Streaming read of every byte of src (calibration); sink int32/uint32 [workgroups]."""
    _need(sink, (torch.int32, torch.uint32), workgroups, "sink")
    nbytes = src.numel() * src.element_size()
    _check("csa2_stream_read", load().csa2_stream_read(
        _p(src), nbytes, workgroups, depth, _p(sink), _stream(stream)))


def sparse_attn_workspace(B, nq, k, n_win) -> int:
    return int(load().csa2_sparse_attn_workspace(B, nq, k, n_win))


def _attn_inputs(q, kv_codes, kv_scales, topk_idx, swa, swa_end, lse):
    """(B, nq, n_cap, k) of an attention call after checking q [B, nq, 64, 512] bf16,
    kv_codes [B, n_cap, 256] u8, kv_scales [B, n_cap, 32] u8, topk [B, nq, k] int32,
    swa [B, swa_cap, 512] u8, swa_end [B, nq] int32 and lse [B, nq, 64] fp32."""
    if q.dim() != 4 or q.shape[2:] != (64, 512):
        raise ValueError(f"q: expected [B, nq, 64, 512], got {tuple(q.shape)}")
    B, nq = q.shape[0], q.shape[1]
    _need(q, _BF16, B * nq * 64 * 512, "q")
    if kv_codes.dim() != 3 or kv_codes.shape[0] != B or kv_codes.shape[2] != 256:
        raise ValueError(f"kv_codes: expected [{B}, n_cap, 256], got {tuple(kv_codes.shape)}")
    n_cap = kv_codes.shape[1]
    _need(kv_codes, torch.uint8, B * n_cap * 256, "kv_codes")
    _need(kv_scales, torch.uint8, B * n_cap * 32, "kv_scales")
    k = topk_idx.shape[-1]
    _need(topk_idx, torch.int32, B * nq * k, "topk")
    if swa.dim() != 3 or swa.shape[0] != B or swa.shape[2] != 512:
        raise ValueError(f"swa: expected [{B}, swa_cap, 512], got {tuple(swa.shape)}")
    _need(swa, torch.uint8, swa.numel(), "swa")
    _need(swa_end, torch.int32, B * nq, "swa_end")
    _need(lse, torch.float32, B * nq * 64, "lse", optional=True)
    return B, nq, n_cap, k


def sparse_attn(q, kv_codes, kv_scales, topk_idx, swa, swa_end, out, lse=None, n_win=128,
                softmax_scale=1.0, ws=None, stream=None):
    B, nq, n_cap, k = _attn_inputs(q, kv_codes, kv_scales, topk_idx, swa, swa_end, lse)
    _need(out, torch.float32, B * nq * 64 * 512, "out")
    _need(ws, torch.uint8, 0, "ws", optional=True)
    q = _bf16_bits(q)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("csa2_sparse_attn", load().csa2_sparse_attn(
        _p(q), B, nq, _p(kv_codes), _p(kv_scales), n_cap, _p(topk_idx), k, _p(swa),
        swa.shape[1], _p(swa_end), n_win, float(softmax_scale), _p(out), _p(lse), _p(ws),
        ws_bytes, _stream(stream)))


def sparse_attn_rope_bf16(q, kv_codes, kv_scales, topk_idx, swa, swa_end, rope_cos, rope_sin,
                          out, lse=None, n_win=128, softmax_scale=1.0, rope_offset=448,
                          rope_dim=64, ws=None, stream=None):
    """Attention with the inverse-rotary + bf16 epilogue; out is bf16 (or its uint16 bits)."""
    B, nq, n_cap, k = _attn_inputs(q, kv_codes, kv_scales, topk_idx, swa, swa_end, lse)
    _need(out, _BF16, B * nq * 64 * 512, "out")
    _need(rope_cos, torch.float32, B * nq * (rope_dim // 2), "rope_cos", optional=rope_dim == 0)
    _need(rope_sin, torch.float32, B * nq * (rope_dim // 2), "rope_sin", optional=rope_dim == 0)
    _need(ws, torch.uint8, 0, "ws", optional=True)
    q = _bf16_bits(q)
    out = _bf16_bits(out)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check("csa2_sparse_attn_rope_bf16", load().csa2_sparse_attn_rope_bf16(
        _p(q), B, nq, _p(kv_codes), _p(kv_scales), n_cap, _p(topk_idx), k, _p(swa),
        swa.shape[1], _p(swa_end), n_win, float(softmax_scale), _p(rope_cos), _p(rope_sin),
        rope_offset, rope_dim, _p(out), _p(lse), _p(ws), ws_bytes, _stream(stream)))
