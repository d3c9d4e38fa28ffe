"""CPU oracle of the CSA2 hot path -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py`
may import this package.  The product path (kv_cache_decode_mxfp4_amd) never
does, and shares no code with it.  The arithmetic lives in plain C
(`csa2_oracle.c`, double precision, no FMA contraction); this module only
marshals numpy arrays and strings the per-query steps into the three layer
modes:

  Full    ([N] 2.2, [A] 3.3-3.4): score every visible entry, top-k over the
          entries, block maxima, top-nb blocks as the pool;
  Reindex ([N] 2.2, [A] 3.3-3.4): score only the pool with the layer's own
          indexer query, top-k;
  Reuse   ([N] 2.2, [A] 3.3): attention with the latest top-k, no scoring.

[N] = "DeepSeek V4.1: model architecture and system design, close reading";
[A] = "DeepSeek-V4.1-Flash: pushing KV cache compression to the limit"
(translated abstract); [S] = "DeepSeek-V4 model structure (7)".

Parity unpinned: the indexer score formula (the pages give its shape only).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2_oracle.so")

H_IDX, D_IDX, H, D = 32, 128, 64, 512


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, OpenMP, no FMA contraction, IEEE math."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32, dbl, u8 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_uint8)
        L.oracle_e4m3_decode.restype = dbl
        L.oracle_e4m3_decode.argtypes = [u8]
        L.oracle_e2m1_decode.restype = dbl
        L.oracle_e2m1_decode.argtypes = [u8]
        L.oracle_e4m3_encode.restype = u8
        L.oracle_e4m3_encode.argtypes = [dbl]
        L.oracle_e4m3_encode_signed.restype = u8
        L.oracle_e4m3_encode_signed.argtypes = [dbl]
        L.oracle_quantize_rows.argtypes = [vp, i64, i32, vp, vp, i32, i32, vp, vp]
        L.oracle_encode_fp8.argtypes = [vp, i64, vp]
        L.oracle_dequant_row.argtypes = [vp, vp, i32, vp]
        L.oracle_index_scores.argtypes = [vp, vp, i32, i32, vp, vp, i64, vp]
        L.oracle_block_max.argtypes = [vp, i64, i32, vp]
        L.oracle_select.restype = i64
        L.oracle_select.argtypes = [vp, vp, i64, i64, vp]
        L.oracle_pool_positions.argtypes = [vp, i32, i32, i64, vp]
        L.oracle_index_scores_at.argtypes = [vp, vp, i32, i32, vp, vp, vp, i64, vp]
        L.oracle_attention.argtypes = [vp, i32, i32, vp, vp, i64, vp, i32, vp, i64, i64, i32,
                                       dbl, vp, vp]
        L.oracle_project_rows.argtypes = [vp, i64, i32, vp, i32, vp]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_rne.argtypes = [dbl]
        L.oracle_inverse_rope_bf16.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp]
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


def threads() -> int:
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not depend on it);
    n < 1 restores the default."""
    lib().oracle_set_threads(int(n))


# ---------------------------------------------------------------- formats

def e4m3_decode(b: int) -> float:
    return float(lib().oracle_e4m3_decode(int(b)))


def e2m1_decode(n: int) -> float:
    return float(lib().oracle_e2m1_decode(int(n)))


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def quantize_rows(x, cos=None, sin=None, rope_off: int = 448, rope_dim: int = 64):
    """fp32 rows [R, C] -> (codes u8 [R, C/2], scales u8 [R, C/16]); rotary first if cos given."""
    x = _c(x, np.float32)
    R, C = x.shape
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    if cos is None:
        lib().oracle_quantize_rows(_p(x), R, C, None, None, 0, 0, _p(codes), _p(scales))
    else:
        cos, sin = _c(cos, np.float32), _c(sin, np.float32)
        assert cos.shape == (R, rope_dim // 2) and sin.shape == cos.shape
        lib().oracle_quantize_rows(_p(x), R, C, _p(cos), _p(sin), rope_off, rope_dim,
                                   _p(codes), _p(scales))
    return codes, scales


def encode_fp8(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_encode_fp8(_p(x), x.size, _p(out))
    return out


def dequant_rows(codes, scales) -> np.ndarray:
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    R, half = codes.shape
    C = 2 * half
    out = np.empty((R, C), np.float64)
    for r in range(R):
        lib().oracle_dequant_row(_p(codes[r]), _p(scales[r]), C, _p(out[r]))
    return out


# ---------------------------------------------------------------- indexer

def index_scores(q, w, codes, scales, n_vis: int) -> np.ndarray:
    """Scores of entries [0, n_vis) for one query: q bf16 bits [32,128], w [32]."""
    q, w = _c(q, np.uint16), _c(w, np.float32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    Hq, Dq = q.shape
    assert codes.shape[0] >= n_vis and codes.shape[1] == Dq // 2
    out = np.empty(n_vis, np.float64)
    lib().oracle_index_scores(_p(q), _p(w), Hq, Dq, _p(codes), _p(scales), n_vis, _p(out))
    return out


def index_scores_at(q, w, codes, scales, pos) -> np.ndarray:
    q, w = _c(q, np.uint16), _c(w, np.float32)
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    pos = _c(pos, np.int32)
    assert pos.max(initial=-1) < codes.shape[0]
    out = np.empty(pos.size, np.float64)
    lib().oracle_index_scores_at(_p(q), _p(w), q.shape[0], q.shape[1], _p(codes), _p(scales),
                                 _p(pos), pos.size, _p(out))
    return out


def block_max(s, block: int) -> np.ndarray:
    s = _c(s, np.float64)
    out = np.empty((s.size + block - 1) // block, np.float64)
    lib().oracle_block_max(_p(s), s.size, block, _p(out))
    return out


def select(s, k: int, idx=None) -> np.ndarray:
    s = _c(s, np.float64)
    out = np.empty(k, np.int32)
    if idx is not None:
        idx = _c(idx, np.int32)
        assert idx.size == s.size
    lib().oracle_select(_p(s), _p(idx), s.size, k, _p(out))
    return out


def pool_positions(blocks, block: int, n_vis: int) -> np.ndarray:
    blocks = _c(blocks, np.int32)
    out = np.empty(blocks.size * block, np.int32)
    lib().oracle_pool_positions(_p(blocks), blocks.size, block, n_vis, _p(out))
    return out


# ---------------------------------------------------------------- attention

def attention(q, kv_codes, kv_scales, sel, swa, swa_end: int, n_win: int = 128,
              scale: float = 1.0):
    """One query: q bf16 bits [64,512] -> (out [64,512] f64, lse [64] f64)."""
    q = _c(q, np.uint16)
    kv_codes, kv_scales = _c(kv_codes, np.uint8), _c(kv_scales, np.uint8)
    sel = _c(sel, np.int32)
    swa = _c(swa, np.uint8)
    Hq, Dq = q.shape
    out = np.empty((Hq, Dq), np.float64)
    lse = np.empty(Hq, np.float64)
    lib().oracle_attention(_p(q), Hq, Dq, _p(kv_codes), _p(kv_scales), kv_codes.shape[0],
                           _p(sel), sel.size, _p(swa), swa.shape[0], int(swa_end), n_win,
                           float(scale), _p(out), _p(lse))
    return out, lse


def project_rows(x, w_bits):
    """Indexer-key projection of new entries: x fp32 [R, D] . w bf16 bits [O, D]^T in double."""
    x = _c(x, np.float32)
    w_bits = _c(w_bits, np.uint16)
    R, Dx = x.shape
    O = w_bits.shape[0]
    y = np.empty((R, O), np.float64)
    lib().oracle_project_rows(_p(x), R, Dx, _p(w_bits), O, _p(y))
    return y


def bf16_rne(x: float) -> int:
    """bf16 bit pattern nearest to x (ties to even)."""
    return int(lib().oracle_bf16_rne(float(x)))


def inverse_rope_bf16(o, cos_row, sin_row, rope_off: int = 448, rope_dim: int = 64):
    """Attention output o [H, D] (double) -> bf16 bits [H, D] after rotating the rotary
    channels back by the query's angle (cos_row, sin_row: [rope_dim/2] fp32)."""
    o = _c(o, np.float64)
    Hq, Dq = o.shape
    cs, sn = _c(cos_row, np.float32), _c(sin_row, np.float32)
    bits = np.empty((Hq, Dq), np.uint16)
    lib().oracle_inverse_rope_bf16(_p(o), Hq, Dq, _p(cs), _p(sn), rope_off, rope_dim, _p(bits))
    return bits


def attention_rope_bf16(q, kv_codes, kv_scales, sel, swa, swa_end: int, cos_row, sin_row,
                        n_win: int = 128, scale: float = 1.0, rope_off: int = 448,
                        rope_dim: int = 64):
    """One query: attention, then the inverse-rotary + bf16 epilogue.  Returns
    (bf16 bits [64,512], the double output before the epilogue, lse [64])."""
    out, lse = attention(q, kv_codes, kv_scales, sel, swa, swa_end, n_win, scale)
    return inverse_rope_bf16(out, cos_row, sin_row, rope_off, rope_dim), out, lse


# ---------------------------------------------------------------- layer modes (one query)

def full_layer(q_idx, w_idx, k_codes, k_scales, n_vis: int, k: int, nb: int, block: int = 8):
    """Full mode: scores over the whole visible range, top-k, block maxima, pool of nb blocks."""
    s = index_scores(q_idx, w_idx, k_codes, k_scales, n_vis)
    top = select(s, k)
    res = {"scores": s, "topk": top}
    if nb > 0:
        bm = block_max(s, block)
        res["block_max"] = bm
        res["pool"] = select(bm, nb)
    return res


def reindex_layer(q_idx, w_idx, k_codes, k_scales, n_vis: int, pool, k: int, block: int = 8):
    """Reindex mode: score only the pool's positions with this layer's query, top-k."""
    pos = pool_positions(pool, block, n_vis)
    s = index_scores_at(q_idx, w_idx, k_codes, k_scales, pos)
    top = select(s, k, idx=pos)
    return {"pool_pos": pos, "pool_scores": s, "topk": top}
