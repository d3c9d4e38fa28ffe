"""Seeded synthetic inputs for the CSA2 workloads (shared by the GPU path and the oracle).

Only inputs live here: latent rows, indexer keys, queries, head weights, rotary
tables, and the shapes of the five workloads.  Nothing in this package encodes,
scores, selects or attends; that is the method, which the GPU library and the
CPU oracle each implement on their own.

Workload shapes follow the DeepSeek-V4.1-Flash reading notes (section 1, model
configuration: indexer 32 heads x 128, top-k 512, query 64 heads x 512, pool of
2048 blocks x 8 positions, sliding window 128; section 2.2: Full / Reindex /
Reuse layer modes, hierarchical indexer in the decoder only) and the
translated abstract (section 3.3 CSA2, section 3.4 hierarchical indexer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_synth.c")
_LIB = os.path.join(_HERE, "libcsa2_synth.so")

# tensor tags of the counter-based streams
TAG_IDX_K = 1
TAG_KV = 2
TAG_KV_OUT = 3
TAG_SWA = 4
TAG_SWA_OUT = 5
TAG_Q_IDX = 6
TAG_W_IDX = 7
TAG_Q_MAIN = 8
TAG_W_PROJ = 9

SEED = 0
P_OUTLIER = 1e-3
OUTLIER = 10.0
RMS_EPS = 1e-6
ROPE_BASE = 10000.0
ROPE_OFFSET = 448
ROPE_DIM = 64


def build(force: bool = True) -> str:
    """Compile the generator with gcc (OpenMP) into synth/libcsa2_synth.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64] * 5
        L.synth_normal_f32.argtypes = [u64, i64, i64, dbl, vp]
        L.synth_normal_bf16.argtypes = [u64, i64, i64, dbl, vp]
        L.synth_uniform_f32.argtypes = [u64, i64, i64, dbl, dbl, vp]
        L.synth_latent_rows.argtypes = [u64, u64, i64, i64, i32, dbl, dbl, dbl, vp]
        L.synth_rope_table.argtypes = [vp, i64, i32, dbl, vp, vp]
        L.synth_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(config: int, tag: int, layer: int = 0, seq: int = 0, seed: int = SEED) -> int:
    return int(lib().synth_key(seed, config, tag, layer, seq))


def normal_f32(k: int, start: int, n: int, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(k, start, n, scale, _ptr(out))
    return out


def normal_bf16(k: int, start: int, n: int, scale: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32(scale * N(0,1))."""
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(k, start, n, scale, _ptr(out))
    return out


def uniform_f32(k: int, start: int, n: int, lo: float = 0.0, hi: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_uniform_f32(k, start, n, lo, hi, _ptr(out))
    return out


def latent_rows(k: int, k_out: int, row0: int, rows: int, C: int = 512,
                p_out: float = P_OUTLIER, outlier: float = OUTLIER, eps: float = RMS_EPS,
                out: np.ndarray | None = None) -> np.ndarray:
    if out is None:
        out = np.empty((rows, C), np.float32)
    assert out.dtype == np.float32 and out.shape == (rows, C)
    lib().synth_latent_rows(k, k_out, row0, rows, C, p_out, outlier, eps, _ptr(out))
    return out


def rope_table(positions, rope_dim: int = ROPE_DIM, base: float = ROPE_BASE):
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int64))
    half = rope_dim // 2
    c = np.empty((pos.size, half), np.float32)
    s = np.empty((pos.size, half), np.float32)
    lib().synth_rope_table(_ptr(pos), pos.size, rope_dim, base, _ptr(c), _ptr(s))
    return c, s


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------

@dataclass
class Workload:
    """One of the six synthetic CSA2 workloads.

    B sequences, nq queries each, n_cap compressed entries per sequence of which
    n_visible[b, i] are visible to query i; k = top-k, nb = pool blocks (0 = no
    pool), block = positions per block; layers = call sequence.
    """
    config: int
    name: str
    B: int
    nq: int
    n_cap: int
    k: int
    nb: int
    block: int = 8
    layers: tuple = ("full",)
    m: int = 1
    n_win: int = 128
    # prefill only: token range of the chunk
    tokens: int = 0
    chunk: int = 0
    h_idx: int = 32
    d_idx: int = 128
    h: int = 64
    d: int = 512
    extra: dict = field(default_factory=dict)

    @property
    def decode(self) -> bool:
        return self.nq == 1

    def n_visible(self) -> np.ndarray:
        """[B, nq] visible entries per query.

        Decode: every entry, including the one the current token just appended.
        Prefill (m tokens per entry): entry j covers tokens [m*j, m*j+m) and is
        visible to token t once its last token is, i.e. m*j + m - 1 <= t.
        """
        if self.decode:
            return np.full((self.B, self.nq), self.n_cap, np.int32)
        t = (self.tokens - self.chunk) + np.arange(self.nq, dtype=np.int64)
        nv = (t + 1) // self.m
        return np.broadcast_to(nv.astype(np.int32), (self.B, self.nq)).copy()

    def swa_rows(self) -> int:
        """Rows of the per-(layer, sequence) FP8 window buffer."""
        if self.decode:
            return self.n_win
        return self.n_win - 1 + self.chunk

    def swa_end(self) -> np.ndarray:
        """[B, nq] exclusive end row of each query's window in the window buffer.

        Decode: a 128-slot ring that is full, rows [0, 128).  Prefill: the buffer
        holds token rows [chunk_start - 127, chunk_end) and token chunk_start + i
        sits at row 127 + i, so its window [t - 127, t] is rows [i, i + 128).
        """
        if self.decode:
            return np.full((self.B, self.nq), self.n_win, np.int32)
        e = self.n_win + np.arange(self.nq, dtype=np.int32)
        return np.broadcast_to(e, (self.B, self.nq)).copy()

    def new_entries(self) -> tuple[int, int]:
        """(first, count) of the compressed entries this step appends per sequence."""
        if self.decode:
            return self.n_cap - 1, 1
        first = (self.tokens - self.chunk) // self.m
        return first, self.chunk // self.m


WORKLOADS = {
    0: Workload(0, "tiny CSA2 Full-layer decode, 1 query x 2048 entries, top-64, 32-block pool",
                B=1, nq=1, n_cap=2048, k=64, nb=32),
    1: Workload(1, "CSA2 Full-layer decode, batch 64 x 65536 entries",
                B=64, nq=1, n_cap=65536, k=512, nb=2048),
    2: Workload(2, "decoder CSA2 group Full->Reindex->Reuse->Reuse, batch 128 x 262144 entries",
                B=128, nq=1, n_cap=262144, k=512, nb=2048,
                layers=("full", "reindex", "reuse", "reuse")),
    3: Workload(3, "1M-context CSA2 Full-layer decode, batch 16 x 1048576 entries",
                B=16, nq=1, n_cap=1048576, k=512, nb=2048),
    4: Workload(4, "encoder CSA2 chunked prefill (m=2), 4096 tokens of 131072, 65536 entries",
                B=1, nq=4096, n_cap=65536, k=512, nb=0, m=2, tokens=131072, chunk=4096),
    5: Workload(5, "decoder CSA2 chunked prefill (m=1) Full->Reindex with a 2048-block pool "
                   "per token, 1024 tokens of 65536",
                B=1, nq=1024, n_cap=65536, k=512, nb=2048, m=1, tokens=65536, chunk=1024,
                layers=("full", "reindex")),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    from dataclasses import replace
    return replace(w, **changes)


# ---- per-tensor generators (all seeded by (config, tag, layer, sequence)) ----

def idx_k_rows(w: Workload, seq: int, row0: int, rows: int) -> np.ndarray:
    """Indexer keys, fp32 [rows, 128], N(0,1) per channel."""
    return normal_f32(key(w.config, TAG_IDX_K, 0, seq), row0 * w.d_idx, rows * w.d_idx).reshape(rows, w.d_idx)


def kv_rows(w: Workload, seq: int, row0: int, rows: int, out=None) -> np.ndarray:
    """Main-KV latent rows before rotary, fp32 [rows, 512] (outliers, RMSNorm)."""
    return latent_rows(key(w.config, TAG_KV, 0, seq), key(w.config, TAG_KV_OUT, 0, seq),
                       row0, rows, w.d, out=out)


def swa_rows(w: Workload, layer: int, seq: int, row0: int, rows: int) -> np.ndarray:
    """Sliding-window latent rows of one layer, fp32 [rows, 512] (same recipe as the main KV)."""
    return latent_rows(key(w.config, TAG_SWA, layer, seq), key(w.config, TAG_SWA_OUT, layer, seq),
                       row0, rows, w.d)


def q_idx(w: Workload, layer: int, B: int | None = None) -> np.ndarray:
    """Indexer queries, bf16 bits [B, nq, 32, 128] ~ N(0, 1/128)."""
    B = w.B if B is None else B
    n = w.nq * w.h_idx * w.d_idx
    out = np.empty((B, n), np.uint16)
    for b in range(B):
        out[b] = normal_bf16(key(w.config, TAG_Q_IDX, layer, b), 0, n, 1.0 / np.sqrt(w.d_idx))
    return out.reshape(B, w.nq, w.h_idx, w.d_idx)


def w_idx(w: Workload, layer: int, B: int | None = None) -> np.ndarray:
    """Indexer head weights, fp32 [B, nq, 32] ~ U(0,1)."""
    B = w.B if B is None else B
    n = w.nq * w.h_idx
    out = np.empty((B, n), np.float32)
    for b in range(B):
        out[b] = uniform_f32(key(w.config, TAG_W_IDX, layer, b), 0, n)
    return out.reshape(B, w.nq, w.h_idx)


def w_proj(w: Workload) -> np.ndarray:
    """Indexer-key projection of the main latent, bf16 bits [128, 512], N(0, 1/512), so a
    projected key of an RMS-normalised latent row has unit variance per channel like the
    synthetic indexer keys."""
    return normal_bf16(key(w.config, TAG_W_PROJ, 0, 0), 0, w.d_idx * w.d,
                       1.0 / np.sqrt(w.d)).reshape(w.d_idx, w.d)


def q_main(w: Workload, layer: int, B: int | None = None) -> np.ndarray:
    """Attention queries, bf16 bits [B, nq, 64, 512] ~ N(0, 1/512)."""
    B = w.B if B is None else B
    n = w.nq * w.h * w.d
    out = np.empty((B, n), np.uint16)
    for b in range(B):
        out[b] = normal_bf16(key(w.config, TAG_Q_MAIN, layer, b), 0, n, 1.0 / np.sqrt(w.d))
    return out.reshape(B, w.nq, w.h, w.d)


def rope_rows(row0: int, rows: int):
    """Rotary cos/sin for compressed entries [row0, row0 + rows) (position = entry index)."""
    return rope_table(np.arange(row0, row0 + rows, dtype=np.int64))
