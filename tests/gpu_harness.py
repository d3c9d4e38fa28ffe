"""Helpers of the GPU parity tests: build one workload's inputs, encode them on
both sides, run the GPU layer sequence through the C ABI and the oracle's per
query steps, and compare.

Inputs come only from `synth` (seeded).  The oracle encodes its own caches; the
GPU encodes its own with csa2_quantize_kv / csa2_quantize_swa, and the tests
assert the two encodings are bit-identical before comparing anything
downstream, so every later stage sees identical inputs on both sides.  The only
GPU outputs the oracle ever takes are selections (index sets: a pool, a top-k)
that were first checked against the oracle's own selection with check_set;
the next stage (attention, Reindex) is then compared on that same validated
set, so a near-tie swap cannot hide a downstream comparison.  No GPU score,
code or floating-point value is ever fed to the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import synth
from kv_cache_decode_mxfp4_amd import _lib, layers

NEAR_TIE_REL = 1e-6   # sets may differ only by entries this close to the k-th score
ATTN_TOL = 2e-3       # max-abs error of attention outputs


def dev():
    return torch.device("cuda:0")


# The GPU's indexer-key code cache is tiled (include/csa2.h, csa2_quantize_kv with 128
# channels): byte j of entry f at (f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16.
# The oracle keeps plain [rows, 64] rows; these two permutations convert between them.

def tile_keys(codes: np.ndarray) -> np.ndarray:
    """Row-major key codes [..., rows, 64] (leading dims flattened in order) -> the tiled
    byte array of whole 32-entry tiles [tiles, 2048], padding entries zero."""
    flat = np.ascontiguousarray(codes).reshape(-1, 64)
    n = flat.shape[0]
    tiles = -(-n // 32)
    pad = np.zeros((tiles * 32, 64), np.uint8)
    pad[:n] = flat
    # [tile, entry, chunk, byte] -> [tile, chunk, entry, byte]
    return np.ascontiguousarray(pad.reshape(tiles, 32, 4, 16).transpose(0, 2, 1, 3)).reshape(tiles, 2048)


def seq_keys(tiled: torch.Tensor, b: int, n_cap: int) -> np.ndarray:
    """Row-major codes [n_cap, 64] of sequence b of a tiled [B, n_cap] key cache (copies
    only that sequence's tiles to the host)."""
    flat = tiled.reshape(-1)
    t0, t1 = (b * n_cap) // 32, -(-((b + 1) * n_cap) // 32)
    rows = untile_keys(flat[t0 * 2048:t1 * 2048], (t1 - t0) * 32)
    return rows[b * n_cap - t0 * 32:][:n_cap]


def untile_keys(tiled, rows: int) -> np.ndarray:
    """Inverse of tile_keys: the first `rows` entries as row-major [rows, 64]."""
    a = tiled.cpu().numpy() if isinstance(tiled, torch.Tensor) else np.asarray(tiled)
    a = a.reshape(-1, 4, 32, 16).transpose(0, 2, 1, 3).reshape(-1, 64)
    return np.ascontiguousarray(a[:rows])


@dataclass
class Case:
    w: synth.Workload
    n_layers: int
    idx_x: np.ndarray = None      # [B, n_cap, 128] f32
    kv_x: np.ndarray = None       # [B, n_cap, 512] f32 (before rotary)
    cos: np.ndarray = None        # [n_cap, 32]
    sin: np.ndarray = None
    swa_x: list = field(default_factory=list)   # per layer [B, swa_rows, 512]
    q_idx: list = field(default_factory=list)   # per layer [B, nq, 32, 128] u16
    w_idx: list = field(default_factory=list)   # per layer [B, nq, 32]
    q_main: list = field(default_factory=list)  # per layer [B, nq, 64, 512] u16
    # oracle encodings
    o_kc: np.ndarray = None
    o_ks: np.ndarray = None
    o_vc: np.ndarray = None
    o_vs: np.ndarray = None
    o_swa: list = field(default_factory=list)


def build_case(w: synth.Workload, n_layers: int | None = None, idx_transform=None) -> Case:
    """Inputs of one workload from synth, and the oracle's encodings of them.
    idx_transform(idx_x [B, n_cap, 128]) -> idx_x: changes the indexer-key rows before
    both sides encode them (adversarial cases: duplicated keys)."""
    n_layers = len(w.layers) if n_layers is None else n_layers
    c = Case(w=w, n_layers=n_layers)
    B, N = w.B, w.n_cap
    c.idx_x = np.stack([synth.idx_k_rows(w, b, 0, N) for b in range(B)])
    if idx_transform is not None:
        c.idx_x = np.ascontiguousarray(idx_transform(c.idx_x), dtype=np.float32)
    c.kv_x = np.stack([synth.kv_rows(w, b, 0, N) for b in range(B)])
    c.cos, c.sin = synth.rope_rows(0, N)
    for layer in range(n_layers):
        c.swa_x.append(np.stack([synth.swa_rows(w, layer, b, 0, w.swa_rows()) for b in range(B)]))
        c.q_idx.append(synth.q_idx(w, layer))
        c.w_idx.append(synth.w_idx(w, layer))
        c.q_main.append(synth.q_main(w, layer))
    kc, ks, vc, vs = [], [], [], []
    for b in range(B):
        a, s = oracle.quantize_rows(c.idx_x[b])
        kc.append(a)
        ks.append(s)
        a, s = oracle.quantize_rows(c.kv_x[b], c.cos, c.sin, synth.ROPE_OFFSET, synth.ROPE_DIM)
        vc.append(a)
        vs.append(s)
    c.o_kc, c.o_ks, c.o_vc, c.o_vs = map(np.stack, (kc, ks, vc, vs))
    c.o_swa = [oracle.encode_fp8(x) for x in c.swa_x]
    return c


def t(a, dtype=None):
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.view(dtype)
    return x.to(dev())


def gpu_encode(c: Case) -> dict:
    """Device caches encoded by the GPU library from the same fp32 inputs."""
    w = c.w
    B, N = w.B, w.n_cap
    d = {}
    d["kc"] = _lib.key_codes_empty(B * N, device=dev())
    d["ks"] = torch.empty(B, N, 8, dtype=torch.uint8, device=dev())
    d["vc"] = torch.empty(B, N, 256, dtype=torch.uint8, device=dev())
    d["vs"] = torch.empty(B, N, 32, dtype=torch.uint8, device=dev())
    cos, sin = t(c.cos), t(c.sin)
    for b in range(B):
        _lib.quantize_kv(t(c.idx_x[b]), d["kc"], d["ks"], dst_row=b * N)
        _lib.quantize_kv(t(c.kv_x[b]), d["vc"][b], d["vs"][b], cos, sin, synth.ROPE_OFFSET,
                         synth.ROPE_DIM)
    d["swa"] = []
    for layer in range(c.n_layers):
        out = torch.empty(B, w.swa_rows(), 512, dtype=torch.uint8, device=dev())
        _lib.quantize_swa(t(c.swa_x[layer]), out)
        d["swa"].append(out)
    d["q_idx"] = [t(q, torch.uint16) for q in c.q_idx]
    d["w_idx"] = [t(x) for x in c.w_idx]
    d["q_main"] = [t(q, torch.uint16) for q in c.q_main]
    d["n_vis"] = t(w.n_visible())
    d["n_blk"] = layers.n_valid_blocks(d["n_vis"])
    d["swa_end"] = t(w.swa_end())
    torch.cuda.synchronize()
    return d


def assert_encodings_equal(c: Case, d: dict):
    B, N = c.w.B, c.w.n_cap
    assert np.array_equal(untile_keys(d["kc"], B * N).reshape(B, N, 64), c.o_kc), \
        "indexer key codes differ"
    assert np.array_equal(d["ks"].cpu().numpy(), c.o_ks), "indexer key scales differ"
    assert np.array_equal(d["vc"].cpu().numpy(), c.o_vc), "main KV codes differ"
    assert np.array_equal(d["vs"].cpu().numpy(), c.o_vs), "main KV scales differ"
    for layer in range(c.n_layers):
        assert np.array_equal(d["swa"][layer].cpu().numpy(), c.o_swa[layer]), "window bytes differ"


def check_set(gpu: np.ndarray, ref: np.ndarray, score_of, what: str) -> int:
    """Selections agree up to near-ties: every index in the symmetric difference
    has an oracle score within NEAR_TIE_REL * |tau| of the oracle's k-th score tau.
    Returns the number of such swaps."""
    g = set(int(x) for x in gpu if x >= 0)
    o = set(int(x) for x in ref if x >= 0)
    assert len(g) == len(o), f"{what}: {len(g)} selected vs {len(o)}"
    assert np.all(np.diff(gpu[gpu >= 0]) > 0), f"{what}: output not ascending"
    assert np.all(gpu[len(g):] == -1), f"{what}: padding"
    diff = g ^ o
    if not diff:
        return 0
    tau = min(score_of(i) for i in o)
    for i in diff:
        assert abs(score_of(i) - tau) <= NEAR_TIE_REL * abs(tau), (
            f"{what}: index {i} score {score_of(i)!r} is not a near-tie of {tau!r}")
    return len(diff) // 2


def oracle_full(c: Case, b: int, i: int, layer: int = 0):
    w = c.w
    nv = int(w.n_visible()[b, i])
    return oracle.full_layer(c.q_idx[layer][b, i], c.w_idx[layer][b, i], c.o_kc[b], c.o_ks[b],
                             nv, w.k, w.nb, w.block)


def oracle_attention(c: Case, b: int, i: int, layer: int, sel):
    w = c.w
    return oracle.attention(c.q_main[layer][b, i], c.o_vc[b], c.o_vs[b], sel, c.o_swa[layer][b],
                            int(w.swa_end()[b, i]), w.n_win, 1.0)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def cdiv(a, b):
    return (a + b - 1) // b


def finite_close(gpu, ref, rtol=1e-5, atol=1e-5):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    same_inf = np.isinf(gpu) & np.isinf(ref) & (np.sign(gpu) == np.sign(ref))
    ok = same_inf | (np.abs(gpu - ref) <= atol + rtol * np.abs(ref))
    return bool(np.all(ok)), float(np.max(np.abs(np.where(same_inf, 0, gpu - ref)), initial=0.0))


__all__ = ["Case", "build_case", "gpu_encode", "assert_encodings_equal", "check_set",
           "oracle_full", "oracle_attention", "max_abs", "cdiv", "finite_close", "t", "dev",
           "ATTN_TOL", "NEAR_TIE_REL", "math"]
