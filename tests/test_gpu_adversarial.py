"""Adversarial end-to-end parity of the Full layer ([N] 2.2, [A] 3.4: the block score
is the largest index score of its positions; the pool holds the 2048 best blocks; the
top-k entries are ranked over the whole visible range with the lower index winning a
tie) through the production call sequence (csa2_index_full_select -> csa2_sparse_attn),
against the oracle's literal full-range top-k:

* duplicated indexer keys -- every key repeats with a period, so scores and block
  maxima tie EXACTLY across periods, at the k-th score and at the 2048-th block maximum;
  exact ties are bit-identical on both sides (the same key bytes), so the selections
  must be equal, not merely near-tie equivalent;
* a zero indexer query -- every score is 0, so the top-k is entries 0..k-1 and the
  pool blocks 0..nb-1 exactly (the tie-break's closed form);
both at a small shape (direct block select) and at a shape whose rows take the scan's
per-chunk candidates (and, for the ties, their exact fallback).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (ATTN_TOL, assert_encodings_equal, build_case, check_set, gpu_encode,
                         max_abs, oracle_attention, oracle_full)

pytestmark = pytest.mark.gpu

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
layers = kv.layers

W = synth.WORKLOADS
SHAPES = {
    "small_direct": synth.scaled(W[1], B=2, n_cap=40000),
    "candidates_4x256k": synth.scaled(W[1], B=4, n_cap=262144),
}


def _periodic(period):
    def f(x):
        y = x.copy()
        for s in range(period, x.shape[1], period):
            n = min(period, x.shape[1] - s)
            y[:, s:s + n] = x[:, :n]
        return y
    return f


def _run_full(c, d):
    w = c.w
    buf = layers.Buffers.create(w.B, 1, w.n_cap, w.k, w.nb, w.n_win)
    layers.full_indexer(buf, d["q_idx"][0], d["w_idx"][0], d["kc"], d["ks"], d["n_vis"],
                        d["n_blk"], w.k, w.nb)
    layers.attention(buf, d["q_main"][0], d["vc"], d["vs"], buf.topk, d["swa"][0], d["swa_end"])
    torch.cuda.synchronize()
    return buf.pool.cpu().numpy(), buf.topk.cpu().numpy(), buf.out.cpu().numpy()


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("period", [4096, 8000])
def test_full_layer_exact_ties_from_duplicated_keys(shape, period):
    w = SHAPES[shape]
    print(f"[case] {shape} period={period}", flush=True)
    c = build_case(w, n_layers=1, idx_transform=_periodic(period))
    d = gpu_encode(c)
    assert_encodings_equal(c, d)
    g_pool, g_top, g_out = _run_full(c, d)
    tied_k = tied_nb = 0
    for b in range(w.B):
        full = oracle_full(c, b, 0)
        s, bm = full["scores"], full["block_max"]
        # the tie groups really straddle the k-th score and the nb-th block maximum
        tau = np.sort(s)[::-1][w.k - 1]
        tied_k += int(np.sum(s == tau) > 1)
        beta = np.sort(bm)[::-1][w.nb - 1]
        tied_nb += int(np.sum(bm == beta) > 1)
        assert np.array_equal(g_top[b, 0], full["topk"]), f"top-k seq {b}"
        assert np.array_equal(g_pool[b, 0], full["pool"]), f"pool seq {b}"
        ro, _ = oracle_attention(c, b, 0, 0, g_top[b, 0])
        assert max_abs(g_out[b, 0], ro) <= ATTN_TOL, f"attention seq {b}"
    assert tied_k == w.B and tied_nb == w.B, (tied_k, tied_nb)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_full_layer_zero_query_takes_the_lowest_positions(shape):
    w = SHAPES[shape]
    print(f"[case] {shape} zero indexer query", flush=True)
    c = build_case(w, n_layers=1)
    c.q_idx[0][:] = 0  # every score is exactly 0
    d = gpu_encode(c)
    assert_encodings_equal(c, d)
    g_pool, g_top, g_out = _run_full(c, d)
    for b in range(w.B):
        full = oracle_full(c, b, 0)
        assert np.all(full["scores"] == 0.0)
        assert np.array_equal(full["topk"], np.arange(w.k))    # the oracle's own closed form
        assert np.array_equal(full["pool"], np.arange(w.nb))
        assert np.array_equal(g_top[b, 0], np.arange(w.k)), f"top-k seq {b}"
        assert np.array_equal(g_pool[b, 0], np.arange(w.nb)), f"pool seq {b}"
        ro, _ = oracle_attention(c, b, 0, 0, g_top[b, 0])
        assert max_abs(g_out[b, 0], ro) <= ATTN_TOL, f"attention seq {b}"
