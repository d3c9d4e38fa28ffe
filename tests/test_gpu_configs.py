"""End-to-end parity of the Full / Reindex / Reuse call sequences with the oracle,
on the five workloads (config 0 at full size, the others at sizes the oracle
finishes in seconds that still span many tiles, several top-k segments and
ragged tails).  The full-size launch configurations are covered by
test_gpu_fullsize.py on sampled outputs.

Every run checks, in order: the GPU encodings equal the oracle's bit for bit;
the scan's scores match the oracle's; the GPU pool and top-k equal the oracle's
up to near-ties (check_set); the Reindex top-k against the oracle's Reindex of
the GPU's own pool (validated just before); attention outputs within 2e-3 of
the oracle's attention over the GPU's own selection, for EVERY row (the number
of rows compared is asserted); and stage-isolated, the attention and the
Reindex layer on the oracle's selections.  The GPU chain runs the production
call sequence (layers.full_indexer without per-entry scores); the scores come
from a separate csa2_index_full call on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (ATTN_TOL, assert_encodings_equal, build_case, check_set, finite_close,
                         gpu_encode, max_abs, oracle_attention, oracle_full, t)

pytestmark = pytest.mark.gpu

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
layers = kv.layers
L = kv._lib

W = synth.WORKLOADS
CASES = {
    "cfg0_full_size": W[0],
    "cfg1_small": synth.scaled(W[1], B=3, n_cap=40001),
    "cfg2_small": synth.scaled(W[2], B=2, n_cap=30005),
    "cfg3_small_multilevel_topk": synth.scaled(W[3], B=2, n_cap=140003),
}


def _attention_stage(c, d, layer, sel):
    """GPU attention with a given (oracle) selection [B, nq, k]."""
    w = c.w
    buf = layers.Buffers.create(w.B, w.nq, w.n_cap, w.k, w.nb, w.n_win)
    layers.attention(buf, d["q_main"][layer], d["vc"], d["vs"], t(sel), d["swa"][layer],
                     d["swa_end"], w.n_win)
    return buf.out.cpu().numpy(), buf.lse.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_decode_layer_sequence(name):
    w = CASES[name]
    print(f"[case] {name}: B={w.B} n_cap={w.n_cap} k={w.k} nb={w.nb} layers={w.layers}", flush=True)
    c = build_case(w)
    d = gpu_encode(c)
    assert_encodings_equal(c, d)
    B, k, nb = w.B, w.k, w.nb

    # ---- GPU chain, end to end, in the production call sequence
    buf = layers.Buffers.create(B, 1, w.n_cap, k, nb, w.n_win)
    layers.full_indexer(buf, d["q_idx"][0], d["w_idx"][0], d["kc"], d["ks"], d["n_vis"], d["n_blk"],
                        k, nb)
    g_pool = buf.pool.cpu().numpy().copy()
    g_top = [buf.topk.cpu().numpy().copy()]
    layers.attention(buf, d["q_main"][0], d["vc"], d["vs"], buf.topk, d["swa"][0], d["swa_end"])
    g_out = [buf.out.cpu().numpy().copy()]
    if "reindex" in w.layers:
        layers.reindex_indexer(buf, d["q_idx"][1], d["w_idx"][1], d["kc"], d["ks"], d["n_vis"],
                               buf.pool, k)
        g_top.append(buf.topk.cpu().numpy().copy())
        for layer in range(1, len(w.layers)):
            layers.attention(buf, d["q_main"][layer], d["vc"], d["vs"], buf.topk, d["swa"][layer],
                             d["swa_end"])
            g_out.append(buf.out.cpu().numpy().copy())
    scores = torch.empty(B, 1, w.n_cap, device="cuda")
    L.index_full(d["q_idx"][0], d["w_idx"][0], d["kc"], d["ks"], d["n_vis"],
                 torch.empty(B, 1, -(-w.n_cap // 8), device="cuda"), scores=scores)
    g_scores = scores.cpu().numpy()

    # ---- oracle, per sequence, and comparisons (every row, every layer)
    swaps, compared = 0, 0
    o_top = np.empty((len(w.layers), B, 1, k), np.int32)
    o_pool = np.empty((B, 1, nb), np.int32)
    for b in range(B):
        full = oracle_full(c, b, 0)
        ok, err = finite_close(g_scores[b, 0], full["scores"])
        assert ok, f"scores seq {b}: {err}"
        swaps += check_set(g_pool[b, 0], full["pool"], lambda i: full["block_max"][i], f"pool seq {b}")
        swaps += check_set(g_top[0][b, 0], full["topk"], lambda i: full["scores"][i], f"top-k seq {b}")
        o_top[0, b, 0], o_pool[b, 0] = full["topk"], full["pool"]
        # attention over the GPU's own (validated) selection
        ro, rl = oracle_attention(c, b, 0, 0, g_top[0][b, 0])
        assert max_abs(g_out[0][b, 0], ro) <= ATTN_TOL, f"attention seq {b}"
        compared += 1
        if "reindex" in w.layers:
            # the oracle's Reindex over the GPU's own (validated) pool
            ri = oracle.reindex_layer(c.q_idx[1][b, 0], c.w_idx[1][b, 0], c.o_kc[b], c.o_ks[b],
                                      w.n_cap, g_pool[b, 0], k)
            sc = dict(zip(ri["pool_pos"].tolist(), ri["pool_scores"].tolist()))
            swaps += check_set(g_top[1][b, 0], ri["topk"], lambda i: sc[i], f"reindex seq {b}")
            for layer in range(1, len(w.layers)):
                ro, _ = oracle_attention(c, b, 0, layer, g_top[1][b, 0])
                assert max_abs(g_out[layer][b, 0], ro) <= ATTN_TOL, f"layer {layer} seq {b}"
                compared += 1
            ri_o = oracle.reindex_layer(c.q_idx[1][b, 0], c.w_idx[1][b, 0], c.o_kc[b], c.o_ks[b],
                                        w.n_cap, full["pool"], k)
            for layer in range(1, len(w.layers)):
                o_top[layer, b, 0] = ri_o["topk"]
    assert compared == B * len(w.layers), f"{compared} rows compared"
    print(f"[case] {name}: near-tie swaps {swaps}, rows compared {compared}", flush=True)

    # ---- stage-isolated: Reindex on the oracle's pool, attention on the oracle's top-k
    if "reindex" in w.layers:
        layers.reindex_indexer(buf, d["q_idx"][1], d["w_idx"][1], d["kc"], d["ks"], d["n_vis"],
                               t(o_pool), k)
        s_top = buf.topk.cpu().numpy()
        for b in range(B):
            ri = oracle.reindex_layer(c.q_idx[1][b, 0], c.w_idx[1][b, 0], c.o_kc[b], c.o_ks[b],
                                      w.n_cap, o_pool[b, 0], k)
            sc = dict(zip(ri["pool_pos"].tolist(), ri["pool_scores"].tolist()))
            check_set(s_top[b, 0], ri["topk"], lambda i: sc[i], f"reindex stage seq {b}")
    for layer in range(len(w.layers)):
        out, lse = _attention_stage(c, d, layer, o_top[layer])
        for b in range(B):
            ro, rl = oracle_attention(c, b, 0, layer, o_top[layer, b, 0])
            err = max_abs(out[b, 0], ro)
            assert err <= ATTN_TOL, f"attention layer {layer} seq {b}: {err}"
            assert max_abs(lse[b, 0], rl) <= 1e-4


def test_prefill_chunk_causal():
    """Encoder chunked prefill (m = 2, no pool): per-query causal visibility and window."""
    w = synth.scaled(W[4], tokens=16384, chunk=256, nq=256, n_cap=8192)
    print(f"[case] prefill tokens={w.tokens} chunk={w.chunk} n_cap={w.n_cap}", flush=True)
    c = build_case(w, n_layers=1)
    d = gpu_encode(c)
    assert_encodings_equal(c, d)
    T, k = w.nq, w.k
    buf = layers.Buffers.create(1, T, w.n_cap, k, 0, w.n_win)
    layers.full_indexer(buf, d["q_idx"][0], d["w_idx"][0], d["kc"], d["ks"], d["n_vis"], d["n_blk"],
                        k, 0)
    g_top = buf.topk.cpu().numpy()[0]
    layers.attention(buf, d["q_main"][0], d["vc"], d["vs"], buf.topk, d["swa"][0], d["swa_end"])
    g_out = buf.out.cpu().numpy()[0]
    nv = w.n_visible()[0]
    o_top = np.empty((1, T, k), np.int32)
    swaps, compared = 0, 0
    for i in range(T):
        full = oracle_full(c, 0, i)
        assert full["topk"].max() < nv[i]
        swaps += check_set(g_top[i], full["topk"], lambda j: full["scores"][j], f"top-k query {i}")
        o_top[0, i] = full["topk"]
        if i % 16 == 0 or i == T - 1:  # attention over the GPU's own (validated) selection
            ro, _ = oracle_attention(c, 0, i, 0, g_top[i])
            assert max_abs(g_out[i], ro) <= ATTN_TOL, f"attention query {i}"
            compared += 1
    assert compared == len(range(0, T, 16)) + (0 if (T - 1) % 16 == 0 else 1)
    out, lse = _attention_stage(c, d, 0, o_top)
    for i in list(range(0, T, 8)) + [T - 1]:
        ro, rl = oracle_attention(c, 0, i, 0, o_top[0, i])
        assert max_abs(out[0, i], ro) <= ATTN_TOL, f"query {i}"
    print(f"[case] prefill: near-tie swaps {swaps}, rows compared end to end {compared}", flush=True)


def test_decoder_prefill_with_pool():
    """Decoder chunked prefill (m = 1): every token of the chunk builds its own pool of
    2048 blocks under its causal limit (Full) and a Reindex layer rescores that pool."""
    w = synth.scaled(W[5], tokens=40000, chunk=64, nq=64, n_cap=40000)
    print(f"[case] decoder prefill tokens={w.tokens} chunk={w.chunk} n_cap={w.n_cap}", flush=True)
    c = build_case(w)
    d = gpu_encode(c)
    assert_encodings_equal(c, d)
    T, k, nb = w.nq, w.k, w.nb
    buf = layers.Buffers.create(1, T, w.n_cap, k, nb, w.n_win)
    layers.full_indexer(buf, d["q_idx"][0], d["w_idx"][0], d["kc"], d["ks"], d["n_vis"], d["n_blk"],
                        k, nb)
    g_pool = buf.pool.cpu().numpy()[0].copy()
    g_top0 = buf.topk.cpu().numpy()[0].copy()
    layers.reindex_indexer(buf, d["q_idx"][1], d["w_idx"][1], d["kc"], d["ks"], d["n_vis"],
                           buf.pool, k)
    g_top1 = buf.topk.cpu().numpy()[0].copy()
    layers.attention(buf, d["q_main"][1], d["vc"], d["vs"], buf.topk, d["swa"][1], d["swa_end"])
    g_out1 = buf.out.cpu().numpy()[0]
    nv = w.n_visible()[0]
    swaps, compared = 0, 0
    for i in range(T):
        full = oracle_full(c, 0, i)
        assert full["topk"].max() < nv[i] and full["pool"].max() < (nv[i] + 7) // 8
        swaps += check_set(g_pool[i], full["pool"], lambda j: full["block_max"][j], f"pool {i}")
        swaps += check_set(g_top0[i], full["topk"], lambda j: full["scores"][j], f"top-k {i}")
        # the oracle's Reindex over the GPU's own (validated) pool, every token
        ri = oracle.reindex_layer(c.q_idx[1][0, i], c.w_idx[1][0, i], c.o_kc[0], c.o_ks[0],
                                  int(nv[i]), g_pool[i], k)
        sc = dict(zip(ri["pool_pos"].tolist(), ri["pool_scores"].tolist()))
        swaps += check_set(g_top1[i], ri["topk"], lambda j: sc[j], f"reindex {i}")
        if i % 8 == 0 or i == T - 1:  # attention over the GPU's own Reindex selection
            ro, _ = oracle_attention(c, 0, i, 1, g_top1[i])
            assert max_abs(g_out1[i], ro) <= ATTN_TOL, f"attention query {i}"
            compared += 1
    assert compared == len(range(0, T, 8)) + (0 if (T - 1) % 8 == 0 else 1)
    print(f"[case] decoder prefill: near-tie swaps {swaps}, rows compared {compared}", flush=True)
