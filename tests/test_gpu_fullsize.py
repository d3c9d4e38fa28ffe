"""Parity at the workloads' full sizes, in the launch configuration bench.py times,
on sampled outputs the oracle can compute one by one.

For each workload the whole batch is encoded and run on the GPU exactly as the
benchmark does; the oracle then re-encodes the sampled sequences from the same
seeded rows (asserting the GPU caches of those sequences are bit-identical) and
runs the Full / Reindex / Reuse steps for the sampled query rows.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_harness import ATTN_TOL, check_set, max_abs, seq_keys, t

pytestmark = pytest.mark.gpu

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
L = kv._lib
layers = kv.layers


def _oracle_caches(w, b, n_layers):
    cos, sin = synth.rope_rows(0, w.n_cap)
    kc, ks = oracle.quantize_rows(synth.idx_k_rows(w, b, 0, w.n_cap))
    vc, vs = oracle.quantize_rows(synth.kv_rows(w, b, 0, w.n_cap), cos, sin,
                                  synth.ROPE_OFFSET, synth.ROPE_DIM)
    sw = [oracle.encode_fp8(synth.swa_rows(w, layer, b, 0, w.swa_rows())) for layer in range(n_layers)]
    return kc, ks, vc, vs, sw


def _run(w, sample_seqs, sample_queries=None):
    print(f"[fullsize] {w.name}: building caches", flush=True)
    st = bench.build_device(w, torch, L)
    step, _ = bench.make_step(st, torch, L, layers)
    buf = st["buf"]
    n_blk = layers.n_valid_blocks(st["n_vis"])
    # Full layer of the benchmark step, keeping the Full top-k and pool
    layers.full_indexer(buf, st["q_idx"][0], st["w_idx"][0], st["kc"], st["ks"], st["n_vis"], n_blk,
                        w.k, w.nb)
    g_pool = buf.pool.cpu().numpy().copy() if buf.pool is not None else None
    g_top = [buf.topk.cpu().numpy().copy()]
    layers.attention(buf, st["q_main"][0], st["vc"], st["vs"], buf.topk, st["swa"][0],
                     st["swa_end"], w.n_win)
    g_out = [buf.out.cpu().numpy().copy()]
    if "reindex" in w.layers:
        layers.reindex_indexer(buf, st["q_idx"][1], st["w_idx"][1], st["kc"], st["ks"], st["n_vis"],
                               buf.pool, w.k)
        g_top.append(buf.topk.cpu().numpy().copy())
        for layer in range(1, len(w.layers)):
            layers.attention(buf, st["q_main"][layer], st["vc"], st["vs"], buf.topk, st["swa"][layer],
                             st["swa_end"], w.n_win)
            g_out.append(buf.out.cpu().numpy().copy())
    torch.cuda.synchronize()

    nv, se = w.n_visible(), w.swa_end()
    qi = [synth.q_idx(w, layer) for layer in range(len(w.layers))]
    wi = [synth.w_idx(w, layer) for layer in range(len(w.layers))]
    qm = [synth.q_main(w, layer) for layer in range(len(w.layers))]
    swaps = 0
    for b in sample_seqs:
        print(f"[fullsize] oracle for sequence {b}", flush=True)
        kc, ks, vc, vs, sw = _oracle_caches(w, b, len(w.layers))
        assert np.array_equal(seq_keys(st["kc"], b, w.n_cap), kc), f"indexer codes of sequence {b}"
        assert np.array_equal(st["ks"][b].cpu().numpy(), ks)
        assert np.array_equal(st["vc"][b].cpu().numpy(), vc), f"main KV codes of sequence {b}"
        assert np.array_equal(st["vs"][b].cpu().numpy(), vs)
        for layer in range(len(w.layers)):
            assert np.array_equal(st["swa"][layer][b].cpu().numpy(), sw[layer])
        queries = range(w.nq) if sample_queries is None else sample_queries
        for i in queries:
            full = oracle.full_layer(qi[0][b, i], wi[0][b, i], kc, ks, int(nv[b, i]), w.k, w.nb, w.block)
            swaps += check_set(g_top[0][b, i], full["topk"], lambda j: full["scores"][j],
                               f"top-k ({b},{i})")
            if w.nb:
                swaps += check_set(g_pool[b, i], full["pool"], lambda j: full["block_max"][j],
                                   f"pool ({b},{i})")
            if np.array_equal(g_top[0][b, i], full["topk"]):
                ro, _ = oracle.attention(qm[0][b, i], vc, vs, full["topk"], sw[0], int(se[b, i]),
                                         w.n_win, 1.0)
                err = max_abs(g_out[0][b, i], ro)
                assert err <= ATTN_TOL, f"attention ({b},{i}): {err}"
            if "reindex" in w.layers and np.array_equal(g_pool[b, i], full["pool"]):
                ri = oracle.reindex_layer(qi[1][b, i], wi[1][b, i], kc, ks, int(nv[b, i]),
                                          full["pool"], w.k)
                sc = dict(zip(ri["pool_pos"].tolist(), ri["pool_scores"].tolist()))
                swaps += check_set(g_top[1][b, i], ri["topk"], lambda j: sc[j], f"reindex ({b},{i})")
                if np.array_equal(g_top[1][b, i], ri["topk"]):
                    for layer in range(1, len(w.layers)):
                        ro, _ = oracle.attention(qm[layer][b, i], vc, vs, ri["topk"], sw[layer],
                                                 int(se[b, i]), w.n_win, 1.0)
                        err = max_abs(g_out[layer][b, i], ro)
                        assert err <= ATTN_TOL, f"attention layer {layer} ({b},{i}): {err}"
    print(f"[fullsize] {w.name}: near-tie swaps {swaps}", flush=True)
    # the timed step itself runs on the same buffers and reproduces the Full top-k
    step()
    torch.cuda.synchronize()
    assert np.array_equal(buf.topk.cpu().numpy(), g_top[-1])
    del st
    torch.cuda.empty_cache()


def test_fullsize_cfg3_1m_decode():
    _run(synth.WORKLOADS[3], sample_seqs=[0, 15])


def test_fullsize_cfg1_64k_decode():
    _run(synth.WORKLOADS[1], sample_seqs=[0, 37, 63])


def test_fullsize_cfg2_group_of_four():
    _run(synth.WORKLOADS[2], sample_seqs=[0, 127])


def test_fullsize_cfg4_prefill():
    _run(synth.WORKLOADS[4], sample_seqs=[0],
         sample_queries=list(range(0, 4096, 256)) + [1, 2047, 4095])


def test_fullsize_cfg5_decoder_prefill_with_pool():
    _run(synth.WORKLOADS[5], sample_seqs=[0], sample_queries=[0, 1, 511, 1023])
