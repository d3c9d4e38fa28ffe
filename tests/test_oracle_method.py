"""Pins of the oracle's indexer, selection, pool, Reindex and attention code.

Independent references: numpy matmul / softmax / lexsort written here from the
definitions, the E2M1 table in tests/golden, torch's E4M3 decoder, closed forms
(q = 0, a single key), and the structural facts the pages state about the
hierarchical indexer (the Full layer's pool of blocks ranked by their largest
index score; Reindex scores only inside it).  CPU only.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
import synth
from conftest import e2m1_table, page_value


def decode_mxfp4(codes, scales):
    """Independent MXFP4 decoder: golden E2M1 table, torch E4M3 decoder."""
    lut = np.array([e2m1_table()[c] for c in range(16)])
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    s = torch.tensor(scales).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return lut[nib] * np.repeat(s, 16, axis=1)


def decode_fp8(b):
    return torch.tensor(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def make_keys(n, seed=0, C=128):
    x = np.random.default_rng(seed).standard_normal((n, C)).astype(np.float32)
    return oracle.quantize_rows(x)


def make_q(H, D, scale, seed):
    return synth.normal_bf16(synth.key(50, 6, 0, seed), 0, H * D, scale).reshape(H, D)


def make_w(H, seed):
    return synth.uniform_f32(synth.key(50, 7, 0, seed), 0, H)


def numpy_scores(q, w, codes, scales):
    k = decode_mxfp4(codes, scales)
    d = synth.bf16_to_f32(q).astype(np.float64) @ k.T  # [H, n]
    return (w.astype(np.float64)[:, None] * np.maximum(d, 0.0)).sum(axis=0)


def numpy_topk(s, k, idx=None):
    idx = np.arange(s.size) if idx is None else np.asarray(idx)
    keep = idx >= 0
    s, idx = np.asarray(s)[keep], idx[keep]
    order = np.lexsort((idx, -s))
    top = np.sort(idx[order[:k]])
    return np.concatenate([top, -np.ones(k - top.size, np.int64)]).astype(np.int32)


# ------------------------------------------------------------------- indexer

def test_index_scores_match_numpy_definition():
    codes, scales = make_keys(75, seed=1)
    q = make_q(32, 128, 1 / np.sqrt(128), 1)
    w = make_w(32, 1)
    got = oracle.index_scores(q, w, codes, scales, 75)
    ref = numpy_scores(q, w, codes, scales)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # and only the visible prefix is scored
    assert np.array_equal(oracle.index_scores(q, w, codes, scales, 40), got[:40])


def test_index_scores_relu_per_head_not_after_sum():
    """One head sees +d, another -d: the negative head must contribute zero."""
    k = np.zeros((1, 128), np.float32)
    k[0, :16] = 1.5  # amax / 6 = 0.25 is an E4M3 value, so the key decodes exactly
    codes, scales = oracle.quantize_rows(k)
    qf = np.zeros((2, 128), np.float32)
    qf[0, :16] = 0.5
    qf[1, :16] = -0.5
    q = (qf.view(np.uint32) >> 16).astype(np.uint16)
    s = oracle.index_scores(q, np.array([1.0, 1.0], np.float32), codes, scales, 1)
    assert s[0] == 12.0


def test_zero_query_ties_pick_lowest_indices():
    codes, scales = make_keys(300, seed=2)
    q = np.zeros((32, 128), np.uint16)
    res = oracle.full_layer(q, make_w(32, 2), codes, scales, 300, k=17, nb=5, block=8)
    assert np.all(res["scores"] == 0)
    assert np.array_equal(res["topk"], np.arange(17))
    assert np.array_equal(res["pool"], np.arange(5))


def test_weight_power_of_two_scaling_keeps_selection():
    codes, scales = make_keys(500, seed=3)
    q = make_q(32, 128, 1 / np.sqrt(128), 3)
    w = make_w(32, 3)
    a = oracle.full_layer(q, w, codes, scales, 500, k=31, nb=9)
    b = oracle.full_layer(q, w * 4, codes, scales, 500, k=31, nb=9)
    assert np.array_equal(a["topk"], b["topk"]) and np.array_equal(a["pool"], b["pool"])


def test_block_max_over_visible_entries_only():
    s = np.random.default_rng(4).standard_normal(61)
    bm = oracle.block_max(s, 8)
    assert bm.size == 8
    for b in range(8):
        assert bm[b] == s[8 * b: min(8 * b + 8, 61)].max()


# ------------------------------------------------------------------- selection

@pytest.mark.parametrize("n,k", [(1, 4), (50, 50), (200, 17), (1000, 64), (5000, 512)])
def test_select_matches_full_sort(n, k):
    rng = np.random.default_rng(n)
    s = np.round(rng.standard_normal(n), 1)  # many exact ties
    s[rng.integers(0, n, n // 10)] = 0.0
    s[rng.integers(0, n, n // 10)] = -0.0
    assert np.array_equal(oracle.select(s, k), numpy_topk(s, k))
    idx = np.arange(n, dtype=np.int32)
    idx[rng.integers(0, n, n // 7)] = -1
    assert np.array_equal(oracle.select(s, k, idx), numpy_topk(s, k, idx))


def test_full_layer_topk_and_pool_against_sort():
    codes, scales = make_keys(2048, seed=5)
    q, w = make_q(32, 128, 1 / np.sqrt(128), 5), make_w(32, 5)
    res = oracle.full_layer(q, w, codes, scales, 2043, k=64, nb=32)
    s = numpy_scores(q, w, codes[:2043], scales[:2043])
    assert np.array_equal(res["topk"], numpy_topk(s, 64))
    bm = np.array([s[8 * b: 8 * b + 8].max() for b in range(256)])
    assert np.array_equal(res["pool"], numpy_topk(bm, 32))


# ------------------------------------------------------------------- hierarchical pool

def _ties_keys(n, seed):
    """Keys with many exact duplicates so scores tie across blocks."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((n // 4, 128)).astype(np.float32)
    x = base[rng.integers(0, n // 4, n)]
    return oracle.quantize_rows(x)


@pytest.mark.parametrize("ties", [False, True])
def test_full_topk_lies_in_pool_when_pool_has_at_least_k_blocks(ties):
    """A block ranked above a winner's block holds another winner, so with nb >= k blocks
    every top-k entry is a pool position (the pages: the pool is larger than the top-k)."""
    n = 4096
    codes, scales = _ties_keys(n, 6) if ties else make_keys(n, 6)
    for seed in range(4):
        q, w = make_q(32, 128, 1 / np.sqrt(128), 10 + seed), make_w(32, 10 + seed)
        res = oracle.full_layer(q, w, codes, scales, n - seed, k=40, nb=40)
        pos = oracle.pool_positions(res["pool"], 8, n - seed)
        assert set(res["topk"].tolist()) <= set(pos.tolist())
        # Reindex with the Full layer's own query reproduces its top-k
        ri = oracle.reindex_layer(q, w, codes, scales, n - seed, res["pool"], k=40)
        assert np.array_equal(ri["topk"], res["topk"])


def test_reindex_scores_only_pool_positions():
    n = 3000
    codes, scales = make_keys(n, 7)
    q, w = make_q(32, 128, 1 / np.sqrt(128), 7), make_w(32, 7)
    full = oracle.full_layer(q, w, codes, scales, n, k=32, nb=48)
    q2, w2 = make_q(32, 128, 1 / np.sqrt(128), 8), make_w(32, 8)
    ri = oracle.reindex_layer(q2, w2, codes, scales, n, full["pool"], k=32)
    pos = oracle.pool_positions(full["pool"], 8, n)
    assert set(ri["topk"].tolist()) <= set(pos[pos >= 0].tolist())
    s_all = numpy_scores(q2, w2, codes, scales)
    ok = pos >= 0
    np.testing.assert_allclose(ri["pool_scores"][ok], s_all[pos[ok]], rtol=1e-12)
    assert np.array_equal(ri["topk"], numpy_topk(s_all[pos[ok]], 32, pos[ok]))
    # the selection differs from the full-range top-k of the same query in general
    assert not np.array_equal(ri["topk"], numpy_topk(s_all, 32))


def test_pool_positions_partial_last_block():
    pos = oracle.pool_positions(np.array([0, 3, -1], np.int32), 8, 29)
    assert pos[:8].tolist() == list(range(8))
    assert pos[8:16].tolist() == [24, 25, 26, 27, 28, -1, -1, -1]
    assert pos[16:].tolist() == [-1] * 8


def test_pool_size_matches_pages():
    assert page_value("pool_blocks") * page_value("block_positions") == page_value("pool_positions")


# ------------------------------------------------------------------- attention

def _attn_inputs(n=300, swa_rows=200, seed=11):
    w = synth.WORKLOADS[0]
    x = synth.latent_rows(synth.key(60, 2, 0, seed), synth.key(60, 3, 0, seed), 0, n, 512)
    cos, sin = synth.rope_rows(0, n)
    codes, scales = oracle.quantize_rows(x, cos, sin)
    sw = oracle.encode_fp8(synth.latent_rows(synth.key(60, 4, 0, seed), synth.key(60, 5, 0, seed),
                                             0, swa_rows, 512))
    q = make_q(64, 512, 1 / np.sqrt(512), seed)
    return q, codes, scales, sw


def numpy_attention(q, keys, scale):
    qf = synth.bf16_to_f32(q).astype(np.float64)
    logits = scale * qf @ keys.T
    p = softmax(logits, axis=1)
    return p @ keys, logsumexp(logits, axis=1)


@pytest.mark.parametrize("scale", [1.0, 0.37])
def test_attention_matches_textbook_softmax(scale):
    q, codes, scales, sw = _attn_inputs()
    sel = np.array([5, 17, 100, 299, 0, 42], np.int32)
    out, lse = oracle.attention(q, codes, scales, sel, sw, swa_end=150, n_win=128, scale=scale)
    keys = np.concatenate([decode_mxfp4(codes[sel], scales[sel]), decode_fp8(sw[22:150])])
    ro, rl = numpy_attention(q, keys, scale)
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_when_k_covers_context():
    q, codes, scales, sw = _attn_inputs(n=100)
    qi, wi = make_q(32, 128, 1 / np.sqrt(128), 3), make_w(32, 3)
    kc, ks = make_keys(100, 3)
    top = oracle.full_layer(qi, wi, kc, ks, 100, k=128, nb=0)["topk"]
    assert np.array_equal(top[:100], np.arange(100)) and np.all(top[100:] == -1)
    sparse = oracle.attention(q, codes, scales, top, sw, 128)
    dense = oracle.attention(q, codes, scales, np.arange(100, dtype=np.int32), sw, 128)
    assert np.array_equal(sparse[0], dense[0]) and np.array_equal(sparse[1], dense[1])


def test_attention_single_key_returns_it():
    q, codes, scales, sw = _attn_inputs()
    out, lse = oracle.attention(q, codes, scales, np.array([-1, 7, -1], np.int32), sw, swa_end=0)
    v = decode_mxfp4(codes[7:8], scales[7:8])[0]
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse, synth.bf16_to_f32(q).astype(np.float64) @ v, rtol=1e-12)


def test_attention_zero_query_is_mean_of_keys():
    _, codes, scales, sw = _attn_inputs()
    q = np.zeros((64, 512), np.uint16)
    sel = np.arange(10, 74, dtype=np.int32)
    out, lse = oracle.attention(q, codes, scales, sel, sw, swa_end=128)
    keys = np.concatenate([decode_mxfp4(codes[sel], scales[sel]), decode_fp8(sw[:128])])
    np.testing.assert_allclose(out, np.broadcast_to(keys.mean(0), out.shape), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(keys.shape[0]), rtol=1e-14)


def test_attention_permutation_and_padding_invariant():
    q, codes, scales, sw = _attn_inputs()
    sel = np.array([3, 9, 27, 81, 243], np.int32)
    a = oracle.attention(q, codes, scales, sel, sw, 140)
    b = oracle.attention(q, codes, scales, np.array([-1, 243, 27, -1, 3, 81, 9, 500], np.int32), sw, 140)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)


def test_attention_empty_and_window_only():
    q, codes, scales, sw = _attn_inputs()
    out, lse = oracle.attention(q, codes, scales, -np.ones(8, np.int32), sw, swa_end=0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = oracle.attention(q, codes, scales, -np.ones(8, np.int32), sw, swa_end=60)
    ro, rl = numpy_attention(q, decode_fp8(sw[0:60]), 1.0)
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, rl, rtol=1e-12)


def test_needle_entry_is_selected_and_dominates():
    """An indexer key aligned with every head's query scores highest and is selected."""
    n = 4000
    rng = np.random.default_rng(12)
    x = rng.standard_normal((n, 128)).astype(np.float32)
    q = make_q(32, 128, 1 / np.sqrt(128), 12)
    qf = synth.bf16_to_f32(q)
    x[1234] = 4.0 * qf.sum(0) / np.abs(qf.sum(0)).max()
    codes, scales = oracle.quantize_rows(x)
    res = oracle.full_layer(q, make_w(32, 12), codes, scales, n, k=8, nb=8)
    assert 1234 in res["topk"] and 1234 // 8 in res["pool"]
    assert np.argmax(res["scores"]) == 1234
