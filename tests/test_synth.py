"""The seeded input generator: determinism, slice addressing and the recipe's moments."""
import numpy as np

import synth


def test_slices_regenerate_independently():
    k = synth.key(3, synth.TAG_IDX_K, 0, 5)
    whole = synth.normal_f32(k, 0, 10000)
    assert np.array_equal(whole[1234:5678], synth.normal_f32(k, 1234, 5678 - 1234))
    w = synth.WORKLOADS[3]
    a = synth.kv_rows(w, 2, 100, 50)
    b = synth.kv_rows(w, 2, 0, 200)[100:150]
    assert np.array_equal(a, b)


def test_streams_differ_by_tag_layer_and_sequence():
    base = synth.normal_f32(synth.key(1, 1, 0, 0), 0, 64)
    for args in [(1, 2, 0, 0), (1, 1, 1, 0), (1, 1, 0, 1), (2, 1, 0, 0)]:
        assert not np.array_equal(base, synth.normal_f32(synth.key(*args), 0, 64))


def test_recipe_moments():
    z = synth.normal_f32(synth.key(0, 1), 0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    u = synth.uniform_f32(synth.key(0, 7), 0, 1 << 20).astype(np.float64)
    assert 0 < u.min() and u.max() < 1 and abs(u.mean() - 0.5) < 2e-3
    w = synth.WORKLOADS[0]
    q = synth.bf16_to_f32(synth.q_idx(w, 0)).astype(np.float64)
    assert abs(q.std() * np.sqrt(128) - 1) < 0.05
    x = synth.kv_rows(synth.WORKLOADS[1], 0, 0, 2000)
    frac = (np.abs(x) > 7).mean()  # outliers at +-10 before normalisation
    assert 5e-4 < frac < 2e-3


def test_workload_visibility_and_windows():
    w = synth.WORKLOADS[4]
    nv = w.n_visible()[0]
    assert nv[0] == 63488 and nv[-1] == 65536 and np.all(np.diff(nv) >= 0)
    end = w.swa_end()[0]
    assert end[0] == 128 and end[-1] == 128 + 4095 and w.swa_rows() == 4223
    assert w.new_entries() == (63488, 2048)
    d = synth.WORKLOADS[3]
    assert d.n_visible().shape == (16, 1) and d.new_entries() == (1048575, 1)


def test_decoder_prefill_visibility():
    # m = 1: entry j is token j; token t of the chunk sees entries [0, t + 1)
    w = synth.WORKLOADS[5]
    nv = w.n_visible()[0]
    assert nv[0] == 65536 - 1024 + 1 and nv[-1] == 65536 and np.all(np.diff(nv) == 1)
    assert w.new_entries() == (64512, 1024) and w.swa_rows() == 127 + 1024
    assert w.layers == ("full", "reindex") and w.nb == 2048
