"""Pins of the oracle's indexer-key projection (new entries project their indexer key
from the main latent): against numpy's matrix product in double on the decoded bf16
weights, and the closed form of a channel-selection matrix (exact)."""
import numpy as np
import torch

import oracle


def _bf16(a):
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.float().numpy().astype(np.float64)


def test_projection_matches_numpy_matmul():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 512)).astype(np.float32)
    w_bits, w = _bf16(rng.standard_normal((128, 512)) / np.sqrt(512))
    y = oracle.project_rows(x, w_bits)
    ref = x.astype(np.float64) @ w.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_projection_of_a_selection_matrix_is_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    pick = rng.permutation(512)[:128]
    w = np.zeros((128, 512), np.float32)
    w[np.arange(128), pick] = 1.0
    w[::3] *= -2.0                     # signs and powers of two stay exact
    w_bits, wd = _bf16(w)
    y = oracle.project_rows(x, w_bits)
    scale = np.where(np.arange(128) % 3 == 0, -2.0, 1.0)
    assert np.array_equal(y, x[:, pick].astype(np.float64) * scale)
