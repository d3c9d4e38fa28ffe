"""Pins of the oracle's attention output epilogue (inverse rotary + bf16 cast),
against what the format definition and the mathematics fix: an independent bf16
rounding (torch's fp32 -> bfloat16 conversion, round to nearest even), constructed
ties, the closed-form quarter turn, and the round trip through the oracle's own
forward rotary (the rotation composed with its inverse is the identity)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    mags = rng.standard_normal(20000) * 10.0 ** rng.integers(-44, 38, 20000)  # incl. subnormals
    x = np.concatenate([
        mags.astype(np.float32),
        # exact ties (finite): low 16 bits 0x8000, both parities of the kept part
        (rng.integers(0, 0x7F80, 4000).astype(np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -3e-39, 3.3895e38, 3.3961e38, -3.4e38, np.inf, -np.inf],
                 np.float32),
    ])
    ref = _torch_bf16_bits(x)
    got = np.array([oracle.bf16_rne(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.bf16_rne(float("nan")) == 0x7FC0


def test_bf16_rne_ties_to_even_from_double():
    # halfway cases that no fp32 value can express exactly in fewer bits
    assert oracle.bf16_rne(1.0 + 2 ** -8) == 0x3F80           # tie -> even (down)
    assert oracle.bf16_rne(1.0 + 3 * 2 ** -8) == 0x3F82       # tie -> even (up)
    assert oracle.bf16_rne(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81  # just above the tie


def test_inverse_rotary_quarter_turn_and_passthrough():
    o = np.zeros((2, 512))
    o[:, 448], o[:, 449] = 1.5, -2.25          # a rotary pair
    o[:, 100] = 0.75                           # a plain channel
    cs = np.ones(32, np.float32)
    sn = np.zeros(32, np.float32)
    cs[0], sn[0] = 0.0, 1.0                    # quarter turn on the first pair
    bits = oracle.inverse_rope_bf16(o, cs, sn, 448, 64)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    # rotating back by +90 degrees: (a, b) -> (a*0 + b*1, b*0 - a*1) = (b, -a)
    assert vals[0, 448] == -2.25 and vals[0, 449] == -1.5
    assert vals[1, 100] == 0.75 and np.all(vals[:, :100] == 0)
    # rope_dim 0: a plain cast
    plain = oracle.inverse_rope_bf16(o, cs, sn, 448, 0)
    assert np.array_equal(plain, np.vectorize(oracle.bf16_rne, otypes=[np.uint16])(o))


def test_inverse_rotary_undoes_the_forward_rotary():
    rng = np.random.default_rng(3)
    # bf16-representable values, so the round trip's fp32 rounding stays far
    # below half a bf16 ulp and the bits come back exactly
    x = torch.from_numpy(rng.standard_normal(512).astype(np.float32)).to(torch.bfloat16).float().numpy()
    ang = rng.uniform(-np.pi, np.pi, 32)
    cs, sn = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = x.copy()
    oracle.lib().oracle_rope_row(y.ctypes.data_as(ctypes.c_void_p), cs.ctypes.data_as(ctypes.c_void_p),
                                 sn.ctypes.data_as(ctypes.c_void_p), 448, 64)
    assert not np.array_equal(y[448:], x[448:])
    bits = oracle.inverse_rope_bf16(y.astype(np.float64)[None], cs, sn, 448, 64)
    assert np.array_equal(bits[0], _torch_bf16_bits(x))
