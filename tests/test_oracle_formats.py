"""Pins of the oracle's format code (decoders, encoders, rotary) against what
the pages and independent routines fix.  CPU only.

Independent references used here: torch's float8_e4m3fn conversions (a library
implementation of OCP E4M3FN with round-to-nearest-even), the E2M1 value table
in tests/golden, a brute-force nearest-grid search written with numpy, and
exact identities of the rotation.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import e2m1_table, page_value


def torch_e4m3_value(b):
    return torch.tensor(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_e4m3_encode(x_f32):
    """RNE cast of fp32 values to E4M3FN bytes (torch returns NaN above 464, no saturation)."""
    return torch.tensor(np.asarray(x_f32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_bytes_match_library():
    ref = torch_e4m3_value(np.arange(256))
    got = np.array([oracle.e4m3_decode(b) for b in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2  # only S.1111.111 is NaN in the FN variant
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_max_is_the_page_value():
    finite = [oracle.e4m3_decode(b) for b in range(127)]
    assert max(finite) == page_value("e4m3_max") == 448.0
    assert oracle.e4m3_decode(0x7E) == 448.0


def test_e2m1_decode_matches_format_table():
    table = e2m1_table()
    for code, val in table.items():
        got = oracle.e2m1_decode(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val) or (val == 0 and got == 0)
    # the format maximum quoted on the pages: 448 x 6 = 2688
    assert max(table.values()) * page_value("e4m3_max") == page_value("mxfp4_max")


def test_e4m3_encode_matches_library_rne():
    rng = np.random.default_rng(1)
    grid = np.array([oracle.e4m3_decode(b) for b in range(127)])
    mids = (grid[1:] + grid[:-1]) / 2  # exact ties between neighbouring codes
    vals = np.concatenate([
        rng.uniform(0, 464, 4000), rng.uniform(0, 0.02, 2000), 2.0 ** rng.uniform(-12, 8.7, 4000),
        grid, mids, np.nextafter(mids.astype(np.float32), 0), np.nextafter(mids.astype(np.float32), 1000),
    ]).astype(np.float32)
    vals = vals[vals < 464]
    ref = torch_e4m3_encode(vals)
    got = np.array([oracle.e4m3_encode(float(v)) for v in vals], np.uint8)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates_at_page_max():
    for v in [448.0, 463.9, 464.0, 500.0, 1e6]:
        assert oracle.e4m3_decode(oracle.e4m3_encode(v)) == page_value("e4m3_max")


# --------------------------------------------------------------------- encoder

def brute_force_encode(x):
    """Independent MXFP4 encoder: torch E4M3 cast of fp32(amax/6), then per element the
    nearest E2M1 grid value (numpy argmin over the table) with ties to the even code."""
    x = np.asarray(x, np.float32)
    R, C = x.shape
    g = x.reshape(R, C // 16, 16).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    sb = torch_e4m3_encode((amax / 6.0).astype(np.float32))  # fp32 division, then RNE
    s = torch_e4m3_value(sb)
    mags = np.array([e2m1_table()[c] for c in range(8)])
    a = np.abs(g)
    dist = np.abs(a[..., None] - mags[None, None, None, :] * s[..., None, None])
    best = np.argmin(dist, axis=-1)  # first (lower) code on ties
    # ties between code c-1 (odd) and c (even): take the even one
    dmin = dist.min(axis=-1)
    for c in range(2, 8, 2):
        tie = (dist[..., c] == dmin) & (best == c - 1)
        best = np.where(tie, c, best)
    best = np.where(s[..., None] == 0, 0, best)
    code = best | np.where((g < 0) & (best != 0), 8, 0)
    code = code.reshape(R, C).astype(np.uint8)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb.reshape(R, C // 16)


def _groups_with_ties(rng, n):
    """Rows whose elements sit exactly on E2M1 midpoints of their group's scale."""
    rows = []
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for _ in range(n):
        s_byte = rng.integers(8, 0x78)
        s = oracle.e4m3_decode(int(s_byte))
        row = rng.choice(mids, 16) * s * rng.choice([-1, 1], 16)
        row[0] = 6.0 * s  # pins amax / 6 = s exactly
        rows.append(row)
    return np.array(rows, np.float32).reshape(-1, 16)


@pytest.mark.parametrize("kind", ["latent", "normal", "ties", "tiny", "huge"])
def test_encoder_matches_brute_force(kind):
    rng = np.random.default_rng(7)
    if kind == "latent":
        x = synth.latent_rows(synth.key(99, 2), synth.key(99, 3), 0, 64, 512)
    elif kind == "normal":
        x = rng.standard_normal((64, 128)).astype(np.float32)
    elif kind == "ties":
        x = _groups_with_ties(rng, 512).reshape(-1, 128)
    elif kind == "tiny":
        x = (rng.standard_normal((16, 128)) * 1e-4).astype(np.float32)
        x[:, :16] = 0.0
        x[0, 16:32] = -0.0
    else:
        x = (rng.standard_normal((16, 128)) * 300).astype(np.float32)
    codes, scales = oracle.quantize_rows(x)
    rc, rs = brute_force_encode(x)
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def test_encoder_no_negative_zero_and_nibble_order():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6.0   # channel 0 -> low nibble of byte 0
    x[0, 1] = -3.0  # channel 1 -> high nibble of byte 0
    x[0, 2] = -1e-9  # rounds to zero: no sign
    codes, scales = oracle.quantize_rows(x)
    assert oracle.e4m3_decode(scales[0, 0]) == 1.0
    assert codes[0, 0] == (0x7 | (0xD << 4))
    assert codes[0, 1] == 0


def test_encoder_error_bound_and_roundtrip():
    x = synth.latent_rows(synth.key(98, 2), synth.key(98, 3), 0, 256, 512)
    codes, scales = oracle.quantize_rows(x)
    xh = oracle.dequant_rows(codes, scales)
    s = np.repeat(np.array([[oracle.e4m3_decode(b) for b in r] for r in scales]), 16, axis=1)
    assert np.all(np.abs(x - xh) <= s + 1e-30)
    # a group that holds a +-6 code re-encodes to itself
    c2, s2 = oracle.quantize_rows(xh.astype(np.float32))
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(256, 32, 16)
    has6 = ((nib & 7) == 7).any(axis=2)
    nib2 = np.stack([c2 & 15, c2 >> 4], axis=-1).reshape(256, 32, 16)
    assert has6.mean() > 0.5
    assert np.array_equal(nib[has6], nib2[has6])
    assert np.array_equal(scales[has6], s2[has6])


def test_sliding_window_fp8_matches_library():
    x = synth.latent_rows(synth.key(97, 4), synth.key(97, 5), 0, 32, 512)
    assert np.array_equal(oracle.encode_fp8(x), torch_e4m3_encode(x))


# --------------------------------------------------------------------- rotary

def test_rope_special_angles_and_norm():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    half = 32
    ident = oracle.quantize_rows(x, np.ones((4, half), np.float32), np.zeros((4, half), np.float32))
    assert all(np.array_equal(a, b) for a, b in zip(ident, oracle.quantize_rows(x)))
    # a quarter turn maps (a, b) -> (-b, a) exactly
    quarter = oracle.quantize_rows(x, np.zeros((4, half), np.float32), np.ones((4, half), np.float32))
    y = x.copy()
    a, b = x[:, 448::2].copy(), x[:, 449::2].copy()
    y[:, 448::2], y[:, 449::2] = -b, a
    assert all(np.array_equal(p, q) for p, q in zip(quarter, oracle.quantize_rows(y)))
    # a half turn negates the rotated dims only
    half_turn = oracle.quantize_rows(x, -np.ones((4, half), np.float32), np.zeros((4, half), np.float32))
    z = x.copy()
    z[:, 448:] = -z[:, 448:]
    assert all(np.array_equal(p, q) for p, q in zip(half_turn, oracle.quantize_rows(z)))


def test_amplitude_bound_of_pages():
    """A post-RMSNorm 512-channel latent: L2 <= sqrt(512), every channel <= ~22.6, scales far
    below the format range and never the 2688 maximum."""
    w = synth.WORKLOADS[1]
    x = synth.kv_rows(w, 0, 0, 4096)
    l2 = np.sqrt((x.astype(np.float64) ** 2).sum(axis=1))
    assert np.all(l2 <= math.sqrt(page_value("latent_l2_bound_sq")) * (1 + 1e-6))
    assert np.abs(x).max() <= page_value("latent_channel_bound") + 0.1
    # outliers of +-10 land near the observed maximum of about 10
    assert 8.0 < np.abs(x).max() <= page_value("observed_max")
    cos, sin = synth.rope_rows(0, 4096)
    codes, scales = oracle.quantize_rows(x, cos, sin)
    smax = max(oracle.e4m3_decode(b) for b in np.unique(scales))
    assert smax <= oracle.e4m3_decode(oracle.e4m3_encode(page_value("latent_channel_bound") / 6))
    xh = oracle.dequant_rows(codes[:256], scales[:256])
    assert np.abs(xh).max() <= 6 * smax < page_value("mxfp4_max")
