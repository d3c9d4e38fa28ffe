"""Stage-by-stage parity of the GPU library (through the C ABI) with the oracle.

Each stage gets inputs from `synth` or from the oracle, never from another GPU
stage, so a failure names one kernel.  Bars: bit-exact for codes, scales and
selected indices; near-tie-tolerant for selections made from float scores;
2e-3 max-abs for attention outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_harness import (ATTN_TOL, cdiv, check_set, dev, finite_close, max_abs, t, tile_keys,
                         untile_keys)

pytestmark = pytest.mark.gpu

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
L = kv._lib


def _ties_rows(rng, rows, C):
    """Groups whose elements sit exactly on E2M1 midpoints of their scale, plus
    groups whose amax/6 sits exactly on E4M3 midpoints."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    out = np.empty((rows, C), np.float32)
    for r in range(rows):
        for g in range(C // 16):
            sb = int(rng.integers(1, 0x7E))
            s = oracle.e4m3_decode(sb)
            if rng.random() < 0.5:
                grp = rng.choice(mids, 16) * s * rng.choice([-1, 1], 16)
                grp[rng.integers(16)] = 6.0 * s
            else:
                s2 = oracle.e4m3_decode(sb + 1)
                grp = rng.uniform(-1, 1, 16) * 3 * (s + s2)
                grp[rng.integers(16)] = 3.0 * (s + s2)  # amax / 6 = midpoint of two scales
            out[r, 16 * g:16 * g + 16] = grp
    return out


@pytest.mark.parametrize("kind", ["latent_rope", "normal_index", "ties", "extremes"])
def test_quantize_kv_bit_exact(kind):
    rng = np.random.default_rng(5)
    rows = 1031  # ragged
    cos = sin = None
    if kind == "latent_rope":
        x = synth.latent_rows(synth.key(7, 2), synth.key(7, 3), 0, rows, 512)
        cos, sin = synth.rope_rows(100000, rows)
    elif kind == "normal_index":
        x = rng.standard_normal((rows, 128)).astype(np.float32)
    elif kind == "ties":
        x = _ties_rows(rng, 64, 512)
    else:
        x = np.concatenate([
            rng.standard_normal((16, 128)) * 1e-5, rng.standard_normal((16, 128)) * 2000,
            np.zeros((4, 128)), -np.zeros((4, 128)), rng.standard_normal((8, 128)) * 1e-40,
        ]).astype(np.float32)
    C = x.shape[1]
    # 128 channels: the indexer-key cache's tiled code layout
    codes = (L.key_codes_empty(x.shape[0], device=dev()) if C == 128 else
             torch.empty(x.shape[0], C // 2, dtype=torch.uint8, device=dev()))
    scales = torch.empty(x.shape[0], C // 16, dtype=torch.uint8, device=dev())
    if cos is None:
        L.quantize_kv(t(x), codes, scales)
        ref = oracle.quantize_rows(x)
    else:
        L.quantize_kv(t(x), codes, scales, t(cos), t(sin), 448, 64)
        ref = oracle.quantize_rows(x, cos, sin, 448, 64)
    got = untile_keys(codes, x.shape[0]) if C == 128 else codes.cpu().numpy()
    assert np.array_equal(got, ref[0])
    assert np.array_equal(scales.cpu().numpy(), ref[1])


def test_quantize_kv_key_tiles_strided_rows():
    """Indexer-key rows at rows dst_row + r*dst_stride of a tiled code array: every
    row lands in its tile slot and nothing else is written."""
    rng = np.random.default_rng(9)
    R, row0, stride, cap = 23, 5, 3, 100
    x = rng.standard_normal((R, 128)).astype(np.float32)
    codes = torch.full((L.key_code_bytes(cap),), 0x5A, dtype=torch.uint8, device=dev())
    scales = torch.full((cap, 8), 0x5A, dtype=torch.uint8, device=dev())
    L.quantize_kv(t(x), codes, scales, dst_row=row0, dst_stride=stride)
    rc, rs = oracle.quantize_rows(x)
    rows = row0 + stride * np.arange(R)
    got_c = untile_keys(codes, L.key_code_bytes(cap) // 64)
    got_s = scales.cpu().numpy()
    assert np.array_equal(got_c[rows], rc) and np.array_equal(got_s[rows], rs)
    other = np.setdiff1d(np.arange(got_c.shape[0]), rows)
    assert np.all(got_c[other] == 0x5A)
    assert np.all(got_s[np.setdiff1d(np.arange(cap), rows)] == 0x5A)
    # the tiled placement itself: entry f, byte j at (f//32)*2048 + (j//16)*512 + (f%32)*16 + j%16
    raw = codes.cpu().numpy()
    f, j = rows[7], 37
    assert raw[(f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16] == rc[7, j]


def _rotary_tie_rows(n, seed=21):
    """Rows whose rotated pair lands exactly on a rounding tie when each product and
    difference is rounded on its own (as the encoder defines), but one ulp away when
    a*c - b*s is evaluated as a fused multiply-add: half of them make the group
    maximum 6x an E4M3 midpoint (a scale tie), half put an element on an E2M1
    midpoint of the group scale (an element tie)."""
    f32 = np.float32
    rng = np.random.default_rng(seed)
    rows = np.zeros((n, 512), np.float32)
    cos = np.ones((n, 32), np.float32)
    sin = np.zeros((n, 32), np.float32)
    rows[:, :448] = rng.standard_normal((n, 448)).astype(np.float32) * 0.1
    r = 0
    while r < n:
        scale_tie = r % 2 == 0
        m = int(rng.integers(24, 70))
        if scale_tie:
            target = f32(6 * (oracle.e4m3_decode(m) + oracle.e4m3_decode(m + 1)) / 2)
        else:
            s = oracle.e4m3_decode(m)
            target = f32(rng.choice([0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * s)
        ang = rng.uniform(0, 2 * np.pi)
        c, s_ = f32(np.cos(ang)), f32(np.sin(ang))
        b = f32(rng.uniform(-0.5, 0.5) * target)
        bs = f32(b * s_)
        a0 = f32((np.float64(target) + np.float64(bs)) / np.float64(c))
        for a in [a0, *[np.nextafter(a0, f32(d * np.inf)) for d in (1, -1)]]:
            a = f32(a)
            sep = f32(f32(a * c) - bs)
            fused = f32(np.float64(a) * np.float64(c) - np.float64(bs))
            other = abs(f32(f32(a * s_) + f32(b * c)))
            if sep == target and fused != target and other < target:
                rows[r, 448], rows[r, 449] = a, b
                cos[r, 0], sin[r, 0] = c, s_
                if not scale_tie:  # pair 1 (identity rotation) carries the group max 6*s
                    rows[r, 450], rows[r, 451] = f32(6 * oracle.e4m3_decode(m)), 0.0
                rows[r, 452:464] = rng.uniform(-0.1, 0.1, 12) * target
                r += 1
                break
    return rows, cos, sin


def test_quantize_kv_rotary_rounds_each_operation():
    x, cos, sin = _rotary_tie_rows(256)
    codes = torch.empty(256, 256, dtype=torch.uint8, device=dev())
    scales = torch.empty(256, 32, dtype=torch.uint8, device=dev())
    L.quantize_kv(t(x), codes, scales, t(cos), t(sin), 448, 64)
    ref = oracle.quantize_rows(x, cos, sin, 448, 64)
    assert np.array_equal(scales.cpu().numpy(), ref[1])
    assert np.array_equal(codes.cpu().numpy(), ref[0])


def test_quantize_kv_strided_append():
    """One new row per sequence written into a [B, n_cap] cache (dst_stride = n_cap)."""
    B, n_cap = 5, 37
    x = synth.latent_rows(synth.key(8, 2), synth.key(8, 3), 0, B, 512)
    cos, sin = synth.rope_rows(36, B)
    codes = torch.zeros(B, n_cap, 256, dtype=torch.uint8, device=dev())
    scales = torch.zeros(B, n_cap, 32, dtype=torch.uint8, device=dev())
    xd, cd, sd = t(x), t(cos), t(sin)
    # rows go to row n_cap-1 of every sequence: dst_row n_cap-1, stride n_cap
    st = L.load().csa2_quantize_kv(xd.data_ptr(), B, 512, cd.data_ptr(), sd.data_ptr(), 448, 64,
                                   codes.data_ptr(), scales.data_ptr(), n_cap - 1, n_cap,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows(x, cos, sin, 448, 64)
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(c[:, n_cap - 1], rc) and np.array_equal(s[:, n_cap - 1], rs)
    assert not c[:, :n_cap - 1].any() and not s[:, :n_cap - 1].any()


def test_quantize_swa_bit_exact():
    rng = np.random.default_rng(6)
    grid = np.array([oracle.e4m3_decode(b) for b in range(127)])
    mids = (grid[1:] + grid[:-1]) / 2
    x = np.concatenate([
        synth.latent_rows(synth.key(9, 4), synth.key(9, 5), 0, 20, 512).ravel(),
        mids, -mids, grid, [500.0, -1e6, 1e-30, -1e-30, 0.0, -0.0],
        rng.standard_normal(4096) * 100,
    ]).astype(np.float32)
    x = np.concatenate([x, np.zeros((-x.size) % 512, np.float32)]).reshape(-1, 512)
    out = torch.empty(x.shape, dtype=torch.uint8, device=dev())
    L.quantize_swa(t(x), out)
    assert np.array_equal(out.cpu().numpy(), oracle.encode_fp8(x))


# ------------------------------------------------------------------ top-k

def _topk_case(rng, rows, Lr, kind, k=1):
    if kind == "ties":
        s = np.round(rng.standard_normal((rows, Lr)), 1).astype(np.float32)
    elif kind == "allequal":
        s = np.zeros((rows, Lr), np.float32)
    else:
        s = rng.standard_normal((rows, Lr)).astype(np.float32) * 10
        if kind == "near_ties":
            # eight equal scores straddling rank k-1 of the full row: the bin that
            # holds the k-th key is small but not all of its equal keys are taken
            for r in range(rows):
                o = np.argsort(-s[r], kind="stable")
                a = max(0, min(k, Lr) - 4)
                s[r, o[a:a + 8]] = s[r, o[a]]
    s[:, ::97] = -0.0
    s[:, 5::211] = np.nan
    s[:, 7::301] = -np.inf
    return s


@pytest.mark.parametrize("Lr,k", [(1, 1), (100, 7), (2048, 64), (4096, 512), (4097, 2048),
                                  (8192, 512), (8193, 512), (16384, 2048), (16385, 512),
                                  (40000, 512), (131072, 2048), (131072, 512), (300000, 512), (300000, 2048),
                                  (50000, 6000)])
@pytest.mark.parametrize("kind", ["random", "ties", "near_ties"])
def test_topk_bit_exact(Lr, k, kind):
    rng = np.random.default_rng(Lr + k)
    rows = 3
    s = _topk_case(rng, rows, Lr, kind, k)
    n_valid = np.array([Lr, max(0, Lr - 13), min(Lr, k // 2)], np.int32)
    out = torch.empty(rows, k, dtype=torch.int32, device=dev())
    ws_n = L.topk_workspace(Lr, rows, k)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev())
    L.topk(t(s), k, out, n_valid=t(n_valid), ws=ws)
    got = out.cpu().numpy()
    for r in range(rows):
        idx = np.arange(Lr, dtype=np.int32)
        idx[np.isnan(s[r])] = -1
        idx[n_valid[r]:] = -1
        ref = oracle.select(s[r].astype(np.float64), k, idx)
        assert np.array_equal(got[r], ref), f"row {r}"


def test_topk_of_the_longest_row():
    """csa2_topk at its limit, one row of 2^31 - 1 keys (8 GiB; positions up to 2^31 - 2
    pass through four levels of segment candidates): 512 planted keys above every other
    key, at positions including the first and the last, are exactly the selection, in
    position order.  The other keys are seeded uniform in [0, 1), the planted ones
    2 + i; a valid prefix one short of the row leaves the last planted key out."""
    Lr, k = (1 << 31) - 1, 512
    print(f"[case] top-{k} of one row of {Lr} keys", flush=True)
    g = torch.Generator(device=dev())
    g.manual_seed(31)
    sc = torch.empty(Lr, device=dev())
    for o in range(0, Lr, 1 << 28):
        sc[o:o + (1 << 28)].uniform_(0.0, 1.0, generator=g)
    rng = np.random.default_rng(31)
    pos = np.unique(np.concatenate([[0, Lr - 1, (1 << 30), (1 << 31) - 16384],
                                    rng.integers(1, Lr - 1, 600)]))[:k]
    pos[-1] = Lr - 1
    pos = np.unique(pos)
    assert pos.size == k
    sc[t(pos.astype(np.int64))] = t(2.0 + np.arange(k, dtype=np.float32))
    ws = torch.empty(L.topk_workspace(Lr, 1, k), dtype=torch.uint8, device=dev())
    out = torch.full((1, k), -7, dtype=torch.int32, device=dev())
    L.topk(sc[None], k, out, ws=ws)
    assert np.array_equal(out.cpu().numpy()[0], pos), "top-k of the full row"
    # valid prefix Lr - 1: the last planted key is out, the best unplanted key comes in
    nv = t(np.array([Lr - 1], np.int32))
    L.topk(sc[None], k, out, n_valid=nv, ws=ws)
    got = out.cpu().numpy()[0]
    best = int(torch.argmax(torch.where(sc < 2.0, sc, torch.zeros((), device=dev()))[:Lr - 1]))
    assert np.array_equal(got, np.sort(np.concatenate([pos[:-1], [best]]))), "top-k of the prefix"
    del sc, ws
    torch.cuda.empty_cache()


def test_topk_with_index_array_and_all_equal():
    rng = np.random.default_rng(9)
    rows, Lr, k = 2, 16384, 512
    s = _topk_case(rng, rows, Lr, "allequal")
    idx = np.tile(np.arange(0, 3 * Lr, 3, dtype=np.int32), (rows, 1))
    idx[:, 100:200] = -1
    out = torch.empty(rows, k, dtype=torch.int32, device=dev())
    L.topk(t(s), k, out, idx=t(idx))
    for r in range(rows):
        ref = oracle.select(s[r].astype(np.float64), k, np.where(np.isnan(s[r]), -1, idx[r]))
        assert np.array_equal(out.cpu().numpy()[r], ref)


# ------------------------------------------------------------------ indexer

def _index_case(B=3, N=5003, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, N, 128)).astype(np.float32)
    enc = [oracle.quantize_rows(x[b]) for b in range(B)]
    kc = np.stack([e[0] for e in enc])
    ks = np.stack([e[1] for e in enc])
    q = np.stack([synth.normal_bf16(synth.key(11, 6, 0, b), 0, 4096, 1 / np.sqrt(128))
                  for b in range(B)]).reshape(B, 1, 32, 128)
    w = np.stack([synth.uniform_f32(synth.key(11, 7, 0, b), 0, 32) for b in range(B)]).reshape(B, 1, 32)
    nv = np.array([[N], [N - 777], [1]], np.int32)[:B]
    return x, kc, ks, q, w, nv


def test_index_full_scores_and_block_max_match_oracle():
    x, kc, ks, q, w, nv = _index_case()
    B, N = kc.shape[0], kc.shape[1]
    nblk = cdiv(N, 8)
    bm = torch.full((B, 1, nblk), 12345.0, device=dev())
    sc = torch.full((B, 1, N), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), t(tile_keys(kc)), t(ks), t(nv), bm, sc)
    bm, sc = bm.cpu().numpy(), sc.cpu().numpy()
    for b in range(B):
        n = int(nv[b, 0])
        ref = oracle.index_scores(q[b, 0], w[b, 0], kc[b], ks[b], n)
        ok, err = finite_close(sc[b, 0, :n], ref)
        assert ok, f"scores seq {b}: max err {err}"
        rb = oracle.block_max(ref, 8)
        ok, err = finite_close(bm[b, 0, :rb.size], rb)
        assert ok, f"block max seq {b}: max err {err}"
        assert np.all(sc[b, 0, n:] == 12345.0) and np.all(bm[b, 0, rb.size:] == 12345.0)


def test_index_full_long_chunks_ragged_rows():
    """512 query rows of one sequence: the launch picks the longest chunk per
    workgroup; visible lengths straddle chunk, prefetch-round and block edges."""
    N, nq = 20000, 512
    rng = np.random.default_rng(4)
    x = rng.standard_normal((N, 128)).astype(np.float32)
    kc, ks = oracle.quantize_rows(x)
    q = synth.normal_bf16(synth.key(11, 8, 0, 0), 0, nq * 4096, 1 / np.sqrt(128)).reshape(1, nq, 32, 128)
    w = synth.uniform_f32(synth.key(11, 9, 0, 0), 0, nq * 32).reshape(1, nq, 32)
    edges = [1, 7, 8, 9, 511, 512, 513, 16383, 16384, 16385, 19999, 20000, 0, -3, 30000]
    nv = rng.integers(1, N + 1, (1, nq)).astype(np.int32)
    nv[0, :len(edges)] = edges
    nblk = cdiv(N, 8)
    bm = torch.full((1, nq, nblk), 12345.0, device=dev())
    sc = torch.full((1, nq, N), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), t(tile_keys(kc)), t(ks[None]), t(nv), bm, sc)
    bm2 = torch.full((1, nq, nblk), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), t(tile_keys(kc)), t(ks[None]), t(nv), bm2)
    bm, sc, bm2 = bm.cpu().numpy()[0], sc.cpu().numpy()[0], bm2.cpu().numpy()[0]
    assert np.array_equal(bm, bm2)  # with and without the score output
    for i in list(range(len(edges))) + [100, 311, 511]:
        n = int(min(max(nv[0, i], 0), N))
        ref = oracle.index_scores(q[0, i], w[0, i], kc, ks, n)
        ok, err = finite_close(sc[i, :n], ref)
        assert ok, f"row {i} (n_visible {nv[0, i]}): max err {err}"
        rb = oracle.block_max(ref, 8)
        ok, err = finite_close(bm[i, :rb.size], rb)
        assert ok, f"block max row {i}: max err {err}"
        assert np.all(sc[i, n:] == 12345.0) and np.all(bm[i, rb.size:] == 12345.0)


def test_index_full_at_the_largest_sequence():
    """The scan at its limit: one sequence of 2^30 entries (64 GiB of key codes, 8 GiB of
    scales), so its addresses pass 2^32 bytes.  Every key byte is seeded random (any
    code, any finite E4M3 scale) except the last 40 entries, which csa2_quantize_kv
    writes from known rows (bytes against the oracle's encoding); the scores and block
    maxima of key tiles at the start,
    the middle and the end, and of sampled tiles, against the oracle's; then the
    multi-row form over the same cache."""
    N = 1 << 30
    print(f"[case] scan of one sequence of {N} entries", flush=True)
    g = torch.Generator(device=dev())
    g.manual_seed(30)
    kc = torch.empty(N * 64, dtype=torch.uint8, device=dev())
    ks = torch.empty((1, N, 8), dtype=torch.uint8, device=dev())
    part = 1 << 30  # bytes per fill: every fill launch stays below 2^31 elements
    for o in range(0, kc.numel(), part):
        kc[o:o + part].random_(0, 256, generator=g)
    for o in range(0, N, part // 8):
        sl = ks[0, o:o + part // 8]
        sl.random_(0, 256, generator=g)
        sl.bitwise_and_(0x77).bitwise_or_(0x30)  # finite E4M3 scales
    # the writer at the top of the cache: 40 rows (across the last key-tile boundary)
    # encoded by csa2_quantize_kv into the last 40 entries, byte-exact against the oracle
    xr = np.random.default_rng(31).standard_normal((40, 128)).astype(np.float32)
    L.quantize_kv(t(xr), kc, ks.view(-1), dst_row=N - 40)
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows(xr)
    assert np.array_equal(untile_keys(kc[(N // 32 - 2) * 2048:], 64)[24:], rc)
    assert np.array_equal(ks[0, N - 40:].cpu().numpy(), rs)
    q = synth.normal_bf16(synth.key(11, 30, 0, 0), 0, 4096, 1 / np.sqrt(128)).reshape(1, 1, 32, 128)
    w = synth.uniform_f32(synth.key(11, 31, 0, 0), 0, 32).reshape(1, 1, 32)
    bm = torch.full((1, 1, N // 8), 12345.0, device=dev())
    sc = torch.full((1, 1, N), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), kc, ks, t(np.array([[N]], np.int32)), bm, sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(30)
    n_tiles = N // 32
    tiles = [0, 1, n_tiles // 2, n_tiles - 2, n_tiles - 1] + rng.integers(0, n_tiles, 11).tolist()
    for tl in tiles:
        codes = untile_keys(kc[tl * 2048:(tl + 1) * 2048], 32)
        scales = ks[0, 32 * tl:32 * tl + 32].cpu().numpy()
        ref = oracle.index_scores(q[0, 0], w[0, 0], codes, scales, 32)
        ok, err = finite_close(sc[0, 0, 32 * tl:32 * tl + 32].cpu().numpy(), ref)
        assert ok, f"scores of tile {tl}: max err {err}"
        ok, err = finite_close(bm[0, 0, 4 * tl:4 * tl + 4].cpu().numpy(), oracle.block_max(ref, 8))
        assert ok, f"block maxima of tile {tl}: max err {err}"
    # two query rows of the sequence take the multi-row scan: row 0 (the same query)
    # gives the one-row scan's block maxima bit for bit, row 1 (its own query, visible
    # up to N - 12345) the oracle's on sampled tiles and its edge tile, and nothing
    # past its visible blocks
    print("[case] multi-row scan of the same sequence", flush=True)
    n1 = N - 12345
    q1 = synth.normal_bf16(synth.key(11, 32, 0, 0), 0, 4096, 1 / np.sqrt(128)).reshape(32, 128)
    w1 = synth.uniform_f32(synth.key(11, 33, 0, 0), 0, 32)
    q2 = np.stack([q[0, 0], q1])[None]
    w2 = np.stack([w[0, 0], w1])[None]
    bm2 = torch.full((1, 2, N // 8), 12345.0, device=dev())
    L.index_full(t(q2, torch.uint16), t(w2), kc, ks, t(np.array([[N, n1]], np.int32)), bm2)
    torch.cuda.synchronize()
    assert torch.equal(bm2[0, 0], bm[0, 0]), "multi-row block maxima differ from the one-row scan's"
    edge = (n1 - 1) // 32
    for tl in tiles + [edge]:
        if tl > edge:
            continue
        nv = min(32, n1 - 32 * tl)
        codes = untile_keys(kc[tl * 2048:(tl + 1) * 2048], 32)[:nv]
        scales = ks[0, 32 * tl:32 * tl + nv].cpu().numpy()
        rb = oracle.block_max(oracle.index_scores(q1, w1, codes, scales, nv), 8)
        ok, err = finite_close(bm2[0, 1, 4 * tl:4 * tl + rb.size].cpu().numpy(), rb)
        assert ok, f"row 1 block maxima of tile {tl}: max err {err}"
    assert bool((bm2[0, 1, (n1 + 7) // 8:] == 12345.0).all()), "row 1 wrote past its visible blocks"
    del kc, ks, bm, sc, bm2
    torch.cuda.empty_cache()


def test_index_pool_scores_bit_identical_to_scan():
    x, kc, ks, q, w, nv = _index_case(seed=1)
    B, N = kc.shape[0], kc.shape[1]
    sc = torch.zeros((B, 1, N), device=dev())
    bm = torch.zeros((B, 1, cdiv(N, 8)), device=dev())
    L.index_full(t(q, torch.uint16), t(w), t(tile_keys(kc)), t(ks), t(nv), bm, sc)
    rng = np.random.default_rng(2)
    nb = 300
    blocks = np.sort(rng.choice(cdiv(N, 8), (B, 1, nb), replace=True), axis=-1).astype(np.int32)
    blocks[:, :, -5:] = -1
    blocks[0, 0, -6] = cdiv(N, 8) - 1  # partial last block
    ps = torch.empty(B, 1, nb * 8, device=dev())
    pi = torch.empty(B, 1, nb * 8, dtype=torch.int32, device=dev())
    L.index_pool(t(q, torch.uint16), t(w), t(tile_keys(kc)), t(ks), t(blocks), t(nv), ps, pi)
    ps, pi, sc = ps.cpu().numpy(), pi.cpu().numpy(), sc.cpu().numpy()
    for b in range(B):
        pos = oracle.pool_positions(blocks[b, 0], 8, int(nv[b, 0]))
        assert np.array_equal(pi[b, 0], pos)
        ok = pos >= 0
        assert np.array_equal(ps[b, 0][ok], sc[b, 0][pos[ok]])  # bitwise equal
        assert np.all(np.isneginf(ps[b, 0][~ok]))


@pytest.mark.parametrize("B,nq", [(1, 5), (2, 5), (1, 11)])
def test_multirow_scan_bit_identical_to_one_row_scan_and_pool(B, nq):
    """Several query rows of one sequence take the multi-row scan (8 rows per workgroup,
    one dequantisation per key tile, shared through LDS): every score and block maximum
    must equal, bit for bit, the one-row scan of the same row and the pool scan of the
    same positions; 5 or 11 rows leave slots of a row group empty, rows see different
    causal lengths (0 to all 5003 entries, over two 4096-entry chunks), and with two
    sequences the second starts inside a key tile."""
    N = 5003
    rng = np.random.default_rng(6)
    x = rng.standard_normal((B, N, 128)).astype(np.float32)
    enc = [oracle.quantize_rows(x[b]) for b in range(B)]
    kc = np.stack([e[0] for e in enc])
    ks = np.stack([e[1] for e in enc])
    kct, kst = t(tile_keys(kc)), t(ks)
    q = synth.normal_bf16(synth.key(11, 10, 0, 0), 0, B * nq * 4096, 1 / np.sqrt(128)).reshape(B, nq, 32, 128)
    w = synth.uniform_f32(synth.key(11, 11, 0, 0), 0, B * nq * 32).reshape(B, nq, 32)
    nv = np.array([[N, N - 1, 700, 0, 4099], [4097, N, 1, 33, N - 31]], np.int32)[:B]
    if nq > 5:
        extra = np.array([[4096, 4095, 31, 32, 2048, N]], np.int32)[:, :nq - 5]
        nv = np.concatenate([nv, np.repeat(extra, B, axis=0)], axis=1)
    nblk = cdiv(N, 8)
    sc = torch.full((B, nq, N), 12345.0, device=dev())
    bm = torch.full((B, nq, nblk), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), kct, kst, t(nv), bm, sc)
    sc, bm = sc.cpu().numpy(), bm.cpu().numpy()
    blocks = np.sort(np.stack([[rng.choice(nblk, 64, replace=False) for _ in range(nq)]
                               for _ in range(B)]), axis=-1).astype(np.int32)
    ps = torch.empty(B, nq, 64 * 8, device=dev())
    pi = torch.empty(B, nq, 64 * 8, dtype=torch.int32, device=dev())
    L.index_pool(t(q, torch.uint16), t(w), kct, kst, t(blocks), t(nv), ps, pi)
    ps, pi = ps.cpu().numpy(), pi.cpu().numpy()
    for b in range(B):
        for i in range(nq):
            n = int(nv[b, i])
            # the same row through the one-row scan: a one-row batch per sequence
            qb = np.zeros((B, 1, 32, 128), np.uint16)
            wb = np.zeros((B, 1, 32), np.float32)
            nb1 = np.zeros((B, 1), np.int32)
            qb[b, 0], wb[b, 0], nb1[b, 0] = q[b, i], w[b, i], n
            s1 = torch.full((B, 1, N), 12345.0, device=dev())
            b1 = torch.full((B, 1, nblk), 12345.0, device=dev())
            L.index_full(t(qb, torch.uint16), t(wb), kct, kst, t(nb1), b1, s1)
            assert np.array_equal(sc[b, i], s1.cpu().numpy()[b, 0]), f"seq {b} row {i}: scores"
            assert np.array_equal(bm[b, i], b1.cpu().numpy()[b, 0]), f"seq {b} row {i}: maxima"
            if n:
                ref = oracle.index_scores(q[b, i], w[b, i], kc[b], ks[b], n)
                ok, err = finite_close(sc[b, i, :n], ref)
                assert ok, f"seq {b} row {i}: max err {err}"
            ok = pi[b, i] >= 0
            assert np.array_equal(pi[b, i], oracle.pool_positions(blocks[b, i], 8, n))
            assert np.array_equal(ps[b, i][ok], sc[b, i][pi[b, i][ok]])


@pytest.mark.parametrize("nv", [[20, 7], [64, 40], [96, 1], [33, 0]])
def test_multirow_scan_short_row_groups(nv):
    """Row groups whose longest row covers 1, 2 or 3 key tiles (the multi-row scan pads
    its tile loop to whole prefetch rounds: the padded tile and the epilogue of the tile
    before the first must write nothing): scores and block maxima equal the one-row scan
    bit for bit, entries past each row's end keep the sentinel, scores match the oracle."""
    N = 200
    rng = np.random.default_rng(17)
    x = rng.standard_normal((N, 128)).astype(np.float32)
    kc, ks = oracle.quantize_rows(x)
    kct, kst = t(tile_keys(kc[None])), t(ks[None])
    nq = len(nv)
    q = synth.normal_bf16(synth.key(11, 12, 0, 0), 0, nq * 4096, 1 / np.sqrt(128)).reshape(1, nq, 32, 128)
    w = synth.uniform_f32(synth.key(11, 13, 0, 0), 0, nq * 32).reshape(1, nq, 32)
    nva = np.array([nv], np.int32)
    nblk = cdiv(N, 8)
    sc = torch.full((1, nq, N), 12345.0, device=dev())
    bm = torch.full((1, nq, nblk), 12345.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), kct, kst, t(nva), bm, sc)
    sc, bm = sc.cpu().numpy(), bm.cpu().numpy()
    for i, n in enumerate(nv):
        s1 = torch.full((1, 1, N), 12345.0, device=dev())
        b1 = torch.full((1, 1, nblk), 12345.0, device=dev())
        L.index_full(t(q[:, i:i + 1].copy(), torch.uint16), t(w[:, i:i + 1].copy()), kct, kst,
                     t(np.array([[n]], np.int32)), b1, s1)
        assert np.array_equal(sc[0, i], s1.cpu().numpy()[0, 0]), f"row {i}: scores"
        assert np.array_equal(bm[0, i], b1.cpu().numpy()[0, 0]), f"row {i}: maxima"
        assert np.all(sc[0, i, n:] == 12345.0), f"row {i}: scores past the end"
        assert np.all(bm[0, i, cdiv(n, 8):] == 12345.0), f"row {i}: maxima past the end"
        if n:
            ok, err = finite_close(sc[0, i, :n], oracle.index_scores(q[0, i], w[0, i], kc, ks, n))
            assert ok, f"row {i}: max err {err}"
            ref_bm = [sc[0, i, 8 * j:min(8 * j + 8, n)].max() for j in range(cdiv(n, 8))]
            assert np.array_equal(bm[0, i, :cdiv(n, 8)], np.array(ref_bm, np.float32))


@pytest.mark.parametrize("B,nq,n_cap,nb,nvis", [
    (1, 1, 1 << 20, 2048, [1 << 20]),                      # groups of 8 blocks
    (2, 1, 1 << 20, 2048, [(1 << 20) - 5000, 300001]),     # chunks past the end, partial groups
    (1, 2, 1 << 20, 2048, [1 << 20, 999999]),              # multi-row scans write group keys too
    (1, 1, 1 << 20, 512, [654321]),                        # groups of 8, k = 512
    (2, 1, 140003, 2048, [140003, 70001]),                 # groups of 2
    (1, 3, 300000, 2048, [300000, 299999, 5]),             # groups of 3: the select's own pass
    (2, 1, 65536, 2048, [70000, 100]),                     # one segment: direct select
    (1, 1, 2048, 2048, [0]),                               # nothing visible
    (1, 1, 0, 64, [5]),                                    # empty cache: no blocks
])
def test_index_full_pool_matches_scan_then_topk(B, nq, n_cap, nb, nvis):
    """csa2_index_full_pool returns exactly csa2_index_full's block maxima and
    csa2_topk's selection over them (n_valid = ceil(n_visible / 8)), whether the scan
    writes the select's group maxima itself or the select computes them."""
    print(f"[case] B={B} nq={nq} n_cap={n_cap} nb={nb} nvis={nvis}", flush=True)
    g = torch.Generator(device=dev())
    g.manual_seed(n_cap + nb)
    kc = torch.randint(0, 256, (L.key_code_bytes(B * n_cap),), dtype=torch.uint8, device=dev(),
                       generator=g)
    ks = (torch.randint(0, 256, (B, n_cap, 8), dtype=torch.uint8, device=dev(), generator=g)
          & 0x77) | 0x30  # finite E4M3 scales
    q = synth.normal_bf16(synth.key(11, 12, 0, 0), 0, B * nq * 4096, 1 / np.sqrt(128)).reshape(B, nq, 32, 128)
    w = synth.uniform_f32(synth.key(11, 13, 0, 0), 0, B * nq * 32).reshape(B, nq, 32)
    nv = np.array(nvis, np.int32).reshape(B, nq)
    nblk = cdiv(n_cap, 8)
    ws_n = max(L.index_full_pool_workspace(n_cap, B * nq, nb), 8)
    assert ws_n >= L.topk_workspace(nblk, B * nq, nb)
    bm1 = torch.full((B, nq, nblk), 777.0, device=dev())
    pool1 = torch.full((B, nq, nb), -7, dtype=torch.int32, device=dev())
    ws = torch.full((ws_n,), 0xC3, dtype=torch.uint8, device=dev())  # stale contents
    evs = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in evs:
        e.record()  # created before the library records them
    L.index_full_pool(t(q, torch.uint16), t(w), kc, ks, t(nv), bm1, pool1, ws=ws, scan_events=evs)
    torch.cuda.synchronize()
    if max(nvis) > 0:  # the scan's dispatch recorded both events
        assert evs[0].elapsed_time(evs[1]) > 0.0
    bm2 = torch.full((B, nq, nblk), 777.0, device=dev())
    L.index_full(t(q, torch.uint16), t(w), kc, ks, t(nv), bm2)
    pool2 = torch.full((B, nq, nb), -7, dtype=torch.int32, device=dev())
    nblk_valid = t(((np.maximum(nv.astype(np.int64), 0) + 7) // 8).astype(np.int32))
    L.topk(bm2, nb, pool2, n_valid=nblk_valid, ws=torch.empty(ws_n, dtype=torch.uint8, device=dev()))
    bm1, bm2 = bm1.cpu().numpy(), bm2.cpu().numpy()
    assert np.array_equal(bm1, bm2)
    p1, p2 = pool1.cpu().numpy(), pool2.cpu().numpy()
    assert np.array_equal(p1, p2)
    for r in range(B * nq):  # a valid pool: ascending ids of visible blocks, -1 padded
        row = p1.reshape(B * nq, nb)[r]
        n_ok = min(nb, cdiv(min(max(int(nv.reshape(-1)[r]), 0), n_cap), 8))
        assert np.all(np.diff(row[:n_ok]) > 0) and np.all(row[n_ok:] == -1)


# ------------------------------------------------------------------ attention

def _attn_case(B=2, N=3000, k=100, swa_cap=160, seed=3):
    w = synth.WORKLOADS[1]
    vc, vs, sw, sel, q = [], [], [], [], []
    rng = np.random.default_rng(seed)
    for b in range(B):
        x = synth.latent_rows(synth.key(12, 2, 0, b), synth.key(12, 3, 0, b), 0, N, 512)
        cos, sin = synth.rope_rows(0, N)
        c, s = oracle.quantize_rows(x, cos, sin, 448, 64)
        vc.append(c)
        vs.append(s)
        sw.append(oracle.encode_fp8(synth.latent_rows(synth.key(12, 4, 0, b),
                                                      synth.key(12, 5, 0, b), 0, swa_cap, 512)))
        sel.append(np.sort(rng.choice(N, k, replace=False)).astype(np.int32))
        q.append(synth.normal_bf16(synth.key(12, 8, 0, b), 0, 64 * 512, 1 / np.sqrt(512)))
    return (np.stack(vc), np.stack(vs), np.stack(sw), np.stack(sel)[:, None],
            np.stack(q).reshape(B, 1, 64, 512))


def test_topk_of_empty_rows_is_all_padding():
    """Rows of length 0 (an empty cache has no blocks) select nothing: -1 everywhere."""
    out = torch.full((3, 5), 7, dtype=torch.int32, device=dev())
    L.topk(torch.empty((3, 0), device=dev()), 5, out)
    assert np.all(out.cpu().numpy() == -1)


@pytest.mark.parametrize("use_ws", [True, False])
def test_attention_with_empty_main_cache_is_window_only(use_ws):
    """No compressed entries yet (n_cap = 0, every top-k index -1): the softmax runs over
    the window rows alone, as the oracle's attention over an empty selected set."""
    _, _, sw, _, q = _attn_case(B=2, N=64, k=16, seed=17)
    B = q.shape[0]
    vc = np.zeros((B, 0, 256), np.uint8)
    vs = np.zeros((B, 0, 32), np.uint8)
    sel = np.full((B, 1, 16), -1, np.int32)
    swa_end = np.array([[128], [37]], np.int32)
    out, lse = _run_attn(q, vc, vs, sel, sw, swa_end, use_ws=use_ws)
    for b in range(B):
        ref, ref_lse = oracle.attention(q[b, 0], vc[b], vs[b], sel[b, 0], sw[b], int(swa_end[b, 0]))
        assert max_abs(out[b, 0], ref) <= ATTN_TOL
        assert max_abs(lse[b, 0], ref_lse) <= 1e-4


def _run_attn(q, vc, vs, sel, sw, swa_end, n_win=128, scale=1.0, use_ws=True):
    B = q.shape[0]
    k = sel.shape[-1]
    out = torch.full((B, 1, 64, 512), 777.0, device=dev())
    lse = torch.full((B, 1, 64), 777.0, device=dev())
    ws = None
    if use_ws:
        n = L.sparse_attn_workspace(B, 1, k, n_win)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev())
    L.sparse_attn(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end), out, lse,
                  n_win=n_win, softmax_scale=scale, ws=ws)
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("variant", ["plain", "padded", "window_only", "empty", "short_window",
                                     "scale", "zero_q", "no_ws", "huge_q", "tiny_q"])
def test_sparse_attn_matches_oracle(variant):
    vc, vs, sw, sel, q = _attn_case()
    B = q.shape[0]
    swa_end = np.array([[128], [150]], np.int32)
    n_win, scale, use_ws = 128, 1.0, True
    if variant == "padded":
        sel = sel.copy()
        sel[:, :, ::7] = -1
        sel[:, :, 3] = 10 ** 6  # out of range: skipped
    elif variant == "window_only":
        sel = -np.ones_like(sel)
    elif variant == "empty":
        sel = -np.ones_like(sel)
        swa_end = np.zeros_like(swa_end)
    elif variant == "short_window":
        swa_end = np.array([[40], [200]], np.int32)  # 200 > capacity 160
    elif variant == "scale":
        scale = 0.6
    elif variant == "zero_q":
        q = np.zeros_like(q)
    elif variant == "no_ws":
        use_ws = False
    elif variant in ("huge_q", "tiny_q"):
        # query amplitudes beyond fp16's range (|q| up to ~2^20, where a plain cast would
        # overflow) or in its subnormals (~2^-22), the softmax scale bringing the logits
        # back: each head's query is rescaled by a power of two inside the kernel
        e = 20 if variant == "huge_q" else -22
        qf = (q.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** e)
        q = (qf.view(np.uint32) >> 16).astype(np.uint16)  # exact: a power of two
        q[:, :, 5] = 0  # an all-zero head too
        scale = 2.0 ** -e
    out, lse = _run_attn(q, vc, vs, sel, sw, swa_end, n_win, scale, use_ws)
    for b in range(B):
        ro, rl = oracle.attention(q[b, 0], vc[b], vs[b], sel[b, 0], sw[b], int(swa_end[b, 0]),
                                  n_win, scale)
        assert max_abs(out[b, 0], ro) <= ATTN_TOL, f"seq {b}: {max_abs(out[b, 0], ro)}"
        if np.all(np.isinf(rl)):
            assert np.all(np.isneginf(lse[b, 0])) and np.all(out[b, 0] == 0)
        else:
            assert max_abs(lse[b, 0], rl) <= 1e-4


@pytest.mark.parametrize("use_ws", [True, False])
def test_sparse_attn_rows_at_the_top_of_the_largest_caches(use_ws):
    """The attention addresses rows with 32-bit byte offsets, so its caches hold at most
    2^24 main entries (256 code bytes each: offsets up to 2^32 - 256) and 2^22 window
    rows: selected entries up to the very last of a 2^24-entry cache and window rows
    ending at 2^22, against the oracle over the same rows in small arrays."""
    N, W, n = 1 << 24, 1 << 22, 600
    print(f"[case] attention rows below {N} / {W}, workspace {use_ws}", flush=True)
    vc, vs, sw, sel, q = _attn_case(B=1, N=n, k=100, seed=31)
    sel[0, 0, -1] = n - 1  # the cache's last entry (sel stays sorted and distinct)
    vcd = torch.zeros((1, N, 256), dtype=torch.uint8, device=dev())
    vsd = torch.zeros((1, N, 32), dtype=torch.uint8, device=dev())
    swd = torch.zeros((1, W, 512), dtype=torch.uint8, device=dev())
    vcd[0, N - n:] = t(vc[0])
    vsd[0, N - n:] = t(vs[0])
    swd[0, W - sw.shape[1]:] = t(sw[0])
    out = torch.full((1, 1, 64, 512), 777.0, device=dev())
    lse = torch.full((1, 1, 64), 777.0, device=dev())
    ws = None
    if use_ws:
        ws = torch.empty(max(L.sparse_attn_workspace(1, 1, 100, 128), 16), dtype=torch.uint8,
                         device=dev())
    L.sparse_attn(t(q, torch.uint16), vcd, vsd, t(sel + (N - n)), swd,
                  t(np.array([[W]], np.int32)), out, lse, n_win=128, softmax_scale=1.0, ws=ws)
    torch.cuda.synchronize()
    # the window rows [W - 128, W) are rows [32, 160) of the small window
    ro, rl = oracle.attention(q[0, 0], vc[0], vs[0], sel[0, 0], sw[0], sw.shape[1], 128, 1.0)
    assert max_abs(out.cpu().numpy()[0, 0], ro) <= ATTN_TOL
    assert max_abs(lse.cpu().numpy()[0, 0], rl) <= 1e-4
    del vcd, vsd, swd
    torch.cuda.empty_cache()


def test_sparse_attn_k_not_multiple_of_tile_and_large_k():
    vc, vs, sw, sel, q = _attn_case(B=1, N=5000, k=1000, seed=4)
    swa_end = np.array([[128]], np.int32)
    out, lse = _run_attn(q, vc, vs, sel, sw, swa_end)
    ro, rl = oracle.attention(q[0, 0], vc[0], vs[0], sel[0, 0], sw[0], 128)
    assert max_abs(out[0, 0], ro) <= ATTN_TOL
    assert max_abs(lse[0, 0], rl) <= 1e-4


def test_sparse_attn_batched_kernel_many_rows():
    """300 query rows of one sequence (one workgroup per row and its 64 heads, the
    channels split over the waves), sampled rows against the oracle."""
    N, nq, k, cap = 3000, 300, 96, 500
    x = synth.latent_rows(synth.key(13, 2), synth.key(13, 3), 0, N, 512)
    cos, sin = synth.rope_rows(0, N)
    vc, vs = oracle.quantize_rows(x, cos, sin, 448, 64)
    sw = oracle.encode_fp8(synth.latent_rows(synth.key(13, 4), synth.key(13, 5), 0, cap, 512))
    rng = np.random.default_rng(14)
    sel = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(nq)]).astype(np.int32)
    sel[::7, ::5] = -1
    q = synth.normal_bf16(synth.key(13, 8), 0, nq * 64 * 512, 1 / np.sqrt(512)).reshape(1, nq, 64, 512)
    swa_end = (np.arange(nq, dtype=np.int32) + 40).reshape(1, nq)  # ragged windows, some short
    out = torch.full((1, nq, 64, 512), 777.0, device=dev())
    lse = torch.full((1, nq, 64), 777.0, device=dev())
    L.sparse_attn(t(q, torch.uint16), t(vc[None]), t(vs[None]), t(sel[None]), t(sw[None]),
                  t(swa_end), out, lse)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in list(range(0, nq, 23)) + [nq - 1]:
        ro, rl = oracle.attention(q[0, i], vc, vs, sel[i], sw, int(swa_end[0, i]), 128, 1.0)
        assert max_abs(out[0, i], ro) <= ATTN_TOL, f"query {i}"
        assert max_abs(lse[0, i], rl) <= 1e-4


def _grouped_case(seed=21, B=3, nq=8):
    """24 query rows (3 sequences x 8 queries), called without a workspace: the grouped
    form without key splits runs.  Row r mixes top-k padding and window shapes by r % 6: plain,
    padded (-1 and out-of-range ids), window only, empty, window past the ring capacity,
    short window; k = 100 leaves a ragged last tile."""
    N, k, cap = 2000, 100, 160
    rng = np.random.default_rng(seed)
    vc, vs, sw = [], [], []
    for b in range(B):
        x = synth.latent_rows(synth.key(15, 2, 0, b), synth.key(15, 3, 0, b), 0, N, 512)
        cos, sin = synth.rope_rows(0, N)
        c, sc = oracle.quantize_rows(x, cos, sin, 448, 64)
        vc.append(c)
        vs.append(sc)
        sw.append(oracle.encode_fp8(synth.latent_rows(synth.key(15, 4, 0, b),
                                                      synth.key(15, 5, 0, b), 0, cap, 512)))
    sel = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B * nq)])
    sel = sel.astype(np.int32).reshape(B, nq, k)
    ends = np.array([128, 150, 140, 0, 200, 40], np.int32)
    swa_end = np.zeros((B, nq), np.int32)
    for r in range(B * nq):
        b, i = divmod(r, nq)
        kind = r % 6
        swa_end[b, i] = ends[kind]
        if kind == 1:
            sel[b, i, ::7] = -1
            sel[b, i, 3] = 10 ** 6
        elif kind in (2, 3):
            sel[b, i] = -1
    q = synth.normal_bf16(synth.key(15, 8), 0, B * nq * 64 * 512, 1 / np.sqrt(512))
    return np.stack(vc), np.stack(vs), np.stack(sw), sel, q.reshape(B, nq, 64, 512), swa_end


def test_sparse_attn_grouped_form_matches_oracle():
    vc, vs, sw, sel, q, swa_end = _grouped_case()
    B, nq = q.shape[:2]
    out = torch.full((B, nq, 64, 512), 777.0, device=dev())
    lse = torch.full((B, nq, 64), 777.0, device=dev())
    L.sparse_attn(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end), out, lse,
                  softmax_scale=0.8)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(B):
        for i in range(nq):
            ro, rl = oracle.attention(q[b, i], vc[b], vs[b], sel[b, i], sw[b],
                                      int(swa_end[b, i]), 128, 0.8)
            assert max_abs(out[b, i], ro) <= ATTN_TOL, f"row {b},{i}"
            if np.all(np.isinf(rl)):
                assert np.all(np.isneginf(lse[b, i])) and np.all(out[b, i] == 0)
            else:
                assert max_abs(lse[b, i], rl) <= 1e-4, f"row {b},{i}"


def test_sparse_attn_grouped_form_rope_bf16():
    """The bf16 epilogue in the grouped form: oracle parity and bit-exact agreement with
    the grouped fp32 output rotated and rounded on the host."""
    vc, vs, sw, sel, q, swa_end = _grouped_case(seed=22)
    B, nq = q.shape[:2]
    rng = np.random.default_rng(23)
    ang = rng.uniform(-np.pi, np.pi, (B * nq, 32))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    out16 = torch.full((B, nq, 64, 512), 0x7777, dtype=torch.int16, device=dev())
    lse16 = torch.empty((B, nq, 64), device=dev())
    L.sparse_attn_rope_bf16(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end),
                            t(cos), t(sin), out16, lse16)
    out32 = torch.empty((B, nq, 64, 512), device=dev())
    lse32 = torch.empty((B, nq, 64), device=dev())
    L.sparse_attn(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end), out32, lse32)
    got = out16.cpu().numpy().view(np.uint16)
    out32 = out32.cpu().numpy()
    assert np.array_equal(lse16.cpu().numpy(), lse32.cpu().numpy())
    for r in range(B * nq):
        b, i = divmod(r, nq)
        ref_bits, _, _ = oracle.attention_rope_bf16(
            q[b, i], vc[b], vs[b], sel[b, i], sw[b], int(swa_end[b, i]), cos[r], sin[r])
        g, ref = _bf16_to_f32(got[b, i]), _bf16_to_f32(ref_bits)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        assert np.all(np.abs(g - ref) <= 2 * ATTN_TOL + ulp), f"row {r}"
        o = out32[b, i].astype(np.float32).copy()
        a, c = o[:, 448::2].copy(), o[:, 449::2].copy()
        co, si = cos[r][None, :], sin[r][None, :]
        o[:, 448::2] = (a * co) + (c * si)
        o[:, 449::2] = (c * co) - (a * si)
        host = torch.from_numpy(o).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[b, i], host), f"row {r}"


@pytest.mark.parametrize("bf16", [False, True])
def test_sparse_attn_head_group_sizes(bf16):
    """A workgroup serves 64 heads from 256 query rows, 32 heads from 128 and 16 below.  The
    16- and 64-head forms (both on 32-key tiles) give bit-identical outputs and lse; the
    32-head form (64-key tiles) differs from them only in fp32 rounding.  Sampled rows of
    every padding / window kind match the oracle."""
    vc, vs, sw, sel, q, swa_end = _grouped_case(seed=24, B=1, nq=300)
    nq = q.shape[1]
    rng = np.random.default_rng(25)
    ang = rng.uniform(-np.pi, np.pi, (nq, 32))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)

    def run(r0, r1):
        n = r1 - r0
        lse = torch.empty((1, n, 64), device=dev())
        args = (t(q[:, r0:r1], torch.uint16), t(vc), t(vs), t(sel[:, r0:r1]), t(sw),
                t(swa_end[:, r0:r1]))
        if bf16:
            out = torch.empty((1, n, 64, 512), dtype=torch.int16, device=dev())
            L.sparse_attn_rope_bf16(*args, t(cos[r0:r1]), t(sin[r0:r1]), out, lse)
        else:
            out = torch.empty((1, n, 64, 512), device=dev())
            L.sparse_attn(*args, out, lse)
        return out.cpu().numpy(), lse.cpu().numpy()

    def chunks(size):
        parts = [run(r0, min(r0 + size, nq)) for r0 in range(0, nq, size)]
        return (np.concatenate([p[0] for p in parts], axis=1),
                np.concatenate([p[1] for p in parts], axis=1))

    o64, l64 = run(0, nq)        # 64 heads per workgroup
    o16, l16 = chunks(100)       # 16 heads
    o32, l32 = chunks(150)       # 32 heads
    assert np.array_equal(o64, o16) and np.array_equal(l64, l16)
    fin = np.isfinite(l64)
    assert np.array_equal(fin, np.isfinite(l32))
    assert np.all(np.abs(l32[fin] - l64[fin]) <= 1e-5)
    if bf16:
        a, b = _bf16_to_f32(o32.view(np.uint16)), _bf16_to_f32(o64.view(np.uint16))
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(b), 1e-30))) - 7)
        assert np.all(np.abs(a - b) <= 1e-5 + ulp)
    else:
        assert max_abs(o32, o64) <= 1e-5
        for i in list(range(0, nq, 37)) + list(range(nq - 6, nq)):
            ro, rl = oracle.attention(q[0, i], vc[0], vs[0], sel[0, i], sw[0],
                                      int(swa_end[0, i]), 128, 1.0)
            for o, lz in ((o64, l64), (o32, l32)):
                assert max_abs(o[0, i], ro) <= ATTN_TOL, f"row {i}"
                if np.all(np.isinf(rl)):
                    assert np.all(np.isneginf(lz[0, i])) and np.all(o[0, i] == 0)
                else:
                    assert max_abs(lz[0, i], rl) <= 1e-4, f"row {i}"


def test_sparse_attn_split_form_32_heads():
    """64 query rows with the workspace: key splits over workgroups of 32 heads (2 splits)
    and the merge.  Every row of every padding / window kind matches the oracle, and the
    outputs differ from the unsplit form (no workspace: 16 heads per workgroup) only in
    fp32 rounding."""
    vc, vs, sw, sel, q, swa_end = _grouped_case(seed=26, B=8, nq=8)
    B, nq = q.shape[:2]
    assert L.sparse_attn_workspace(B, nq, sel.shape[-1], 128) == B * nq * 4 * 2 * (16 * 512 + 32) * 4
    res = []
    for use_ws in (True, False):
        out = torch.full((B, nq, 64, 512), 777.0, device=dev())
        lse = torch.full((B, nq, 64), 777.0, device=dev())
        ws = None
        if use_ws:
            ws = torch.empty(L.sparse_attn_workspace(B, nq, sel.shape[-1], 128), dtype=torch.uint8,
                             device=dev())
        L.sparse_attn(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end), out, lse,
                      ws=ws)
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    (o, l), (o1, l1) = res
    assert max_abs(o, o1) <= 1e-5
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l)) and np.all(np.abs(l[fin] - l1[fin]) <= 1e-5)
    for b in range(B):
        for i in range(nq):
            ro, rl = oracle.attention(q[b, i], vc[b], vs[b], sel[b, i], sw[b],
                                      int(swa_end[b, i]), 128, 1.0)
            assert max_abs(o[b, i], ro) <= ATTN_TOL, f"row {b},{i}"
            if np.all(np.isinf(rl)):
                assert np.all(np.isneginf(l[b, i])) and np.all(o[b, i] == 0)
            else:
                assert max_abs(l[b, i], rl) <= 1e-4, f"row {b},{i}"
    # the bf16 epilogue through the same 32-head splits and merge: the fp32 split
    # output rotated and rounded with the same fp32 operations, bit for bit
    rng = np.random.default_rng(27)
    ang = rng.uniform(-np.pi, np.pi, (B * nq, 32))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    out16 = torch.full((B, nq, 64, 512), 0x7777, dtype=torch.int16, device=dev())
    lse16 = torch.empty((B, nq, 64), device=dev())
    ws = torch.empty(L.sparse_attn_workspace(B, nq, sel.shape[-1], 128), dtype=torch.uint8,
                     device=dev())
    L.sparse_attn_rope_bf16(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end),
                            t(cos), t(sin), out16, lse16, ws=ws)
    got = out16.cpu().numpy().view(np.uint16)
    assert np.array_equal(lse16.cpu().numpy(), l)
    for r in range(B * nq):
        b, i = divmod(r, nq)
        x = o[b, i].astype(np.float32).copy()
        a_, c_ = x[:, 448::2].copy(), x[:, 449::2].copy()
        co, si = cos[r][None, :], sin[r][None, :]
        x[:, 448::2] = (a_ * co) + (c_ * si)
        x[:, 449::2] = (c_ * co) - (a_ * si)
        host = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[b, i], host), f"row {b},{i}"


def _bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_sparse_attn_rope_bf16_epilogue():
    """Inverse rotary + bf16 epilogue: oracle parity within the attention tolerance plus
    one bf16 ulp, and bit-exact agreement with the fp32 entry point's output rotated
    and rounded with the same fp32 operations."""
    vc, vs, sw, sel, q = _attn_case(B=3, N=3000, k=100, seed=7)
    B = 3
    swa_end = np.array([[128], [60], [0]], np.int32)
    rng = np.random.default_rng(8)
    ang = rng.uniform(-np.pi, np.pi, (B, 32))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    out16 = torch.full((B, 1, 64, 512), 0x7777, dtype=torch.int16, device=dev())
    lse16 = torch.empty((B, 1, 64), device=dev())
    # the same key split as _run_attn's fp32 call, so both sum in the same order
    ws = torch.zeros(max(L.sparse_attn_workspace(B, 1, sel.shape[-1], 128), 16),
                     dtype=torch.uint8, device=dev())
    L.sparse_attn_rope_bf16(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end),
                            t(cos), t(sin), out16, lse16, ws=ws)
    got = out16.cpu().numpy().view(np.uint16)
    out32, lse32 = _run_attn(q, vc, vs, sel, sw, swa_end)
    assert np.array_equal(lse16.cpu().numpy(), lse32)
    for b in range(B):
        ref_bits, ref_out, ref_lse = oracle.attention_rope_bf16(
            q[b, 0], vc[b], vs[b], sel[b, 0], sw[b], int(swa_end[b, 0]), cos[b], sin[b])
        g, r = _bf16_to_f32(got[b, 0]), _bf16_to_f32(ref_bits)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
        assert np.all(np.abs(g - r) <= 2 * ATTN_TOL + ulp), f"seq {b}"
        assert np.mean(got[b, 0] == ref_bits) > 0.99
        # the same epilogue on the fp32 entry point's output, fp32 products and sums
        o = out32[b, 0].astype(np.float32).copy()
        a, c = o[:, 448::2].copy(), o[:, 449::2].copy()
        co, si = cos[b][None, :], sin[b][None, :]
        o[:, 448::2] = (a * co) + (c * si)
        o[:, 449::2] = (c * co) - (a * si)
        host = torch.from_numpy(o).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[b, 0], host), f"seq {b}"


# ------------------------------------------------------------------ new entries (one launch)

def _entries_case(R, S, seed):
    rng = np.random.default_rng(seed)
    kv_x = synth.latent_rows(synth.key(13, 1, 0, seed), synth.key(13, 2, 0, seed), 0, R, 512)
    cos, sin = synth.rope_rows(1000 + seed, R)
    idx_x = rng.standard_normal((R, 128)).astype(np.float32)
    swa_x = synth.latent_rows(synth.key(13, 3, 0, seed), synth.key(13, 4, 0, seed), 0, S, 512)
    return kv_x, cos, sin, idx_x, swa_x


def _entries_buffers(n_rows, n_swa):
    """Caches filled with 0xA5; the indexer-key codes in whole key tiles."""
    z = lambda *sh: torch.full(sh, 0xA5, dtype=torch.uint8, device=dev())
    return (z(n_rows, 256), z(n_rows, 32), z(L.key_code_bytes(n_rows)), z(n_rows, 8),
            z(n_swa, 512))


def _host_caches(kc, ks, ic, isc, sw, n_rows):
    """Host copies, the key codes untiled to [n_rows, 64]."""
    return (kc.cpu().numpy(), ks.cpu().numpy(), untile_keys(ic, n_rows), isc.cpu().numpy(),
            sw.cpu().numpy())


def _ambiguous_groups(y, bound):
    """[rows, 8] bool: 16-channel groups of the double projections y [rows, 128] whose
    encoding the +-bound uncertainty of an fp32 projection can change -- the group's
    E4M3 scale decision (amax / 6) or some element's E2M1 decision (|y| / scale) lies
    within the bound of a rounding boundary."""
    R = y.shape[0]
    yg = np.abs(y).reshape(R, 8, 16)
    bg = bound.reshape(R, 8, 16)
    amb = np.zeros((R, 8), bool)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for r in range(R):
        for g in range(8):
            a_lo = max((yg[r, g] - bg[r, g]).max(), 0.0)
            a_hi = (yg[r, g] + bg[r, g]).max()
            s_lo, s_hi = oracle.e4m3_encode(a_lo / 6.0), oracle.e4m3_encode(a_hi / 6.0)
            if s_lo != s_hi:
                amb[r, g] = True
                continue
            sc = oracle.e4m3_decode(s_lo)
            if sc == 0.0:
                continue
            x_lo = (yg[r, g] - bg[r, g]) / sc
            x_hi = (yg[r, g] + bg[r, g]) / sc
            if np.any((x_lo[:, None] <= mids[None, :]) & (mids[None, :] <= x_hi[:, None])):
                amb[r, g] = True
            elif np.any(yg[r, g] <= bg[r, g]):  # the sign itself is uncertain
                amb[r, g] = True
    return amb


@pytest.mark.parametrize("R,S,project", [(1, 1, False), (16, 16, False), (37, 5, False),
                                         (0, 3, False), (1, 0, True), (16, 16, True),
                                         (37, 0, True)])
def test_encode_entries_one_launch(R, S, project):
    kv_x, cos, sin, idx_x, swa_x = _entries_case(R, S, seed=R + 3 * S + project)
    stride, row0, swa_stride, swa_row0 = 3, 2, 2, 1
    n_rows, n_swa = row0 + max(R - 1, 0) * stride + 2, swa_row0 + max(S - 1, 0) * swa_stride + 2
    kc, ks, ic, isc, sw = _entries_buffers(n_rows, n_swa)
    rng = np.random.default_rng(R)
    w_bits = torch.from_numpy((rng.standard_normal((128, 512)) / np.sqrt(512)).astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    y = torch.full((max(R, 1), 128), np.nan, device=dev()) if project else None
    L.encode_entries(t(kv_x), kc, ks, ic, isc, idx_x=None if project else t(idx_x),
                     w_idx=t(w_bits, torch.uint16) if project else None,
                     rope_cos=t(cos), rope_sin=t(sin), rope_offset=448, rope_dim=64,
                     dst_row=row0, dst_stride=stride, idx_y=y,
                     swa_x=t(swa_x) if S else None, swa_out=sw if S else None,
                     swa_row=swa_row0, swa_stride=swa_stride)
    padded = L.key_code_bytes(n_rows) // 64
    tail = untile_keys(ic, padded)[n_rows:]
    assert np.all(tail == 0xA5)  # the padding rows of the last key tile are untouched
    kc, ks, ic, isc, sw = _host_caches(kc, ks, ic, isc, sw, n_rows)
    rows = row0 + stride * np.arange(R)
    other = np.setdiff1d(np.arange(n_rows), rows)
    if R:
        ref_c, ref_s = oracle.quantize_rows(kv_x, cos, sin, 448, 64)
        assert np.array_equal(kc[rows], ref_c) and np.array_equal(ks[rows], ref_s)
        if project:
            yg = y.cpu().numpy()[:R]
            yo = oracle.project_rows(kv_x, w_bits)
            wd = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            bound = 130 * 2.0 ** -24 * (np.abs(kv_x).astype(np.float64) @ np.abs(wd).T)
            assert np.all(np.abs(yg - yo) <= bound)
            # codes against the oracle's own projection and encoder; a group may differ
            # only where the oracle's values lie within the accumulation bound of one of
            # its rounding boundaries (then either side of it is a correct encoding)
            ref_ic, ref_is = oracle.quantize_rows(yo.astype(np.float32))
            amb = _ambiguous_groups(yo, bound)
            got_c = ic[rows].reshape(R, 8, 8)
            got_s = isc[rows]
            differ = ~(np.all(got_c == ref_ic.reshape(R, 8, 8), axis=2) & (got_s == ref_is))
            assert not np.any(differ & ~amb), "projected-key codes differ outside a near-tie"
            print(f"[case] projected groups differing at a rounding near-tie: "
                  f"{int(np.sum(differ))} of {R * 8} ({int(np.sum(amb))} near a boundary)")
        else:
            ref_ic, ref_is = oracle.quantize_rows(idx_x)
            assert np.array_equal(ic[rows], ref_ic) and np.array_equal(isc[rows], ref_is)
    for a in (kc, ks, ic, isc):
        assert np.all(a[other] == 0xA5)
    if S:
        srows = swa_row0 + swa_stride * np.arange(S)
        assert np.array_equal(sw[srows], oracle.encode_fp8(swa_x))
        assert np.all(sw[np.setdiff1d(np.arange(n_swa), srows)] == 0xA5)


def test_encode_entries_per_sequence_destinations_and_ring():
    """Sequences at different positions: each appends its entry at its own cache row and
    its window row at ring slot p % 128; destinations outside the buffers are skipped."""
    R, n_cap, ring = 6, 40, 128
    kv_x, cos, sin, idx_x, swa_x = _entries_case(R, R, seed=11)
    pos = np.array([5, 127, 128, 300, 39, 7], np.int64)       # token positions
    n_b = np.array([3, 39, 0, 17, 39, 2], np.int64)           # append positions in the caches
    kv_dst = np.arange(R) * n_cap + n_b
    kv_dst[5] = R * n_cap + 3                                 # outside: skipped
    swa_dst = np.arange(R) * ring + pos % ring
    swa_dst[4] = -1                                           # skipped
    kc, ks, ic, isc, sw = _entries_buffers(R * n_cap, R * ring)
    L.encode_entries(t(kv_x), kc, ks, ic, isc, idx_x=t(idx_x), rope_cos=t(cos), rope_sin=t(sin),
                     rope_offset=448, rope_dim=64, kv_dst=t(kv_dst), swa_x=t(swa_x), swa_out=sw,
                     swa_dst=t(swa_dst))
    kc, ks, ic, isc, sw = _host_caches(kc, ks, ic, isc, sw, R * n_cap)
    ref_c, ref_s = oracle.quantize_rows(kv_x, cos, sin, 448, 64)
    ref_ic, ref_is = oracle.quantize_rows(idx_x)
    ok = np.arange(5)
    assert np.array_equal(kc[kv_dst[ok]], ref_c[ok]) and np.array_equal(ks[kv_dst[ok]], ref_s[ok])
    assert np.array_equal(ic[kv_dst[ok]], ref_ic[ok]) and np.array_equal(isc[kv_dst[ok]], ref_is[ok])
    untouched = np.setdiff1d(np.arange(R * n_cap), kv_dst[ok])
    assert all(np.all(a[untouched] == 0xA5) for a in (kc, ks, ic, isc))
    sok = np.array([0, 1, 2, 3, 5])
    assert np.array_equal(sw[swa_dst[sok]], oracle.encode_fp8(swa_x)[sok])
    assert np.all(sw[np.setdiff1d(np.arange(R * ring), swa_dst[sok])] == 0xA5)


def test_encode_entries_at_the_top_of_the_largest_caches():
    """Destinations at the top of the largest caches the attention takes (2^24 main and
    indexer-key entries, 2^22 window rows), written in one launch in reverse order: the
    bytes against the oracle's encodings, the rows just below untouched."""
    N, W, R = 1 << 24, 1 << 22, 40
    print(f"[case] encoder destinations below {N} / {W}", flush=True)

    def filled(n):  # 0xA5 in fills of at most 2^30 elements each
        a = torch.empty(n, dtype=torch.uint8, device=dev())
        for o in range(0, n, 1 << 30):
            a[o:o + (1 << 30)].fill_(0xA5)
        return a

    kv_x, cos, sin, idx_x, swa_x = _entries_case(R, R, seed=24)
    kc, ks = filled(N * 256).view(N, 256), filled(N * 32).view(N, 32)
    ic, isc = filled(L.key_code_bytes(N)), filled(N * 8).view(N, 8)
    sw = filled(W * 512).view(W, 512)
    kv_dst = np.arange(N - 1, N - 1 - R, -1, dtype=np.int64)  # the last entry first
    swa_dst = np.arange(W - R, W, dtype=np.int64)
    L.encode_entries(t(kv_x), kc, ks, ic, isc, idx_x=t(idx_x), rope_cos=t(cos), rope_sin=t(sin),
                     rope_offset=448, rope_dim=64, kv_dst=t(kv_dst), swa_x=t(swa_x), swa_out=sw,
                     swa_dst=t(swa_dst))
    torch.cuda.synchronize()
    lo = N - 64  # the top two key tiles
    got = (kc[lo:].cpu().numpy(), ks[lo:].cpu().numpy(),
           untile_keys(ic[(lo // 32) * 2048:], 64), isc[lo:].cpu().numpy())
    ref_c, ref_s = oracle.quantize_rows(kv_x, cos, sin, 448, 64)
    ref_ic, ref_is = oracle.quantize_rows(idx_x)
    at = kv_dst - lo
    for g, r, name in zip(got, (ref_c, ref_s, ref_ic, ref_is), ("codes", "scales", "key codes", "key scales")):
        assert np.array_equal(g[at], r), name
        assert np.all(g[:64 - R] == 0xA5), f"{name}: rows below the destinations touched"
    gw = sw[W - 64:].cpu().numpy()
    assert np.array_equal(gw[64 - R:], oracle.encode_fp8(swa_x)) and np.all(gw[:64 - R] == 0xA5)
    del kc, ks, ic, isc, sw
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [50, 300])
def test_window_ring_replay_matches_linear_window(P):
    """Bounded replay of a prompt's last 128 tokens into the ring (slot p % 128) gives the
    same attention as a linear window holding the same tokens (joint softmax: row order
    does not matter), and both match the oracle."""
    vc, vs, sw_unused, sel, q = _attn_case(B=1, N=2000, k=64, seed=13)
    toks = synth.latent_rows(synth.key(14, 1, 0, P), synth.key(14, 2, 0, P), 0, P, 512)
    lo = max(0, P - 128)
    # linear window: every token row, attention over [P-128, P)
    lin = torch.zeros((1, P, 512), dtype=torch.uint8, device=dev())
    L.quantize_swa(t(toks), lin)
    # ring: replay only the last 128 tokens into slots p % 128
    ring = torch.zeros((1, 128, 512), dtype=torch.uint8, device=dev())
    p = np.arange(lo, P, dtype=np.int64)
    L.encode_entries(t(np.zeros((0, 512), np.float32)), *_entries_buffers(1, 1)[:4],
                     idx_x=t(np.zeros((0, 128), np.float32)), swa_x=t(toks[lo:]), swa_out=ring,
                     swa_dst=t(p % 128))
    o_lin, l_lin = _run_attn(q, vc, vs, sel, lin.cpu().numpy(), np.array([[P]], np.int32))
    o_ring, l_ring = _run_attn(q, vc, vs, sel, ring.cpu().numpy(),
                               np.array([[min(P, 128)]], np.int32))
    assert max_abs(o_ring, o_lin) <= 1e-5 and max_abs(l_ring, l_lin) <= 1e-5
    ro, rl = oracle.attention(q[0, 0], vc[0], vs[0], sel[0, 0], lin.cpu().numpy()[0], P, 128)
    assert max_abs(o_ring[0, 0], ro) <= ATTN_TOL and max_abs(l_ring[0, 0], rl) <= 1e-4


def test_sparse_attn_key_splits_repeated_calls_bit_identical():
    """Few rows: the key splits and their merge.  Three calls on one workspace (stale
    partials from the previous call) give bit-identical outputs that match the oracle."""
    vc, vs, sw, sel, q = _attn_case(B=3, N=2500, k=512, swa_cap=128, seed=21)
    B = 3
    swa_end = np.full((B, 1), 128, np.int32)
    n = L.sparse_attn_workspace(B, 1, 512, 128)
    assert n > 0
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device=dev())
    outs = []
    for rep in range(3):
        out = torch.full((B, 1, 64, 512), 777.0, device=dev())
        lse = torch.full((B, 1, 64), 777.0, device=dev())
        L.sparse_attn(t(q, torch.uint16), t(vc), t(vs), t(sel), t(sw), t(swa_end), out, lse, ws=ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
    for b in range(B):
        ro, rl = oracle.attention(q[b, 0], vc[b], vs[b], sel[b, 0], sw[b], 128, 128)
        assert max_abs(outs[0][0][b, 0], ro) <= ATTN_TOL
        assert max_abs(outs[0][1][b, 0], rl) <= 1e-4
