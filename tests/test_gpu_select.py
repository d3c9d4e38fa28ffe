"""csa2_index_full_select (the Full layer's scan, pool and top-k in one call) against
the same scan's per-entry scores: bit-exact pools (csa2_topk over the block maxima) and
top-k positions (csa2_topk over every score of the row: the literal full-range
definition, on the same fp32 scores), on shapes that take each of its paths -- the
direct block select (rows of at most 16384 blocks), the scan's per-chunk block
candidates and their exact fallback (a chunk holding more winners than it listed: a
planted cluster of strong keys, and exact ties from a zero query or a periodic cache),
csa2_topk calls (rows too long for the candidates); the top-k blocks' positions
rescored in one launch (few rows) or by a pool scan and csa2_topk (many rows) -- with
ragged, empty and stale-workspace rows.  csa2_topk itself is checked against the
oracle's selection in test_gpu_stages.py."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import cdiv, dev, t

pytestmark = pytest.mark.gpu

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
L = kv._lib

STRONG = 0x77  # code byte: both nibbles +6; as a scale byte: E4M3 240


def _caches(B, n_cap, seed, kind):
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    codes = torch.randint(0, 256, (B, n_cap, 64), dtype=torch.uint8, device=dev(), generator=g)
    scales = (torch.randint(0, 256, (B, n_cap, 8), dtype=torch.uint8, device=dev(), generator=g)
              & 0x77) | 0x30  # finite E4M3 scales
    if kind == "cluster":
        # 300 blocks of the strongest key in a row: more winners in one scan chunk than
        # it lists as candidates
        a = n_cap // 3 // 8 * 8
        codes[0, a:a + 2400] = STRONG
        scales[0, a:a + 2400] = STRONG
    elif kind == "periodic":
        # every key repeats 4096 entries later: exact score ties across blocks
        for b in range(B):
            base = codes[b, :4096].clone(), scales[b, :4096].clone()
            for s in range(4096, n_cap, 4096):
                n = min(4096, n_cap - s)
                codes[b, s:s + n] = base[0][:n]
                scales[b, s:s + n] = base[1][:n]
    # the library's tiled indexer-key layout: byte j of entry f at
    # (f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16
    flat = codes.reshape(-1, 64)
    n = flat.shape[0]
    tiles = cdiv(n, 32)
    pad = torch.zeros((tiles * 32, 64), dtype=torch.uint8, device=dev())
    pad[:n] = flat
    kc = pad.reshape(tiles, 32, 4, 16).permute(0, 2, 1, 3).contiguous().reshape(-1)
    return kc, scales


CASES = [
    # (B, nq, n_cap, nb, k, n_visible, kind)
    (16, 1, 1 << 20, 2048, 512, None, "random"),                  # the 1M decode shape: candidates
    (8, 1, 262144, 2048, 512, None, "random"),                    # groups of 2: candidates
    (8, 1, 262144, 2048, 512, [262144, 200001, 131073, 131072, 70000, 9, 0, 262143], "random"),
    (4, 1, 262144, 2048, 512, None, "cluster"),                   # fallback in row 0
    (4, 1, 262144, 2048, 512, None, "zero_query"),                # all ties: fallback
    (4, 1, 262144, 2048, 512, None, "periodic"),                  # exact ties across blocks
    (16, 1, 1 << 20, 2048, 512, None, "periodic"),
    (40, 1, 262144, 2048, 512, None, "random"),                   # candidates; rescoring by pool scan + top-k
    (64, 1, 65536, 2048, 512, None, "random"),                    # direct select; pool scan + top-k
    (2, 1, 140003, 2048, 512, [140003, 70001], "random"),          # too many chunks: two top-k calls
    (3, 1, 65536, 2048, 512, [65536, 40001, 3], "random"),         # direct select
    (1, 4, 300000, 2048, 512, [300000, 299999, 150000, 5], "random"),  # multi-row scan rows
    (2, 1, 2048, 32, 64, [2048, 1000], "random"),                 # pool smaller than k
    (2, 1, 262144, 0, 512, None, "random"),                       # no pool
    (1, 1, 0, 2048, 512, [5], "random"),                          # empty cache
    (1, 1, 1 << 24, 2048, 512, None, "random"),                   # the most a gathering call takes
]


@pytest.mark.parametrize("B,nq,n_cap,nb,k,nvis,kind", CASES)
def test_index_full_select_matches_scan_then_topk(B, nq, n_cap, nb, k, nvis, kind):
    print(f"[case] B={B} nq={nq} n_cap={n_cap} nb={nb} k={k} kind={kind}", flush=True)
    kc, ks = _caches(B, n_cap, seed=n_cap + nb + len(kind), kind=kind)
    q = synth.normal_bf16(synth.key(21, 1, 0, 0), 0, B * nq * 4096, 1 / np.sqrt(128)).reshape(B, nq, 32, 128)
    if kind == "zero_query":
        q[:] = 0
    w = synth.uniform_f32(synth.key(21, 2, 0, 0), 0, B * nq * 32).reshape(B, nq, 32)
    nv = np.full((B, nq), n_cap, np.int32) if nvis is None else np.array(nvis, np.int32).reshape(B, nq)
    nblk = cdiv(n_cap, 8)
    qd, wd, nvd = t(q, torch.uint16), t(w), t(nv)

    ws_n = L.index_full_select_workspace(n_cap, B, nq, nb, k)
    ws = torch.full((max(ws_n, 256),), 0xC3, dtype=torch.uint8, device=dev())  # stale contents
    bm1 = torch.full((B, nq, max(nblk, 1)), 777.0, device=dev())
    pool1 = torch.full((B, nq, max(nb, 1)), -7, dtype=torch.int32, device=dev())
    top1 = torch.full((B, nq, k), -7, dtype=torch.int32, device=dev())
    for rep in range(2):  # the second call finds the first call's workspace contents
        L.index_full_select(qd, wd, kc, ks, nvd, bm1, top1, pool=pool1 if nb else None, ws=ws)
    torch.cuda.synchronize()

    # the same scan with every score, then csa2_topk over the scores and block maxima
    bm2 = torch.full((B, nq, max(nblk, 1)), 777.0, device=dev())
    sc = torch.full((B, nq, max(n_cap, 1)), -1.0, device=dev())
    if n_cap:
        L.index_full(qd, wd, kc, ks, nvd, bm2, scores=sc)
    nvb = t(((np.maximum(nv.astype(np.int64), 0) + 7) // 8).astype(np.int32))
    nve = t(np.clip(nv, 0, n_cap).astype(np.int32))
    tw_n = max(L.topk_workspace(max(n_cap, 1), B * nq, k), L.topk_workspace(max(nblk, 1), B * nq, max(nb, 1)))
    tw = torch.empty(max(tw_n, 8), dtype=torch.uint8, device=dev())
    top2 = torch.full((B, nq, k), -7, dtype=torch.int32, device=dev())
    L.topk(sc if n_cap else sc[..., :0].contiguous(), k, top2, n_valid=nve, ws=tw)
    assert np.array_equal(bm1.cpu().numpy()[..., :nblk], bm2.cpu().numpy()[..., :nblk])
    t1, t2 = top1.cpu().numpy(), top2.cpu().numpy()
    assert np.array_equal(t1, t2), f"top-k differs in {int((t1 != t2).any(-1).sum())} rows"
    if nb:
        pool2 = torch.full((B, nq, nb), -7, dtype=torch.int32, device=dev())
        L.topk(bm2[..., :nblk], nb, pool2, n_valid=nvb, ws=tw)
        p1 = pool1.cpu().numpy()
        assert np.array_equal(p1, pool2.cpu().numpy()), "pools differ"
        # the top-k positions lie in the pool when the pool has at least k blocks
        if nb >= k:
            for r in range(B * nq):
                tr = t1.reshape(-1, k)[r]
                assert set((tr[tr >= 0] // 8).tolist()) <= set(p1.reshape(-1, nb)[r].tolist())


POOL_CASES = [
    # (B, nq, n_cap, n_blocks, k, n_visible): decode Full (k blocks) and Reindex (pool) sizes
    (16, 1, 1 << 20, 512, 512, None),
    (16, 1, 1 << 20, 2048, 512, None),
    (5, 1, 100000, 2048, 512, [100000, 50001, 4000, 7, 0]),   # blocks past the visible end
    (3, 1, 65536, 64, 512, None),                             # fewer positions than k
    (1, 64, 40000, 2048, 512, "causal"),                      # decoder prefill rows
    (2, 1, 20000, 1, 8, None),                                # a single block
    (3, 1, 50003, 2048, 512, [50003, 20001, 0]),              # sequences start inside key tiles
    (1, 1, 1 << 24, 2048, 512, None),                         # 32-bit gather offsets near 2^30 bytes
]


@pytest.mark.parametrize("B,nq,n_cap,nbk,k,nvis", POOL_CASES)
def test_index_pool_topk_matches_pool_scan_then_topk(B, nq, n_cap, nbk, k, nvis):
    """csa2_index_pool_topk (rescoring and top-k in one launch; the last workgroup of a
    row selects) gives exactly csa2_index_pool then csa2_topk, on consecutive calls that
    reuse one workspace (its arrival counters return to zero)."""
    print(f"[case] B={B} nq={nq} n_cap={n_cap} n_blocks={nbk} k={k}", flush=True)
    kc, ks = _caches(B, n_cap, seed=n_cap + nbk, kind="random")
    rng = np.random.default_rng(nbk + k)
    rows = B * nq
    if nvis is None:
        nv = np.full((B, nq), n_cap, np.int32)
    elif nvis == "causal":
        nv = (n_cap - nq + 1 + np.arange(nq, dtype=np.int32))[None, :].repeat(B, 0)
    else:
        nv = np.array(nvis, np.int32).reshape(B, nq)
    nblk = cdiv(n_cap, 8)
    blocks = np.full((rows, nbk), -1, np.int32)
    for r in range(rows):
        m = min(nbk, nblk) - (r % 3)  # some rows padded with -1
        if m > 0:
            blocks[r, :m] = np.sort(rng.choice(nblk, m, replace=False))
    blocks = blocks.reshape(B, nq, nbk)
    qd = t(synth.normal_bf16(synth.key(22, 1, 0, 0), 0, rows * 4096, 1 / np.sqrt(128))
           .reshape(B, nq, 32, 128), torch.uint16)
    wd = t(synth.uniform_f32(synth.key(22, 2, 0, 0), 0, rows * 32).reshape(B, nq, 32))
    nvd, bd = t(nv), t(blocks)

    ps = torch.empty(B, nq, nbk * 8, device=dev())
    pi = torch.empty(B, nq, nbk * 8, dtype=torch.int32, device=dev())
    L.index_pool(qd, wd, kc, ks, bd, nvd, ps, pi)
    ref = torch.full((B, nq, k), -7, dtype=torch.int32, device=dev())
    tw = torch.empty(max(L.topk_workspace(nbk * 8, rows, k), 8), dtype=torch.uint8, device=dev())
    L.topk(ps, k, ref, idx=pi, ws=tw)
    ws = torch.zeros(L.index_pool_topk_workspace(B, nq, max(nbk, 2048)), dtype=torch.uint8,
                     device=dev())
    for rep in range(3):
        got = torch.full((B, nq, k), -7, dtype=torch.int32, device=dev())
        L.index_pool_topk(qd, wd, kc, ks, bd, nvd, got, ws)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy()), f"call {rep}"
    cnt = ws[: 4 * rows].view(torch.int32).cpu().numpy()
    assert np.all(cnt == 0), "arrival counters not returned to zero"
