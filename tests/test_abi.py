"""The C-ABI library: it loads, exports every entry point include/csa2.h declares,
and rejects bad arguments on the host with the documented status before
touching the GPU.  CPU only (no compute call is made)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "csa2.h")

kv = pytest.importorskip("kv_cache_decode_mxfp4_amd")
L = kv._lib


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared()
    for n in ["csa2_quantize_kv", "csa2_index_full", "csa2_index_full_pool", "csa2_index_pool",
              "csa2_topk", "csa2_sparse_attn", "csa2_sparse_attn_rope_bf16",
              "csa2_encode_entries"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for n in declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True).stdout
    for n in declared():
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} not exported"
    assert set(declared()) == set(L.EXPORTS)


def test_version_and_workspace_queries():
    lib = L.load()
    assert lib.csa2_version() == 107
    assert lib.csa2_topk_workspace(16384, 16, 2048) == 0
    assert lib.csa2_topk_workspace(131072, 16, 2048) == 16 * 16384 * 4  # group maxima
    assert lib.csa2_topk_workspace(300000, 4, 2048) == 2 * 4 * 19 * 2048 * 8  # segment levels
    assert lib.csa2_topk_workspace(100, 1, 0) == 0
    assert lib.csa2_sparse_attn_workspace(4096, 1, 512, 128) == 0  # rows fill the CUs
    # 16 rows: 4 key splits per (row, 16 heads), each an O [16, 512] plus max and sum
    assert lib.csa2_sparse_attn_workspace(16, 1, 512, 128) == 16 * 4 * 4 * (16 * 512 + 32) * 4
    assert lib.csa2_sparse_attn_workspace(1, 1, 512, 128) == 8 * 4 * 8 * (16 * 512 + 32) * 4
    # sizes the calls reject (here more than 2^24 query rows, whose product would also
    # wrap in 32 bits) get 0, not a wrapped size
    assert lib.csa2_sparse_attn_workspace(1 << 16, 1 << 16, 512, 128) == 0
    assert lib.csa2_index_pool_topk_workspace(1 << 16, 1 << 16, 512) == 0
    assert lib.csa2_index_full_select_workspace(1 << 20, 1 << 16, 1 << 16, 2048, 512) == 0
    assert lib.csa2_index_pool_topk_workspace(1 << 12, 1 << 12, 512) > 0  # 2^24 rows: taken


def _status(fn, *args):
    lib = L.load()
    st = getattr(lib, fn)(*args)
    return st, lib.csa2_last_error().decode()


def test_host_validation_rejects_bad_arguments():
    vp = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    # channels not a multiple of 16
    st, msg = _status("csa2_quantize_kv", vp, 4, 15, None, None, 0, 0, vp, vp, 0, 1, None)
    assert st == 2 and "channels" in msg
    # rotary range outside the row
    st, msg = _status("csa2_quantize_kv", vp, 4, 512, vp, vp, 480, 64, vp, vp, 0, 1, None)
    assert st == 1 and "rotary" in msg
    # null pointers with work to do
    st, _ = _status("csa2_quantize_kv", None, 4, 512, None, None, 0, 0, None, None, 0, 1, None)
    assert st == 1
    # negative destination row
    st, msg = _status("csa2_quantize_kv", vp, 4, 128, None, None, 0, 0, vp, vp, -1, 1, None)
    assert st == 1 and "dst_row" in msg
    # unsupported block size
    st, msg = _status("csa2_index_full", vp, vp, vp, vp, 100, vp, 1, 1, 4, vp, None, None)
    assert st == 2 and "block" in msg
    # negative sizes
    st, _ = _status("csa2_index_pool", vp, vp, vp, vp, 100, vp, 8, 8, vp, -1, 1, vp, vp, None)
    assert st == 1
    # k out of range
    st, _ = _status("csa2_topk", vp, None, 100, 1, None, 0, vp, None, 0, None)
    assert st == 2
    st, _ = _status("csa2_topk", vp, None, 100, 1, None, 9000, vp, None, 0, None)
    assert st == 2
    # a long row needs a workspace
    st, msg = _status("csa2_topk", vp, None, 131072, 1, None, 512, vp, None, 0, None)
    assert st == 3 and "workspace" in msg
    # misaligned output pointer
    st, msg = _status("csa2_sparse_attn", vp, 16, 1, vp, vp, 100, vp, 512, vp, 128, vp, 128,
                      ctypes.c_float(1.0), ctypes.c_void_p(4100), None, None, 0, None)
    assert st == 1 and "misaligned" in msg
    # misaligned query pointer
    st, msg = _status("csa2_sparse_attn", ctypes.c_void_p(18), 1, 1, vp, vp, 100, vp, 4, vp, 128,
                      vp, 128, ctypes.c_float(1.0), vp, None, None, 0, None)
    assert st == 1 and "misaligned" in msg
    # caches beyond the 32-bit row offsets of the attention: over 2^24 main entries or
    # 2^22 window rows per sequence
    for n_cap, swa_cap in (((1 << 24) + 1, 128), (100, (1 << 22) + 1)):
        st, msg = _status("csa2_sparse_attn", vp, 1, 1, vp, vp, n_cap, vp, 4, vp, swa_cap, vp,
                          128, ctypes.c_float(1.0), vp, None, None, 0, None)
        assert st == 2 and "2^24" in msg, (st, msg)
    # the pool gathers' 32-bit offsets: over 2^24 entries per sequence (rejected before
    # anything is launched)
    big = (1 << 24) + 1
    st, msg = _status("csa2_index_pool", vp, vp, vp, vp, big, vp, 8, 8, vp, 1, 1, vp, vp, None)
    assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _status("csa2_index_pool_topk", vp, vp, vp, vp, big, vp, 8, 8, vp, 1, 1, 4, vp, vp,
                      ctypes.c_size_t(1 << 20), None)
    assert st == 2 and "2^24" in msg, (st, msg)
    st, msg = _status("csa2_index_full_select", vp, vp, vp, vp, big, vp, 1, 1, 8, 16, 4, vp, vp,
                      vp, vp, ctypes.c_size_t(1 << 30), None, None, None)
    assert st == 2 and "2^24" in msg, (st, msg)


def test_launches_beyond_one_dispatch_are_rejected():
    """A dispatch counts its grid in 32-bit work-items: every call whose launch would
    need more than 2^32 - 1 of them is rejected on the host (status 2) before
    anything is enqueued, one shape just past each launch's limit."""
    vp = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    big = ctypes.c_size_t(1 << 46)  # workspace size: never the reason
    f1 = ctypes.c_float(1.0)
    cases = {
        # one 256-thread workgroup per 16-channel group of 256 rows: 2^34 threads
        "quantize_kv": ("csa2_quantize_kv", vp, 1 << 29, 512, None, None, 0, 0, vp, vp, 0, 1,
                        None),
        "quantize_kv rows": ("csa2_quantize_kv", vp, 1 << 60, 4096, None, None, 0, 0, vp, vp, 0,
                             1, None),
        "quantize_swa": ("csa2_quantize_swa", vp, 1 << 34, 512, vp, 1, None),
        "encode_entries": ("csa2_encode_entries", 1 << 27, vp, None, None, 0, 0, vp, vp, 1,
                           None, 0, 1 << 27, vp, None, vp, vp, 1, None, None, 0, None, 1, None,
                           0, None),
        # one-row scan: 256 rows x 65536 chunks of 16384 entries = 2^24 workgroups
        "index_full": ("csa2_index_full", vp, vp, vp, vp, 1 << 30, vp, 256, 1, 8, vp, None,
                       None),
        # multi-row scan: 2^21 groups of 8 rows x 256 chunks
        "index_full rows": ("csa2_index_full", vp, vp, vp, vp, 1 << 20, vp, 1, 1 << 24, 8, vp,
                            None, None),
        "index_full_pool": ("csa2_index_full_pool", vp, vp, vp, vp, 65536, vp, 1 << 22, 1, 8, 16,
                            vp, vp, vp, big, None, None, None),
        # 2^22 rows: the scan and the block select (2 x 1024 threads per row)
        "index_full_select": ("csa2_index_full_select", vp, vp, vp, vp, 65536, vp, 1 << 22, 1, 8,
                              16, 4, vp, vp, vp, vp, big, None, None, None),
        # 4096 rows x 8192 workgroups of 2^20 blocks' positions
        "index_pool": ("csa2_index_pool", vp, vp, vp, vp, 1 << 24, vp, 1 << 20, 8, vp, 4096, 1,
                       vp, vp, None),
        # 2^18 rows x 16 workgroups of 1024 threads
        "index_pool_topk": ("csa2_index_pool_topk", vp, vp, vp, vp, 1 << 24, vp, 2048, 8, vp,
                            1 << 18, 1, 512, vp, vp, big, None),
        # one 1024-thread workgroup per row
        "topk": ("csa2_topk", vp, None, 4096, 1 << 22, None, 8, vp, None, 0, None),
        "topk_noalloc": ("csa2_topk_noalloc", vp, None, 4096, 1 << 22, None, 8, vp, None),
        # one 512-thread workgroup per row and its 64 heads
        "sparse_attn": ("csa2_sparse_attn", vp, 1, 1 << 23, vp, vp, 100, vp, 4, vp, 128, vp, 128,
                        f1, vp, None, None, 0, None),
    }
    for name, (fn, *args) in cases.items():
        st, msg = _status(fn, *args)
        assert st == 2 and "2^32 - 1 work-items" in msg, (name, st, msg)
    # the limit itself: rows of 131072 keys take their group maxima at one thread per 4
    # keys, 2^15 per row, so 2^17 - 1 rows fit (the call then stops at its missing
    # workspace, before any launch) and 2^17 do not
    st, msg = _status("csa2_topk", vp, None, 131072, (1 << 17) - 1, None, 8, vp, None, 0, None)
    assert st == 3 and "workspace" in msg, (st, msg)
    st, msg = _status("csa2_topk", vp, None, 131072, 1 << 17, None, 8, vp, None, 0, None)
    assert st == 2 and "2^32 - 1 work-items" in msg, (st, msg)


def test_empty_inputs_are_no_ops():
    assert _status("csa2_quantize_kv", None, 0, 512, None, None, 0, 0, None, None, 0, 1,
                   None)[0] == 0
    assert _status("csa2_index_full", None, None, None, None, 0, None, 0, 1, 8, None, None,
                   None)[0] == 0
    assert _status("csa2_topk", None, None, 0, 0, None, 5, None, None, 0, None)[0] == 0
    assert _status("csa2_sparse_attn", None, 0, 1, None, None, 0, None, 0, None, 0, None, 128,
                   ctypes.c_float(1.0), None, None, None, 0, None)[0] == 0


def _rope_attn(q=16, out=16, cos=16, sin=16, off=448, dim=64, B=1):
    vp = ctypes.c_void_p
    return _status("csa2_sparse_attn_rope_bf16", vp(q), B, 1, vp(16), vp(16), 100, vp(16), 4,
                   vp(16), 128, vp(16), 128, ctypes.c_float(1.0), vp(cos), vp(sin), off, dim,
                   vp(out), None, None, 0, None)


def test_rope_bf16_attention_validation():
    st, msg = _rope_attn(off=447)
    assert st == 1 and "rotary" in msg
    st, msg = _rope_attn(off=480, dim=64)
    assert st == 1 and "rotary" in msg
    st, msg = _rope_attn(cos=None)
    assert st == 1 and "rotary table" in msg
    st, msg = _rope_attn(out=4)
    assert st == 1 and "misaligned" in msg
    st, msg = _rope_attn(out=None)
    assert st == 1
    assert _rope_attn(B=0, out=None, cos=None, sin=None)[0] == 0


def _entries(rows=4, kv_x=16, idx_x=16, w=None, off=448, dim=64, cos=16, swa_rows=0, swa_x=None,
             kv_stride=1, dst=None, dst_row=0):
    vp = ctypes.c_void_p
    return _status("csa2_encode_entries", rows, vp(kv_x), vp(cos), vp(cos), off, dim, vp(16),
                   vp(16), kv_stride, None, dst_row, 0, vp(idx_x), vp(w), vp(16), vp(16), 1, None,
                   vp(swa_x), swa_rows, vp(16), 1, vp(dst), 10, None)


def test_encode_entries_validation():
    st, msg = _entries(idx_x=None, w=None)
    assert st == 1 and "projection" in msg
    st, msg = _entries(off=447)
    assert st == 1 and "rotary" in msg
    st, msg = _entries(kv_x=20)
    assert st == 1 and "misaligned" in msg
    st, msg = _entries(swa_rows=2, swa_x=None)
    assert st == 1 and "window" in msg
    st, msg = _entries(kv_stride=0)
    assert st == 1
    st, msg = _entries(dst=12)
    assert st == 1 and "destination" in msg
    st, msg = _entries(dst_row=-2)
    assert st == 1 and "dst_row" in msg
    assert _entries(rows=0, kv_x=None, idx_x=None, cos=None)[0] == 0


def test_key_tile_helpers_follow_the_documented_layout():
    """The tests' row <-> key-tile permutations place byte j of entry f at
    (f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16 and invert each other."""
    import numpy as np
    from gpu_harness import tile_keys, untile_keys
    rng = np.random.default_rng(3)
    rows = 77
    codes = rng.integers(0, 256, (rows, 64), dtype=np.uint8)
    tiled = tile_keys(codes)
    assert tiled.shape == (3, 2048)
    flat = tiled.reshape(-1)
    for f in range(rows):
        for j in range(64):
            assert flat[(f // 32) * 2048 + (j // 16) * 512 + (f % 32) * 16 + j % 16] == codes[f, j]
    assert np.array_equal(untile_keys(tiled, rows), codes)
    assert not untile_keys(tiled, 96)[rows:].any()  # padding entries are zero
    assert L.key_code_bytes(rows) == 3 * 2048 and L.key_code_bytes(64) == 2 * 2048


def test_index_full_pool_validation():
    vp = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    args = lambda nb, ws_bytes, block=8: ("csa2_index_full_pool", vp, vp, vp, vp, 1 << 20, vp, 16,
                                          1, block, nb, vp, vp, vp, ws_bytes, None, None, None)
    st, msg = _status(*args(0, 1 << 30))
    assert st == 2 and "nb" in msg
    st, msg = _status(*args(9000, 1 << 30))
    assert st == 2
    st, msg = _status(*args(2048, 1 << 30, block=4))
    assert st == 2 and "block" in msg
    need = L.index_full_pool_workspace(1 << 20, 16, 2048)
    assert need == L.topk_workspace(1 << 17, 16, 2048) and need > 0
    st, msg = _status(*args(2048, need - 1))
    assert st == 3 and "workspace" in msg
    # nothing to do: no rows
    assert _status("csa2_index_full_pool", None, None, None, None, 100, None, 0, 1, 8, 64, None,
                   None, None, 0, None, None, None)[0] == 0


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on exactly one GPU: --gpus above 1 exits with a message (before any
    GPU work)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_topk_noalloc_rejects_workspace_above_static_size():
    """csa2_topk_noalloc refuses, on the host, a call whose workspace would exceed its
    8 MiB static device array (nothing is enqueued, no GPU needed)."""
    lib = L.load()
    vp = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    # 64 rows x 131072 keys, k 2048: group maxima of 64 x 16384 x 4 B = 4 MiB (fits);
    # 256 rows: 16 MiB (does not fit)
    assert lib.csa2_topk_workspace(131072, 256, 2048) > 8 << 20
    st, msg = _status("csa2_topk_noalloc", vp, None, 131072, 256, None, 2048, vp, None)
    assert st == 3 and "static" in msg
    st, msg = _status("csa2_topk_noalloc", vp, None, 100, 1, None, 0, vp, None)
    assert st == 2


def test_bindings_reject_undersized_or_mistyped_tensors_before_any_call():
    """Every binding checks each tensor's dtype and element count against the shape
    include/csa2.h documents, before it takes a pointer: an undersized output raises
    here instead of becoming an out-of-bounds device write.  (CPU tensors: the checks
    fail before the device check would.)"""
    import torch
    u8, i32, f32, bf = torch.uint8, torch.int32, torch.float32, torch.bfloat16
    B, nq, n_cap, k, nb = 2, 1, 4096, 64, 32
    q = torch.zeros(B, nq, 32, 128, dtype=bf)
    w = torch.zeros(B, nq, 32, dtype=f32)
    kc = torch.zeros(L.key_code_bytes(B * n_cap), dtype=u8)
    ks = torch.zeros(B, n_cap, 8, dtype=u8)
    nv = torch.zeros(B, nq, dtype=i32)
    bm = torch.zeros(B, nq, n_cap // 8, dtype=f32)

    def expect(fn, *a, match="elements", **kw):
        with pytest.raises((ValueError, TypeError), match=match):
            fn(*a, **kw)

    expect(L.index_full, q, w, kc, ks, nv, bm[:, :, :-1].contiguous())          # block maxima
    expect(L.index_full, q, w, kc, ks, nv, bm, scores=torch.zeros(B * n_cap - 1))
    expect(L.index_full, q, w[:1].contiguous(), kc, ks, nv, bm)                   # weights
    expect(L.index_full, q, w, kc, ks, nv.to(torch.int64), bm, match="int32")
    sel = torch.zeros(B, nq, k, dtype=i32)
    expect(L.index_full_select, q, w, kc, ks, nv, bm, sel[:1].contiguous())
    expect(L.index_full_select, q, w, kc, ks, nv, bm, sel,
           pool=torch.zeros(B - 1, nq, nb, dtype=i32))
    blocks = torch.zeros(B, nq, nb, dtype=i32)
    ps, pi = torch.zeros(B, nq, nb * 8, dtype=f32), torch.zeros(B, nq, nb * 8, dtype=i32)
    expect(L.index_pool, q, w, kc, ks, blocks, nv, ps[:, :, :-1].contiguous(), pi)
    expect(L.index_pool, q, w, kc, ks, blocks, nv, ps, pi[:, :, :-1].contiguous())
    expect(L.index_pool, q, w, kc, ks, blocks, nv[:1].contiguous(), ps, pi)
    sc = torch.zeros(3, 100, dtype=f32)
    expect(L.topk, sc, 10, torch.zeros(3, 9, dtype=i32))                          # out
    expect(L.topk, sc, 10, torch.zeros(3, 10, dtype=i32), idx=torch.zeros(3, 99, dtype=i32))
    expect(L.topk, sc, 10, torch.zeros(3, 10, dtype=i32), n_valid=torch.zeros(2, dtype=i32))
    expect(L.topk_noalloc, sc, 10, torch.zeros(3, 10, dtype=torch.int64), match="int32")
    qm = torch.zeros(B, nq, 64, 512, dtype=bf)
    vc, vs = torch.zeros(B, n_cap, 256, dtype=u8), torch.zeros(B, n_cap, 32, dtype=u8)
    tk = torch.zeros(B, nq, k, dtype=i32)
    sw, se = torch.zeros(B, 128, 512, dtype=u8), torch.zeros(B, nq, dtype=i32)
    out = torch.zeros(B, nq, 64, 512, dtype=f32)
    expect(L.sparse_attn, qm, vc, vs, tk, sw, se, out[:1].contiguous())
    expect(L.sparse_attn, qm, vc, vs, tk, sw, se, out, lse=torch.zeros(B * nq * 64 - 1))
    expect(L.sparse_attn, qm, vc, vs[:, :-1].contiguous(), tk, sw, se, out)
    expect(L.sparse_attn, qm, vc, vs, tk, sw, se[:, :0].contiguous(), out)
    expect(L.sparse_attn_rope_bf16, qm, vc, vs, tk, sw, se, torch.zeros(B * nq, 31),
           torch.zeros(B * nq, 32), torch.zeros(B, nq, 64, 512, dtype=bf))        # rotary table
    expect(L.sparse_attn_rope_bf16, qm, vc, vs, tk, sw, se, torch.zeros(B * nq, 32),
           torch.zeros(B * nq, 32), torch.zeros(B, nq, 64, 511, dtype=bf))
    x = torch.zeros(4, 512, dtype=f32)
    expect(L.encode_entries, x, vc.view(-1, 256), vs.view(-1, 32), kc, ks.view(-1, 8),
           idx_x=torch.zeros(3, 128), kv_dst=torch.zeros(4, dtype=torch.int64))
    expect(L.encode_entries, x, vc.view(-1, 256), vs.view(-1, 32), kc, ks.view(-1, 8),
           idx_x=torch.zeros(4, 128), kv_dst=torch.zeros(3, dtype=torch.int64))
    expect(L.quantize_kv, x, vc.view(-1), vs.view(-1), torch.zeros(4, 31), torch.zeros(4, 32),
           448, 64)
