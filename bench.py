#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X.

Metric: CSA2 decode queries/s per layer at 1M context, with the achieved HBM
bandwidth of the dominant kernel (the Full-layer indexer scan) against the
MI355X peak.  Workload (default): 16 sequences x 1,048,576 compressed entries,
indexer 32 heads x 128, top-k 512, pool 2048 blocks x 8, attention 64 heads x
512 over MXFP4 main KV + 128 FP8 window rows.  Inputs are seeded synthetic
(synth/), resident in HBM before the timed region.

One step = one Full layer at decode for the whole batch: encode the new
token's main-KV, indexer-key and window rows; block scan over every entry;
pool select (top-2048 blocks); pool rescoring; top-512; sparse attention.

    python bench.py [--steps K] [--warmup W] [--config 3] [--cpu-sample 16]

Prints one JSON line.  Only one GPU is supported (--gpus above 1 exits).
Before the W warm-up steps, the step runs untimed for at least --prewarm-ms
of wall time (default 500 ms): under sustained load an MI355X reaches its
steady step time only after ~100 ms, so a short --warmup alone would time the
ramp.  The pre-warm is reported as its own JSON field (its step count and the
mean step time of its first and last ten steps).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "CSA2 decode queries/sec per layer at 1M ctx; achieved HBM TB/s vs peak"
PEAK_HBM = 8.0e12  # MI355X HBM3E, bytes/s
PEAK_F16 = 2.5e15  # MI355X dense fp16 MFMA, flop/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_full_scan_1M_b16_traffic.txt")
# what the scan kernel is compiled from: its source, the device headers it includes
# and the build script (flags); the traffic counters are valid only for this exact
# input (launch.h holds only host launcher declarations)
SCAN_SOURCES = [os.path.join(ROOT, "kv_cache_decode_mxfp4_amd", *p) for p in (
    ("csrc", "indexer.hip"), ("csrc", "score.h"), ("csrc", "select.h"),
    ("csrc", "device_common.h"), ("csrc", "dims.h"), ("build.py",))]
CHUNK_ROWS = 1 << 18
SCAN_EVENT_EVERY = 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="untimed steps for at least this much wall time before the warm-up "
                         "steps (reported as 'prewarm'; 0 = none)")
    ap.add_argument("--ceiling-reps", type=int, default=10,
                    help="launches per setting of the streaming-read ceiling (0 = skip)")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cold-steps", type=int, default=50,
                    help="steps timed one by one after a 512 MiB cache-evicting write each "
                         "(median / p10 / p90 reported beside value; 0 = skip)")
    ap.add_argument("--cpu-sample", type=int, default=16,
                    help="query rows of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--overlap-steps", type=int, default=0,
                    help="decode workloads: also time this many steps alternating between two "
                         "independent batches on two streams (0: skip); reported apart from value")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--kv-production", choices=["rows", "project"], default="rows",
                    help="indexer key of each new entry: its own synthetic row (default), or "
                         "projected from the new main-KV latent by a bf16 [128, 512] matrix")
    ap.add_argument("--attn-out", choices=["fp32", "bf16"], default="fp32",
                    help="attention output: fp32 (default), or rotated back by the query's "
                         "position and cast to bf16 in the kernel epilogue")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload on the GPU

def build_device(w: synth.Workload, torch, L):
    """Encode the whole cache of every sequence on the GPU from synth rows."""
    dev = torch.device("cuda:0")
    B, N = w.B, w.n_cap
    st = {"w": w}
    st["kc"] = L.key_codes_empty(B * N, device=dev)  # tiled indexer-key codes
    st["ks"] = torch.empty(B, N, 8, dtype=torch.uint8, device=dev)
    st["vc"] = torch.empty(B, N, 256, dtype=torch.uint8, device=dev)
    st["vs"] = torch.empty(B, N, 32, dtype=torch.uint8, device=dev)
    t0 = time.time()
    for r0 in range(0, N, CHUNK_ROWS):
        n = min(CHUNK_ROWS, N - r0)
        cos, sin = synth.rope_rows(r0, n)
        cos_d, sin_d = torch.from_numpy(cos).to(dev), torch.from_numpy(sin).to(dev)
        for b in range(B):
            kx = torch.from_numpy(synth.idx_k_rows(w, b, r0, n)).to(dev)
            L.quantize_kv(kx, st["kc"], st["ks"], dst_row=b * N + r0)
            vx = torch.from_numpy(synth.kv_rows(w, b, r0, n)).to(dev)
            L.quantize_kv(vx, st["vc"][b], st["vs"][b], cos_d, sin_d, synth.ROPE_OFFSET,
                          synth.ROPE_DIM, dst_row=r0)
        torch.cuda.synchronize()
        log(f"caches: {min(r0 + n, N)}/{N} entries x {B} sequences ({time.time() - t0:.0f} s)")
    n_layers = len(w.layers)
    st["swa"], st["q_idx"], st["w_idx"], st["q_main"] = [], [], [], []
    for layer in range(n_layers):
        sw = torch.empty(B, w.swa_rows(), 512, dtype=torch.uint8, device=dev)
        for b in range(B):
            L.quantize_swa(torch.from_numpy(synth.swa_rows(w, layer, b, 0, w.swa_rows())).to(dev), sw[b])
        st["swa"].append(sw)
        st["q_idx"].append(torch.from_numpy(synth.q_idx(w, layer)).to(dev))
        st["w_idx"].append(torch.from_numpy(synth.w_idx(w, layer)).to(dev))
        st["q_main"].append(torch.from_numpy(synth.q_main(w, layer)).to(dev))
    st["n_vis"] = torch.from_numpy(w.n_visible()).to(dev)
    st["swa_end"] = torch.from_numpy(w.swa_end()).to(dev)
    # rows the step encodes: the entries this step appends, and the newest window row
    first, count = w.new_entries()
    st["new_first"], st["new_count"] = first, count
    st["new_idx"] = torch.from_numpy(np.concatenate(
        [synth.idx_k_rows(w, b, first, count) for b in range(B)])).to(dev)
    st["new_kv"] = torch.from_numpy(np.concatenate(
        [synth.kv_rows(w, b, first, count) for b in range(B)])).to(dev)
    cos, sin = synth.rope_rows(first, count)
    st["new_cos"] = torch.from_numpy(np.tile(cos, (B, 1))).to(dev)
    st["new_sin"] = torch.from_numpy(np.tile(sin, (B, 1))).to(dev)
    new_tok = w.chunk if not w.decode else 1
    st["new_swa_row"] = w.swa_rows() - new_tok
    # per-sequence destinations of the new rows (each sequence's own append position and
    # its window slot; the decode window is the ring slot of the newest token)
    st["kv_dst"] = torch.from_numpy((np.arange(B, dtype=np.int64)[:, None] * N + first +
                                     np.arange(count)[None, :]).reshape(-1)).to(dev)
    st["swa_dst"] = torch.from_numpy((np.arange(B, dtype=np.int64)[:, None] * w.swa_rows() +
                                      st["new_swa_row"] + np.arange(new_tok)[None, :])
                                     .reshape(-1)).to(dev)
    st["w_proj"] = torch.from_numpy(synth.w_proj(w)).to(dev)
    # rotary angles of each query row's own position (its last visible entry), for the
    # bf16 output epilogue
    qpos = (w.n_visible().reshape(-1).astype(np.int64) - 1)
    p0 = int(qpos.min())
    qc, qs = synth.rope_rows(p0, int(qpos.max()) - p0 + 1)
    st["q_cos"] = torch.from_numpy(np.ascontiguousarray(qc[qpos - p0])).to(dev)
    st["q_sin"] = torch.from_numpy(np.ascontiguousarray(qs[qpos - p0])).to(dev)
    st["new_swa"] = torch.from_numpy(np.concatenate(
        [synth.swa_rows(w, 0, b, st["new_swa_row"], new_tok) for b in range(B)])).to(dev)
    torch.cuda.synchronize()
    return st


def make_step(st, torch, L, layers, kv_production="rows", attn_out="fp32"):
    """The timed step: one layer group of the workload over the whole batch."""
    w = st["w"]
    B, nq, N = w.B, w.nq, w.n_cap
    from kv_cache_decode_mxfp4_amd.layers import Buffers, n_valid_blocks
    buf = Buffers.create(B, nq, N, w.k, w.nb, w.n_win)
    n_blk = n_valid_blocks(st["n_vis"])
    first, count = st["new_first"], st["new_count"]
    st["buf"] = buf
    scan_events = []

    def encode_new():
        if w.decode:
            # one launch: per sequence, the main-KV and indexer-key entry N-1 of its
            # [N]-row caches and the newest (ring) row of its window
            project = kv_production == "project"
            L.encode_entries(st["new_kv"], st["vc"], st["vs"], st["kc"], st["ks"],
                             idx_x=None if project else st["new_idx"],
                             w_idx=st["w_proj"] if project else None,
                             rope_cos=st["new_cos"], rope_sin=st["new_sin"],
                             rope_offset=synth.ROPE_OFFSET, rope_dim=synth.ROPE_DIM,
                             kv_dst=st["kv_dst"], swa_x=st["new_swa"], swa_out=st["swa"][0],
                             swa_dst=st["swa_dst"])
        else:
            L.quantize_kv(st["new_idx"], st["kc"], st["ks"], dst_row=first)
            L.quantize_kv(st["new_kv"], st["vc"], st["vs"], st["new_cos"], st["new_sin"],
                          synth.ROPE_OFFSET, synth.ROPE_DIM, dst_row=first)
            L.quantize_swa(st["new_swa"], st["swa"][0], dst_row=st["new_swa_row"])

    out16 = (torch.empty(B, nq, 64, 512, dtype=torch.int16, device=buf.out.device)
             if attn_out == "bf16" else None)

    def attn(layer):
        layers.attention(buf, st["q_main"][layer], st["vc"], st["vs"], buf.topk, st["swa"][layer],
                         st["swa_end"], w.n_win, out_bf16=out16, rope_cos=st["q_cos"],
                         rope_sin=st["q_sin"])

    def event_pair():
        # created (by one record) before use: the library's scan dispatch records them
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for e in pair:
            e.record()
        return pair

    spare_events = []

    def prepare_scan_events(n):
        spare_events.extend(event_pair() for _ in range(n))
        torch.cuda.synchronize()

    layer_events = []  # per sampled step of a multi-layer group: events at layer boundaries

    def mark(evl):
        if evl is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            evl.append(e)

    def step(time_scan=False):
        evl = [] if time_scan and len(w.layers) > 1 else None
        mark(evl)
        encode_new()
        evs = None
        if time_scan:
            evs = spare_events.pop() if spare_events else event_pair()
            scan_events.append(evs)
        # scan + pool + top-k blocks in one call (the scan kernel's own dispatch records
        # the timing events), then the top-k blocks' positions rescored and the top-k
        layers.full_indexer(buf, st["q_idx"][0], st["w_idx"][0], st["kc"], st["ks"],
                            st["n_vis"], n_blk, w.k, w.nb, scan_events=evs)
        attn(0)
        mark(evl)
        if "reindex" in w.layers:
            layers.reindex_indexer(buf, st["q_idx"][1], st["w_idx"][1], st["kc"], st["ks"],
                                   st["n_vis"], buf.pool, w.k)
            for layer in range(1, len(w.layers)):
                attn(layer)
                mark(evl)
        if evl is not None:
            layer_events.append(evl)

    step.prepare_scan_events = prepare_scan_events
    step.layer_events = layer_events
    return step, scan_events


def overlap_run(w, step, n, torch, L, layers, kv_production, attn_out):
    """Two independent batches of the same workload (their own caches, buffers and
    inputs), their steps issued alternately on two streams, so that one batch's
    latency-bound chain (select, pool scan, top-k, attention) runs beside the other
    batch's HBM-bound scan.  Each step still runs the whole path for its batch; the
    rate is whole-job throughput over n steps.  Not the headline value: a serving
    loop gets it only when it has two independent micro-batches in flight."""
    st2 = build_device(w, torch, L)
    step2, _ = make_step(st2, torch, L, layers, kv_production, attn_out)
    side = torch.cuda.Stream()  # default priority
    main = torch.cuda.current_stream()
    with torch.cuda.stream(side):
        for _ in range(20):
            step2()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    joined = torch.cuda.Event()
    t0.record(main)
    side.wait_event(t0)
    for i in range(n):
        if i % 2 == 0:
            step()
        else:
            with torch.cuda.stream(side):
                step2()
    joined.record(side)
    main.wait_event(joined)
    t1.record(main)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    rows = w.B * w.nq
    del st2, step2
    torch.cuda.empty_cache()
    return {"batches": 2, "streams": 2, "steps": n, "ms_per_step": round(ms, 4),
            "value": round(rows / (ms / 1e3), 1), "unit": "queries/s"}


def scan_bytes(w: synth.Workload) -> int:
    """Algorithmic bytes of one scan launch at decode: every visible indexer key of the
    query's own sequence (64 B codes + 8 B scales), the query (32x128 bf16) and weights
    (32 fp32) -- what the method must read.  The scan's own outputs (block maxima and the
    pool select's inputs, about 0.8 % more) are not counted: see scan_write_bytes."""
    nv = w.n_visible().astype(np.int64)
    return int(nv.sum()) * 72 + w.B * w.nq * (32 * 128 * 2 + 32 * 4)


def scan_write_bytes(w: synth.Workload) -> int:
    """Bytes the scan launch writes besides reading (not in scan_bytes): the block maxima
    (fp32 per 8 visible entries) and, for rows of more than 16384 blocks, the block
    select's inputs -- one uint32 group key per g blocks and each chunk's block and
    entry candidate lists (bounded by the workspace of csa2_index_full_select, which
    also holds the exact fallback's buffers: an upper bound)."""
    nv = w.n_visible().astype(np.int64)
    b = int(((nv + 7) // 8).sum()) * 4
    from kv_cache_decode_mxfp4_amd import _lib as L
    return b + L.index_full_select_workspace(w.n_cap, w.B, w.nq, w.nb, w.k)


def scan_flops(w: synth.Workload) -> int:
    """MFMA flops of one index_full launch: 32 heads x 128 channels x 2 per visible entry."""
    return int(w.n_visible().astype(np.int64).sum()) * 32 * 128 * 2


def step_algorithmic_bytes(w: synth.Workload) -> int:
    """Algorithmic bytes of one decode step, the bytes the method itself must move: per
    query row the visible indexer keys (72 B each), the indexer query and weights, the
    top-k and pool written (2 KiB + 8 KiB), and the attention's reads and writes (k MXFP4
    rows of 288 B and their ids, the window rows, the main query, the fp32 output) --
    1,215 MB per step at 16 x 1M (at 0.70 of 8 TB/s: 217 us per step)."""
    rows = w.B * w.nq
    nv = int(w.n_visible().astype(np.int64).sum())
    b = nv * 72 + rows * (32 * 128 * 2 + 32 * 4)
    b += rows * (w.k * 4 + w.nb * 4)
    b += rows * (w.k * (288 + 4) + w.n_win * 512 + 64 * 512 * 2 + 64 * 512 * 4) * len(w.layers)
    return b


def step_bytes(w: synth.Workload) -> int:
    """Bytes every stage of one decode step moves, intermediates included (block maxima,
    group keys, gathered pool keys, pool scores), for the step's TB/s."""
    rows = w.B * w.nq
    nsel = max(w.nb, w.k)
    nblk = int(((w.n_visible().astype(np.int64) + 7) // 8).sum())
    b = scan_bytes(w)
    b += nblk * 4 + rows * nsel * 4                                  # block select
    b += rows * (nsel * 8 * (72 + 8) + nsel * 4 + 32 * 128 * 2 + 128)  # pool scan
    b += rows * (nsel * 8 * 8 + w.k * 4)                             # top-k of the pool
    attn = rows * (w.k * (4 + 288) + w.n_win * 512 + 64 * 512 * (2 + 4) + 64 * 4)
    b += attn * len(w.layers)
    if "reindex" in w.layers:
        b += rows * (w.nb * 4 + w.nb * 8 * (72 + 8 + 8) + w.k * 4 + 32 * 128 * 2 + 128)
    first, count = w.new_entries()
    b += w.B * count * ((128 + 512) * 4 + 72 + 288 + 32 * 4 * 2)  # encode appended entries
    return b


def source_hash() -> str:
    h = hashlib.sha256()
    for path in SCAN_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per scan launch from the committed counter summary, if it was taken on
    the current scan source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split(None, 1)
            vals[k] = v.strip()
    if vals.get("source_sha256_16") != source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


FLUSH_BYTES = 512 << 20  # twice the 256 MB last-level cache (MALL) of the MI355X


def cold_steps(step, n, torch):
    """Steps timed one by one (HIP events around each), each after writing a 512 MiB scratch
    buffer, so no step finds the previous one's data in the L2s or the MALL.  Reported
    beside the contract's warm, back-to-back figure."""
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    times = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    t = np.array(times)
    return {"steps": n, "flush_bytes": FLUSH_BYTES, "median_ms": round(float(np.median(t)), 4),
            "p10_ms": round(float(np.percentile(t, 10)), 4),
            "p90_ms": round(float(np.percentile(t, 90)), 4)}


def read_ceiling(src, reps, torch, L):
    """The fastest plain streaming read of `src` (the indexer-key cache, the bytes the scan
    streams) over a few launch shapes, timed with HIP events on the current stream:
    (TB/s, workgroups, depth)."""
    sink = torch.zeros(4096, dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    best = (0.0, 0, 0)
    for wgs in (768, 1024, 1280, 2048):
        for depth in (1, 2, 4):
            L.stream_read(src, wgs, depth, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                L.stream_read(src, wgs, depth, sink)
            e1.record()
            e1.synchronize()
            tbps = nbytes / (e0.elapsed_time(e1) / reps / 1e3) / 1e12
            if tbps > best[0]:
                best = (tbps, wgs, depth)
    return best


def prewarm(step, ms_min, torch):
    """Untimed steps for at least ms_min of wall time; per-step HIP events on the first
    and last ten steps show the ramp."""
    if ms_min <= 0:
        return None
    events = []
    t0 = time.perf_counter()
    n = 0
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        events.append((e0, e1))
        n += 1
        if n % 50 == 0:
            events[-1][1].synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms_min:
                break
            events = events[:10] + events[-10:]
    torch.cuda.synchronize()
    first = float(np.mean([a.elapsed_time(b) for a, b in events[:10]]))
    last = float(np.mean([a.elapsed_time(b) for a, b in events[-10:]]))
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "steps": n,
            "first10_ms_per_step": round(first, 4), "last10_ms_per_step": round(last, 4)}


# ------------------------------------------------------------------ CPU baseline (oracle)

def cpu_baseline(w: synth.Workload, rows: int):
    """The oracle timed on this host's cores over the first `rows` query rows of the same
    workload (same Full-layer step: new-row encode, full scan, top-k, pool, attention)."""
    import oracle
    sample = [(b, i) for b in range(w.B) for i in range(w.nq)][:rows]
    seqs = sorted({b for b, _ in sample})
    enc = {}
    t0 = time.time()
    for b in seqs:
        cos, sin = synth.rope_rows(0, w.n_cap)
        kc, ks = oracle.quantize_rows(synth.idx_k_rows(w, b, 0, w.n_cap))
        vc, vs = oracle.quantize_rows(synth.kv_rows(w, b, 0, w.n_cap), cos, sin,
                                      synth.ROPE_OFFSET, synth.ROPE_DIM)
        sw = oracle.encode_fp8(synth.swa_rows(w, 0, b, 0, w.swa_rows()))
        enc[b] = (kc, ks, vc, vs, sw)
    log(f"cpu baseline: oracle caches for {len(seqs)} sequences ({time.time() - t0:.0f} s)")
    qi, wi, qm = synth.q_idx(w, 0), synth.w_idx(w, 0), synth.q_main(w, 0)
    nv, se = w.n_visible(), w.swa_end()
    first, count = w.new_entries()
    new_kv = {b: synth.kv_rows(w, b, first, count) for b in seqs}
    new_idx = {b: synth.idx_k_rows(w, b, first, count) for b in seqs}
    ncos, nsin = synth.rope_rows(first, count)
    t0 = time.perf_counter()
    for b, i in sample:
        kc, ks, vc, vs, sw = enc[b]
        oracle.quantize_rows(new_idx[b])
        oracle.quantize_rows(new_kv[b], ncos, nsin, synth.ROPE_OFFSET, synth.ROPE_DIM)
        full = oracle.full_layer(qi[b, i], wi[b, i], kc, ks, int(nv[b, i]), w.k, w.nb, w.block)
        oracle.attention(qm[b, i], vc, vs, full["topk"], sw, int(se[b, i]), w.n_win, 1.0)
    dt = time.perf_counter() - t0
    cores = oracle.threads()
    # the same Full-layer step of the first row on one thread
    b, i = sample[0]
    kc, ks, vc, vs, sw = enc[b]
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.quantize_rows(new_idx[b])
        oracle.quantize_rows(new_kv[b], ncos, nsin, synth.ROPE_OFFSET, synth.ROPE_DIM)
        full = oracle.full_layer(qi[b, i], wi[b, i], kc, ks, int(nv[b, i]), w.k, w.nb, w.block)
        oracle.attention(qm[b, i], vc, vs, full["topk"], sw, int(se[b, i]), w.n_win, 1.0)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_threads(0)
    return {"value": round(len(sample) / dt, 4), "unit": "queries/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{len(sample)} query rows ({len(seqs)} sequences) of the same workload, "
                      f"full Full-layer step per row, {dt:.1f} s wall",
            "single_thread_value": round(1.0 / dt1, 4), "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus above 1 is not supported)", file=sys.stderr)
        return 2
    import torch
    import kv_cache_decode_mxfp4_amd as kv
    from kv_cache_decode_mxfp4_amd import _lib as L, layers
    L.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    w = synth.WORKLOADS[args.config]
    log(f"workload: {w.name}")
    st = build_device(w, torch, L)
    step, scan_events = make_step(st, torch, L, layers, args.kv_production, args.attn_out)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    warm_info = prewarm(step, args.prewarm_ms, torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warm (pre-warm {warm_info})")
    scan_events.clear()
    step.layer_events.clear()
    step.prepare_scan_events((args.steps + SCAN_EVENT_EVERY - 1) // SCAN_EVENT_EVERY)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    # the scan's own duration: HIP events that the scan kernel's dispatch records (through
    # the library call) on every SCAN_EVENT_EVERY-th timed step
    for i in range(args.steps):
        step(time_scan=(i % SCAN_EVENT_EVERY == 0))
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    cold = cold_steps(step, args.cold_steps, torch) if args.cold_steps > 0 else None
    overlap = (overlap_run(w, step, args.overlap_steps, torch, L, layers, args.kv_production,
                           args.attn_out)
               if args.overlap_steps > 0 and w.decode else None)
    ms_step = ms_total / args.steps
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in scan_events]))
    rows = w.B * w.nq
    value = rows / (ms_step / 1e3)
    ceiling = None
    if w.decode and args.ceiling_reps > 0:
        tbps, wgs, depth = read_ceiling(st["kc"], args.ceiling_reps, torch, L)
        ceiling = {"read_TBps": round(tbps, 3), "workgroups": wgs, "depth": depth,
                   "bytes": st["kc"].numel(),
                   "what": "fastest plain streaming read of the indexer-key code cache (12 "
                           "launch shapes), the same process and box"}
    if w.decode:
        sb = scan_bytes(w)
        achieved = sb / (scan_ms / 1e3)
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": PEAK_HBM / 1e9,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                "traffic": measured_traffic() if args.config == 3 else None,
                "kernel": "index_full_kernel", "kernel_ms": round(scan_ms, 4),
                "algorithmic_bytes": sb,
                "bytes_counted": "indexer keys (72 B per visible entry) + query + weights; the "
                                 "scan's writes are not counted",
                "writes_bytes": scan_write_bytes(w)}
        if roof["traffic"]:
            roof["traffic_GBps"] = round(roof["traffic"] / (scan_ms / 1e3) / 1e9, 1)
        if ceiling is not None:
            roof["frac_of_read_ceiling"] = round(achieved / 1e12 / ceiling["read_TBps"], 4)
    else:
        fl = scan_flops(w)
        achieved = fl / (scan_ms / 1e3)
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": PEAK_F16 / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16, 4), "traffic": None,
                "kernel": "index_full_kernel", "kernel_ms": round(scan_ms, 4),
                "algorithmic_flops": fl}
    out = {
        "metric": METRIC if args.config == 3 else f"CSA2 query rows/sec, {w.name}",
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "queries_per_seq": w.nq, "n_cap": w.n_cap,
                   "topk": w.k, "pool_blocks": w.nb, "block": w.block, "n_win": w.n_win,
                   "indexer": "32x128", "attention": "64x512", "layers": list(w.layers),
                   "kv_production": args.kv_production, "attn_out": args.attn_out},
        "roofline": roof,
    }
    if w.decode:
        out["step_tbps"] = round(step_bytes(w) / (ms_step / 1e3) / 1e12, 3)
        sbytes = step_algorithmic_bytes(w)
        out["step_roofline"] = {
            "bound": "hbm", "algorithmic_bytes": sbytes,
            "achieved": round(sbytes / (ms_step / 1e3) / 1e9, 1), "peak": PEAK_HBM / 1e9,
            "unit": "GB/s", "frac": round(sbytes / (ms_step / 1e3) / PEAK_HBM, 4),
            "target_frac": 0.70,
            "note": "the whole step (every kernel) against 8 TB/s: the bar the 70 % target "
                    "refers to; roofline.frac is the scan kernel alone"}
        if ceiling is not None:
            out["step_roofline"]["frac_of_read_ceiling"] = round(
                sbytes / (ms_step / 1e3) / 1e12 / ceiling["read_TBps"], 4)
            out["read_ceiling"] = ceiling
    if warm_info is not None:
        out["prewarm"] = warm_info
    if step.layer_events:
        # each layer of the group: Full (encode .. its attention), Reindex (pool rescoring,
        # top-k, attention), Reuse (attention), from events on the sampled steps
        per = np.array([[a.elapsed_time(b) for a, b in zip(ev[:-1], ev[1:])]
                        for ev in step.layer_events])
        out["layers_ms"] = [[name, round(float(v), 4)] for name, v in zip(w.layers, per.mean(0))]
    if cold is not None:
        out["cold"] = cold
    if overlap is not None:
        out["two_batch_overlap"] = overlap
    if args.cpu_sample > 0 and args.config in (1, 3):
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
