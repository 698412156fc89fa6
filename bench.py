#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Headline workload: Qwen3-8B-shaped single-layer batch-1 decode at a context of
15488 tokens (119 compressed 128-token tiles + a 256-token FP32 window; 32
query heads, 8 KV heads, head_dim 128).  One step = one kvarn_decode_attention
call: the split kernel (query rotation, every tile on the matrix cores, the
window tokens) and the log-sum-exp combine with its inverse WHT.

Timing: the K timed steps are captured once in a HIP graph that cycles
through enough distinct layers (records + windows + queries, all resident in
HBM before timing starts) to exceed twice the 256 MB last-level cache; the W
warmup steps are a graph of their own.  Each timed region is one replay of
the K-step graph between two device synchronisations, timed by HIP events on
the replay stream; the reported time is the median over the regions.

The same JSON line carries the other workloads as parity-tested and measured
here: decode at contexts 4096 and 32768 (and over f16-scale and K6V5 records),
multi-query verify, the 0.6B-shaped 64-step decode with appends, the stepped
16-sequence wide-head batch (append, promote, decode), tile compression,
chunked prefill, the measured floors of the part (plain read, matrix-op rate,
empty launch), and the CPU oracle timed on the host's cores (cpu_baseline).

--calibration-copy adds one device-to-device copy of a known size, for
scaling hardware byte counters taken over the same run.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import math
import multiprocessing as mp
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
INT8_MFMA_PEAK_TOPS = 5000.0
LLC_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "quantized_attention_tok_amd", "csrc")
DECODE_SOURCES = ["decode_split.hip", "kvarn_mfma.h", "kvarn_launch.h", "kvarn_device.h", "kvarn_api.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_ctx15488.json")
DTYPE = "f32 (matrix-core contractions as fp16 hi+lo operand pairs with exact integer codes, fp32 accumulate)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_bytes(T, n_w, Hq, Hkv, d, tile_bytes, rows=1):
    """Algorithmic bytes of one decode call: every record and window row read
    once, the query rows read once, the output rows written once."""
    return T * Hkv * tile_bytes + 2 * n_w * Hkv * d * 4 + 2 * rows * Hq * d * 4


def decode_sources_sha():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary, if it was
    taken on the current decode sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("decode_sources_sha") != decode_sources_sha():
        return None
    return t.get("hbm_bytes_per_call")


# ---------------------------------------------------------------------------
# graph timing
# ---------------------------------------------------------------------------

def capture(torch, fn):
    """Run fn once on a side stream (warm-up of allocator and library), then
    capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_regions(torch, g, reps):
    """reps replays of graph g, each between two synchronisations and timed
    by an event pair on the replay stream; ms per region."""
    out = []
    for _ in range(reps):
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e))
    return out


def measure_steps(torch, step, n_steps, warmup, reps):
    """step(i) enqueues step i.  A graph of `warmup` steps is replayed once
    untimed; a graph of exactly n_steps steps is replayed reps times; returns
    (median ms per step, per-region ms list)."""
    if warmup > 0:
        gw = capture(torch, lambda: [step(i) for i in range(warmup)])
        gw.replay()
        torch.cuda.synchronize()
    g = capture(torch, lambda: [step(i) for i in range(n_steps)])
    regions = time_regions(torch, g, reps)
    return float(np.median(regions)) / n_steps, regions


def stats(regions, n_steps):
    r = np.asarray(regions) / n_steps * 1e3
    return {"median_us": float(np.median(r)), "min_us": float(r.min()), "max_us": float(r.max()),
            "regions": len(regions), "steps_per_region": n_steps}


# ---------------------------------------------------------------------------
# decode at the 8B shape (headline), verify
# ---------------------------------------------------------------------------

def decode_case(torch, kvarn, synth, ctx, steps, warmup, reps, seed=2, f16=False, kbits=4, vbits=2):
    d, Hq, Hkv, W = 128, 32, 8, 256
    dev = "cuda:0"
    T = kvarn.visible_tiles(ctx - 1, W)
    n_w = ctx - 128 * T
    tb = kvarn.tile_bytes(d, f16, kbits, vbits)
    k4v2 = (kbits, vbits) == (4, 2)
    scale = 1.0 / math.sqrt(d)
    per_layer = T * Hkv * tb + 2 * n_w * Hkv * d * 4
    L = max(8, int(math.ceil(2 * LLC_BYTES / per_layer)))
    K, V = synth.make_kv(seed, ctx, Hkv, d, synth.outliers_for(d, 0.01))
    kd = torch.from_numpy(K).to(dev)
    vd = torch.from_numpy(V).to(dev)
    rec0 = torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev)
    kvarn.compress_tile(kd, vd, rec0, T, f16_scales=f16, kbits=kbits, vbits=vbits)
    recs = [rec0.clone() for _ in range(L)]
    kw = [kd[128 * T:].clone()[None] for _ in range(L)]
    vw = [vd[128 * T:].clone()[None] for _ in range(L)]
    qs = torch.from_numpy(synth.make_q(seed, L, Hq, d)).to(dev).reshape(L, 1, Hq, d)
    outs = torch.empty_like(qs)
    qr = torch.empty_like(qs[0])
    ws_bytes = kvarn.decode_workspace_bytes(qs[0], None if k4v2 else qr, recs[0], [0], [T], kw[0], vw[0],
                                            [n_w], scale, f16_scales=f16, kbits=kbits, vbits=vbits)
    ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)
    del kd, vd
    torch.cuda.synchronize()

    def step(i):
        l = i % L
        if k4v2:   # q_rot=None: the split kernel rotates q itself
            kvarn.decode_attention(qs[l], None, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                                   out=outs[l], workspace=ws, f16_scales=f16)
        else:      # the vector-unit kernels take a rotated query
            kvarn.rotate_query(qs[l], out=qr)
            kvarn.decode_attention(qs[l], qr, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                                   out=outs[l], workspace=ws, f16_scales=f16, kbits=kbits, vbits=vbits)

    ms, regions = measure_steps(torch, step, steps, warmup, reps)
    alg = decode_bytes(T, n_w, Hq, Hkv, d, tb)
    info = {"context": ctx, "tiles": T, "window": n_w, "scales": "f16" if f16 else "f32",
            "key_bits": kbits, "value_bits": vbits, "record_bytes": tb, "layers_cycled": L,
            "us_per_step": ms * 1e3, "timing": stats(regions, steps),
            "kv_tokens_per_s": ctx / (ms * 1e-3), "algorithmic_bytes": alg,
            "achieved_GBps": alg / (ms * 1e-3) / 1e9}
    return info, (K, V, rec0, T, n_w, scale)


def verify_case(torch, kvarn, synth, ctx, width, reps, seed=2):
    """Multi-query verify of `width` draft rows at the 8B decode shape: one call
    reads every record once for all rows."""
    d, Hq, Hkv, W = 128, 32, 8, 256
    dev = "cuda:0"
    T = kvarn.visible_tiles(ctx - 1, W)
    n_w = ctx - 128 * T
    tb = kvarn.tile_bytes(d)
    scale = 1.0 / math.sqrt(d)
    per_layer = T * Hkv * tb + 2 * n_w * Hkv * d * 4
    L = max(8, int(math.ceil(2 * LLC_BYTES / per_layer)))
    K, V = synth.make_kv(seed, ctx, Hkv, d, synth.outliers_for(d, 0.01))
    kd = torch.from_numpy(K).to(dev)
    vd = torch.from_numpy(V).to(dev)
    rec0 = torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev)
    kvarn.compress_tile(kd, vd, rec0, T)
    recs = [rec0.clone() for _ in range(L)]
    kw = [kd[128 * T:].clone()[None] for _ in range(L)]
    vw = [vd[128 * T:].clone()[None] for _ in range(L)]
    qs = torch.from_numpy(synth.make_q(seed, L * width, Hq, d)).to(dev).reshape(L, 1, width, Hq, d)
    outs = torch.empty_like(qs)
    ws = torch.empty(max(16, kvarn.decode_workspace_bytes(qs[0], None, recs[0], [0], [T], kw[0], vw[0],
                                                          [n_w], scale)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(i):
        l = i % L
        kvarn.decode_attention(qs[l], None, recs[l], [0], [T], kw[l], vw[l], [n_w], scale, out=outs[l],
                               workspace=ws)

    ms, regions = measure_steps(torch, step, L, 0, reps)
    return {"width": width, "context": ctx, "us_per_call": ms * 1e3, "timing": stats(regions, L),
            "query_rows_per_s": width / (ms * 1e-3), "layers_cycled": L,
            "algorithmic_bytes": decode_bytes(T, n_w, Hq, Hkv, d, tb, rows=width)}


# ---------------------------------------------------------------------------
# the 0.6B-shaped layer: 64 decode steps with appends
# ---------------------------------------------------------------------------

def qwen06b_case(torch, kvarn, synth, reps):
    """24 compressed tiles + a 256-token window, then 64 decode steps; each
    step appends the new token's K and V rows to the FP32 window (no step
    crosses a promotion boundary: the window grows from 257 to 320 tokens,
    below the 384 at which a tile is promoted) and attends.  One
    single-layer step = one decode call that takes the new rows (k_new /
    v_new: the split kernel stores them into the window and attends them in
    the same launch); the graph runs the 64 steps over enough distinct layers
    to exceed the cache twice."""
    w = synth.WORKLOADS["qwen3_0.6b_decode"]
    d, Hq, Hkv, W, n_steps = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window, w.steps
    dev = "cuda:0"
    n0 = w.contexts[0]                       # 3072 + 256
    T = kvarn.visible_tiles(n0 - 1, W)       # 24
    tb = kvarn.tile_bytes(d)
    scale = 1.0 / math.sqrt(d)
    K, V = synth.make_kv(w.seed, n0 + n_steps, Hkv, d, w.n_outliers)
    kd, vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
    rec0 = torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev)
    kvarn.compress_tile(kd, vd, rec0, T)
    cap = W + n_steps
    per_layer = T * Hkv * tb + 2 * cap * Hkv * d * 4
    L = max(8, int(math.ceil(2 * LLC_BYTES / per_layer)))
    recs = [rec0.clone() for _ in range(L)]
    # window rows [cap][2][Hkv][d]: a token's K and V rows side by side; the
    # decode call takes the two strided views and stores each step's new rows
    kvwin = [torch.empty(cap, 2, Hkv, d, device=dev) for _ in range(L)]
    for l in range(L):
        kvwin[l][:W, 0] = kd[128 * T:n0]
        kvwin[l][:W, 1] = vd[128 * T:n0]
    kwin = [x[None, :, 0] for x in kvwin]
    vwin = [x[None, :, 1] for x in kvwin]
    src = torch.stack([kd[n0:], vd[n0:]], dim=1).contiguous()   # the 64 appended rows
    qs = torch.from_numpy(synth.make_q(w.seed, n_steps, Hq, d)).to(dev).reshape(n_steps, 1, Hq, d)
    outs = torch.empty(L, 1, Hq, d, device=dev)
    ws = torch.empty(max(16, kvarn.decode_workspace_bytes(qs[0], None, recs[0], [0], [T], kwin[0], vwin[0],
                                                          [cap], scale, max_win=cap)),
                     dtype=torch.uint8, device=dev)
    del kd, vd
    torch.cuda.synchronize()

    def run():
        for s in range(n_steps):
            n_w = W + s + 1
            for l in range(L):
                kvarn.decode_attention(qs[s], None, recs[l], [0], [T], kwin[l], vwin[l], [n_w], scale,
                                       out=outs[l], workspace=ws, max_win=cap,
                                       k_new=src[s, 0][None], v_new=src[s, 1][None])

    g = capture(torch, run)
    regions = time_regions(torch, g, reps)
    ms = float(np.median(regions)) / (n_steps * L)
    kv_tokens = sum(128 * T + W + s + 1 for s in range(n_steps)) / n_steps
    alg = sum(decode_bytes(T, W + s + 1, Hq, Hkv, d, tb) + 2 * Hkv * d * 4 for s in range(n_steps)) / n_steps
    return {"workload": "qwen3-0.6b-shape single layer: 24 tiles + 256-token window, 64 decode steps "
                        "with appends (Hq 16, Hkv 8, head_dim 128)",
            "us_per_layer_step": ms * 1e3, "timing": stats(regions, n_steps * L),
            "steps": n_steps, "layers_cycled": L,
            "decode_steps_per_s": 1.0 / (ms * 1e-3),
            "kv_tokens_per_s": kv_tokens / (ms * 1e-3),
            "ms_for_64_steps": 64 * ms, "achieved_GBps": alg / (ms * 1e-3) / 1e9,
            "includes": "window row append (inside the decode call), query rotation, decode attention"}


# ---------------------------------------------------------------------------
# the 16-sequence wide-head batch, stepped: append, promote, decode
# ---------------------------------------------------------------------------

def wide_step_case(torch, kvarn, synth, name, n_steps, reps, eager_calls=0):
    """16 sequences with contexts uniform in 1k-32k tokens in whole tiles and a
    window of 256 + r_b tokens (r_b uniform in [0, 128)).  One step appends one
    token's K and V rows to every sequence's window, compresses the oldest 128
    window rows of every sequence whose window reaches 384 tokens into its
    next tile (each sequence promotes once in 128 steps), and runs one decode
    call for the batch.  Windows live in one [rows][batch][kv][d] buffer per
    layer (every step appends one row for the whole batch); a sequence's
    window is a view that starts at its own row.  The graph runs the steps
    over enough distinct layers to exceed the cache twice; a second graph
    runs the same decode calls alone."""
    w = synth.WORKLOADS[name]
    d, Hq, Hkv, W, B = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window, w.batch
    dev = "cuda:0"
    T0 = [int(t) for t in synth.ragged_contexts(w.seed, B, w.extra["ctx_lo"], w.extra["ctx_hi"], W)]
    r = [int(x) for x in synth.window_offsets(w.seed, B)]
    tb = kvarn.tile_bytes(d)
    scale = 1.0 / math.sqrt(d)
    base, cap = W + 128, W + 128 + n_steps         # row `base + s` receives step s
    rec_start = [int(x) for x in np.cumsum([0] + [t + 1 for t in T0[:-1]])]
    rows = sum(T0) + B
    pool0 = torch.empty(rows, Hkv, tb, dtype=torch.uint8, device=dev)
    raw0 = torch.zeros(cap, B, 2, Hkv, d, device=dev)    # [row][seq][K or V][kv][d]
    src = torch.empty(n_steps, B, 2, Hkv, d, device=dev)
    for b in range(B):
        n_w0 = W + r[b]
        K, V = synth.batch_sequence_kv(w, b, 128 * T0[b] + n_w0 + n_steps)
        kd, vd = torch.from_numpy(K).to(dev), torch.from_numpy(V).to(dev)
        kvarn.compress_tile(kd, vd, pool0[rec_start[b]:rec_start[b] + T0[b]], T0[b])
        lo = 128 * T0[b]
        raw0[base - n_w0:base, b, 0] = kd[lo:lo + n_w0]
        raw0[base - n_w0:base, b, 1] = vd[lo:lo + n_w0]
        src[:, b, 0] = kd[lo + n_w0:]
        src[:, b, 1] = vd[lo + n_w0:]
        del K, V, kd, vd
    per_layer = rows * Hkv * tb + 2 * cap * B * Hkv * d * 4
    L = max(2, int(math.ceil(2 * LLC_BYTES / per_layer)))
    pools = [pool0] + [pool0.clone() for _ in range(L - 1)]
    raw = [raw0] + [raw0.clone() for _ in range(L - 1)]
    raw_k = [x[:, :, 0] for x in raw]      # [rows][B][kv][d] strided views
    raw_v = [x[:, :, 1] for x in raw]
    q = torch.from_numpy(synth.make_q(w.seed, B, Hq, d)).to(dev)
    out = torch.empty_like(q)
    max_tiles, max_win = max(T0) + 1, W + 128
    win_view = lambda t: t.permute(1, 0, 2, 3)    # [B][rows][kv][d] strided view
    ws = torch.empty(max(16, kvarn.decode_workspace_bytes(q, None, pool0, rec_start, T0, win_view(raw_k[0]),
                                                          win_view(raw_v[0]), [W] * B, scale,
                                                          max_tiles=max_tiles, max_win=max_win)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def state(s):
        """Per-sequence tiles, window start and window length after step s's append."""
        nt, st, nw, promote = [], [], [], []
        for b in range(B):
            done = s >= 127 - r[b]
            if s == 127 - r[b]:
                promote.append(b)
            nt.append(T0[b] + (1 if done else 0))
            st.append(base - W - r[b] + (128 if done else 0))
            nw.append(W + r[b] + s + 1 - (128 if done else 0))
        return nt, st, nw, promote

    plan = [state(s) for s in range(n_steps)]
    assert all(len([s for s in range(n_steps) if b in plan[s][3]]) == 1 for b in range(B))

    def step(l, s, with_updates=True):
        nt, st, nw, promote = plan[s]
        if with_updates:   # one copy appends every sequence's K and V rows
            raw[l][base + s].copy_(src[s])
            for b in promote:   # the oldest 128 window rows become the sequence's next tile
                lo = base - W - r[b]
                kvarn.compress_tile(raw_k[l][lo:, b], raw_v[l][lo:, b],
                                    pools[l][rec_start[b] + T0[b]:rec_start[b] + T0[b] + 1], 1)
        kvarn.decode_attention(q, None, pools[l], rec_start, nt, win_view(raw_k[l]), win_view(raw_v[l]), nw,
                               scale, out=out, workspace=ws, max_tiles=max_tiles, max_win=max_win,
                               win_start=st)

    if eager_calls > 0:   # plain decode calls of step 0's state, outside any graph (for counter passes)
        for i in range(eager_calls):
            step(i % L, 0, False)
        torch.cuda.synchronize()
        return {"workload": f"batch {B}, head_dim {d}: {eager_calls} decode calls outside a graph",
                "head_dim": d, "eager_calls": eager_calls}
    g = capture(torch, lambda: [step(l, s) for s in range(n_steps) for l in range(L)])
    regions = time_regions(torch, g, reps)
    ms = float(np.median(regions)) / (n_steps * L)
    g2 = capture(torch, lambda: [step(l, s, False) for s in range(n_steps) for l in range(L)])
    regions2 = time_regions(torch, g2, reps)
    ms2 = float(np.median(regions2)) / (n_steps * L)
    kv_tokens = sum(sum(128 * plan[s][0][b] + plan[s][2][b] for b in range(B)) for s in range(n_steps)) / n_steps
    dec_alg = sum(sum(decode_bytes(plan[s][0][b], plan[s][2][b], Hq, Hkv, d, tb) for b in range(B))
                  for s in range(n_steps)) / n_steps
    upd_alg = (2 * B * Hkv * d * 4 * 2 * n_steps + B * Hkv * (2 * 128 * d * 4 + tb)) / n_steps
    return {"workload": f"batch {B}, head_dim {d}, Hq {Hq}, Hkv {Hkv}: contexts 1k-32k in whole tiles "
                        f"({sum(T0)} tiles at the start) + windows of 256-383 tokens, {n_steps} steps, "
                        f"each appending one token per sequence, promoting due tiles, decoding the batch",
            "head_dim": d, "batch": B, "steps": n_steps, "layers_cycled": L,
            "promotions": B,
            "us_per_layer_step": ms * 1e3, "timing": stats(regions, n_steps * L),
            "kv_tokens_per_s": kv_tokens / (ms * 1e-3), "decode_tokens_per_s": B / (ms * 1e-3),
            "achieved_GBps": (dec_alg + upd_alg) / (ms * 1e-3) / 1e9,
            "decode_only": {"us_per_layer_step": ms2 * 1e3, "timing": stats(regions2, n_steps * L),
                            "kv_tokens_per_s": kv_tokens / (ms2 * 1e-3),
                            "achieved_GBps": dec_alg / (ms2 * 1e-3) / 1e9},
            "includes": "window row appends, tile compression of due tiles, query rotation, decode attention"}


# ---------------------------------------------------------------------------
# compression, chunked prefill
# ---------------------------------------------------------------------------

def compress_case(torch, kvarn, synth, reps):
    """The 8B-shaped prompt's 119 x 8 tile-heads in one launch, cycling
    distinct raw inputs beyond the cache."""
    d, Hkv, n = 128, 8, 15488
    dev = "cuda:0"
    T = kvarn.visible_tiles(n - 1, 256)
    K, V = synth.make_kv(4, n, Hkv, d, synth.outliers_for(d, 0.01))
    tb = kvarn.tile_bytes(d)
    per = T * Hkv * (2 * 128 * d * 4 + tb)
    L = max(4, int(math.ceil(2 * LLC_BYTES / per)))
    kd = [torch.from_numpy(K).to(dev) for _ in range(L)]
    vd = [torch.from_numpy(V).to(dev) for _ in range(L)]
    rec = [torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev) for _ in range(L)]
    torch.cuda.synchronize()
    ms, regions = measure_steps(torch, lambda i: kvarn.compress_tile(kd[i % L], vd[i % L], rec[i % L], T),
                                L, 0, reps)
    return {"tile_heads": T * Hkv, "us_per_launch": ms * 1e3, "timing": stats(regions, L),
            "layers_cycled": L, "tile_heads_per_s": T * Hkv / (ms * 1e-3),
            "algorithmic_bytes": per, "achieved_GBps": per / (ms * 1e-3) / 1e9}


def prefill_case(torch, kvarn, synth, SequenceCache, d, Hq, Hkv, n, chunk, reps, W=256):
    """Chunked prefill of an n-token prompt in one graph: raw row copies, tile
    compression, query rotation (inside the prefill kernels) and prefill
    attention for every chunk."""
    dev = "cuda:0"
    Kp, Vp = synth.make_kv(4, n, Hkv, d, synth.outliers_for(d, 0.01))
    Qp = synth.make_q(4, n, Hq, d)
    kp, vp, qp = (torch.from_numpy(x).to(dev) for x in (Kp, Vp, Qp))
    outp = torch.empty_like(qp)
    cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=dev)
    # one workspace for every chunk's split partials
    big = max(kvarn.prefill_workspace_bytes(qp[p0:p0 + min(chunk, n - p0)], None, cache.records,
                                            n // 128, cache.k, cache.v, 0, p0, W, 1.0)
              for p0 in range(0, n, chunk))
    ws = torch.empty(max(big, 16), dtype=torch.uint8, device=dev)

    def run_prefill():
        cache.n_tokens = cache.n_tiles = 0
        for p0 in range(0, n, chunk):
            c = min(chunk, n - p0)
            cache.append(kp[p0:p0 + c], vp[p0:p0 + c])
            rb = 128 * kvarn.visible_tiles(p0, W)
            kvarn.prefill_attention(qp[p0:p0 + c], None, cache.records, cache.n_tiles, cache.k[rb:],
                                    cache.v[rb:], rb, p0, W, 1.0 / math.sqrt(d), out=outp[p0:p0 + c],
                                    workspace=ws)

    g = capture(torch, run_prefill)
    regions = time_regions(torch, g, reps)
    ms_p = float(np.median(regions))
    pairs = n * (n + 1) // 2                            # causal (query, key) pairs per head
    ops = 2 * 2 * d * pairs * Hq                         # Q.K and P.V multiply-adds as 2 ops each
    tops = ops / (ms_p * 1e-3) / 1e12
    return {"head_dim": d, "n_q_heads": Hq, "n_kv_heads": Hkv, "tokens_per_s": n / (ms_p * 1e-3),
            "ms": ms_p, "timing": stats(regions, 1), "prompt": n, "chunk": chunk,
            "algorithmic_TOPS": tops, "int8_mfma_frac": tops / INT8_MFMA_PEAK_TOPS,
            "fp16_mfma_frac": tops / FP16_MFMA_PEAK_TFLOPS,
            "includes": "raw row copies, tile compression, query rotation, prefill attention"}


# ---------------------------------------------------------------------------
# measured floors of the part
# ---------------------------------------------------------------------------

def floors_case(torch):
    """Plain read bandwidth (1 GiB, and 16.75 MB per launch cycled over
    distinct buffers like the headline decode), the fp16 and int8 matrix-op
    rates, and the cost of an empty launch inside a graph."""
    from quantized_attention_tok_amd import build_lib
    F = ctypes.CDLL(build_lib.FLOORS_LIB)
    vp = ctypes.c_void_p
    F.kvarn_floor_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    F.kvarn_floor_mfma.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    F.kvarn_floor_empty.argtypes = [vp]
    dev = "cuda:0"
    stream = lambda: vp(torch.cuda.current_stream().cuda_stream)

    def ok(rc):
        if rc != 0:
            raise RuntimeError(f"floor kernel launch returned {rc}")

    res = {}
    big = 1 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device=dev)
    groups = 4096
    sink = torch.empty(groups * 256, dtype=torch.int32, device=dev)
    ms, reg = measure_steps(torch, lambda i: ok(F.kvarn_floor_read(vp(buf.data_ptr()), big, vp(sink.data_ptr()),
                                                                   groups, stream())), 4, 1, 10)
    res["read_1GiB"] = {"GBps": big / (ms * 1e-3) / 1e9, "us_per_launch": ms * 1e3}
    del buf
    small = 16752640
    L = int(math.ceil(2 * LLC_BYTES / small))
    bufs = [torch.ones(small // 4, dtype=torch.int32, device=dev) for _ in range(L)]
    g2 = 1024
    sink2 = torch.empty(g2 * 256, dtype=torch.int32, device=dev)
    ms, reg = measure_steps(torch, lambda i: ok(F.kvarn_floor_read(vp(bufs[i % L].data_ptr()), small,
                                                                   vp(sink2.data_ptr()), g2, stream())),
                            L, L, 10)
    res["read_16.75MB"] = {"GBps": small / (ms * 1e-3) / 1e9, "us_per_launch": ms * 1e3, "buffers_cycled": L}
    del bufs
    out = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    for kind, name, per_op, peak in ((0, "mfma_f16_16x16x32", 16384, FP16_MFMA_PEAK_TFLOPS),
                                     (1, "mfma_i8_16x16x64", 32768, INT8_MFMA_PEAK_TOPS)):
        iters = 4000
        ms, reg = measure_steps(torch, lambda i: ok(F.kvarn_floor_mfma(vp(out.data_ptr()), 2048, iters, kind,
                                                                       stream())), 1, 1, 10)
        rate = 2048 * 4 * iters * 4 * per_op / (ms * 1e-3) / 1e12
        res[name] = {"T_ops_per_s": rate, "peak": peak, "frac_of_peak": rate / peak}
    ms, reg = measure_steps(torch, lambda i: ok(F.kvarn_floor_empty(stream())), 200, 20, 10)
    res["empty_launch_us"] = ms * 1e3
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline (runs before the GPU is touched; worker processes fork)
# ---------------------------------------------------------------------------

_W = {}


def _worker_init(recs, kwin, vwin, qs, T, scale):
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    _W.update(recs=recs, kwin=kwin, vwin=vwin, qs=qs, T=T, scale=scale)


def _worker_decode(i):
    import oracle
    kh, vh = oracle.dequant_records(_W["recs"], 128)
    oracle.decode(_W["qs"][i % len(_W["qs"])], kh, vh, _W["T"], _W["kwin"], _W["vwin"], _W["scale"])
    return i


def _worker_compress(args):
    import oracle
    k, v = args
    return oracle.compress_tile(k, v)


def cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth):
    """The oracle (plain C compressor, fp64 numpy attention) on a bounded sample
    of the headline workload, single-threaded and on the usable host cores
    (processes over independent tile-heads and decode steps)."""
    import oracle
    from threadpoolctl import threadpool_limits
    d, Hq, Hkv, W, ctx = 128, 32, 8, 256, 15488
    T = oracle.visible_tiles(ctx - 1, W)
    scale = 1.0 / math.sqrt(d)
    K, V = synth.make_kv(2, ctx, Hkv, d, synth.outliers_for(d, 0.01))
    qs = synth.make_q(2, 64, Hq, d)
    nproc = os.cpu_count()
    usable = len(os.sched_getaffinity(0))
    workers = max(1, min(usable, 16))
    units = [(K[128 * j:128 * (j + 1), h].copy(), V[128 * j:128 * (j + 1), h].copy())
             for j in range(T) for h in range(Hkv)]
    res = {"nproc": nproc, "usable_cpus": usable, "cpu_model": cpu_model(), "workers": workers}
    with threadpool_limits(1):
        # compression, one thread: tile-heads until 3 s
        t0, n1 = time.perf_counter(), 0
        while n1 < len(units) and (n1 < 8 or time.perf_counter() - t0 < 3.0):
            oracle.compress_tile(*units[n1])
            n1 += 1
        c1 = n1 / (time.perf_counter() - t0)
    ctx_mp = mp.get_context("fork")
    with cf.ProcessPoolExecutor(workers, mp_context=ctx_mp) as ex:
        t0 = time.perf_counter()
        recs_list = list(ex.map(_worker_compress, units, chunksize=8))
        cw = len(units) / (time.perf_counter() - t0)
    recs = np.stack(recs_list).reshape(T, Hkv, -1)
    res["compress"] = {"single_thread_tile_heads_per_s": c1, "all_cores_tile_heads_per_s": cw,
                       "sample": f"{n1} tile-heads on one thread; all {len(units)} tile-heads of the "
                                 f"15488-token prompt on {workers} processes"}
    kwin, vwin = K[128 * T:], V[128 * T:]
    with threadpool_limits(1):
        t0, n_dec = time.perf_counter(), 0
        while n_dec < 2 or (n_dec < 64 and time.perf_counter() - t0 < 6.0):
            kh, vh = oracle.dequant_records(recs, d)
            oracle.decode(qs[n_dec], kh, vh, T, kwin, vwin, scale)
            n_dec += 1
        sec1 = time.perf_counter() - t0
        # prefill: rows of the decode view near the end of the prompt (same records)
        t0, n_rows = time.perf_counter(), 0
        while n_rows < 2 or (n_rows < 32 and time.perf_counter() - t0 < 3.0):
            oracle.prefill_row(qs[n_rows], ctx - 1 - n_rows, W, kh, vh, K, V, scale)
            n_rows += 1
        secp = time.perf_counter() - t0
    with cf.ProcessPoolExecutor(workers, mp_context=ctx_mp, initializer=_worker_init,
                                initargs=(recs, kwin, vwin, qs, T, scale)) as ex:
        list(ex.map(_worker_decode, range(workers)))      # warm every worker
        per_step = sec1 / n_dec                           # about 3 s of work per process
        n_all = workers * max(2, int(round(3.0 / per_step)))
        t0 = time.perf_counter()
        list(ex.map(_worker_decode, range(n_all)))
        secw = time.perf_counter() - t0
    res["decode_single_thread"] = {"kv_tokens_per_s": n_dec * ctx / sec1,
                                   "sample": f"{n_dec} decode steps at context {ctx} ({sec1:.1f} s)"}
    res["prefill_single_thread"] = {"rows_per_s": n_rows / secp,
                                    "sample": f"{n_rows} prompt rows at positions {ctx - n_rows}..{ctx - 1} "
                                              f"of the 15488-token prompt, 32 heads each ({secp:.1f} s)"}
    return {"value": n_all * ctx / secw, "unit": "KV tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_all} decode steps of the 8B-shaped layer at context {ctx} on {workers} "
                      f"processes (one thread each), each: dequantise {T * Hkv} records to fp64 and "
                      f"attend 32 heads over {ctx} keys ({secw:.1f} s)",
            **res}


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=21, help="timed regions (replays) per measurement")
    ap.add_argument("--context", type=int, default=15488)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra-contexts", action="store_true")
    ap.add_argument("--no-steps", action="store_true", help="skip the stepped 0.6B and wide-head workloads")
    ap.add_argument("--no-floors", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-compress", action="store_true")
    ap.add_argument("--eager-wide", type=int, default=0,
                    help="instead of the stepped wide-head graphs: this many plain decode calls of each "
                         "wide batch (for profilers that count per dispatch)")
    ap.add_argument("--step-reps", type=int, default=7,
                    help="timed regions of the stepped workloads (each one graph of 64 or 128 steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the KVarN path here runs on a single MI355X)", flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.reps < 1 or args.step_reps < 1:
        sys.exit("--steps >= 1, --warmup >= 0 and --reps >= 1 are required")

    from quantized_attention_tok_amd import synth
    cpu = None
    if not args.no_cpu_baseline:   # before any device call: the worker processes fork
        cpu = cpu_baseline(synth)
        log(f"cpu oracle: decode {cpu['value']:.3g} KV tokens/s on {cpu['cores']} processes "
            f"({cpu['decode_single_thread']['kv_tokens_per_s']:.3g} on one thread), compress "
            f"{cpu['compress']['all_cores_tile_heads_per_s']:.3g} tile-heads/s")

    import torch
    from quantized_attention_tok_amd import kvarn
    from quantized_attention_tok_amd.cache import SequenceCache

    kvarn.lib()  # fails loudly if the HIP library is missing
    R = args.reps
    head, keep = decode_case(torch, kvarn, synth, args.context, args.steps, args.warmup, R)
    log(f"decode context {head['context']}: {head['us_per_step']:.2f} us per call (median of {R}), "
        f"{head['achieved_GBps']:.0f} GB/s algorithmic")
    extra, dec16, dec65 = [], None, None
    if not args.no_extra_contexts:
        for c in (4096, 32768):
            if c != args.context:
                info, _ = decode_case(torch, kvarn, synth, c, args.steps, args.warmup, R)
                extra.append(info)
                log(f"decode context {c}: {info['us_per_step']:.2f} us per call, "
                    f"{info['achieved_GBps']:.0f} GB/s algorithmic")
        dec16, _ = decode_case(torch, kvarn, synth, args.context, args.steps, args.warmup, R, f16=True)
        log(f"decode context {args.context}, f16 scales: {dec16['us_per_step']:.2f} us per call")
        dec65, _ = decode_case(torch, kvarn, synth, args.context, args.steps, args.warmup, 5, kbits=6, vbits=5)
        log(f"decode context {args.context}, K6V5: {dec65['us_per_step']:.2f} us per call")

    verify = None
    if not args.no_verify:
        verify = verify_case(torch, kvarn, synth, args.context, 8, R)
        verify["vs_decode_call"] = verify["us_per_call"] / head["us_per_step"]
        log(f"verify width 8 at context {args.context}: {verify['us_per_call']:.2f} us per call "
            f"({verify['vs_decode_call']:.2f} decode calls)")

    q06, wide = None, []
    if not args.no_steps and not args.eager_wide:
        q06 = qwen06b_case(torch, kvarn, synth, args.step_reps)
        log(f"0.6B layer, 64 steps with appends: {q06['us_per_layer_step']:.2f} us per step, "
            f"{q06['kv_tokens_per_s']:.3g} KV tokens/s")
    if not args.no_steps:
        for name in ("wide_d256", "wide_d512"):
            info = wide_step_case(torch, kvarn, synth, name, 128, args.step_reps, args.eager_wide)
            wide.append(info)
            if args.eager_wide:
                continue
            log(f"wide batch head_dim {info['head_dim']}, 128 steps: {info['us_per_layer_step']:.1f} us per "
                f"step ({info['decode_only']['us_per_layer_step']:.1f} decode only), "
                f"{info['decode_only']['achieved_GBps']:.0f} GB/s decode")

    compress = None
    if not args.no_compress:
        compress = compress_case(torch, kvarn, synth, R)
        log(f"compress {compress['tile_heads']} tile-heads: {compress['us_per_launch']:.1f} us, "
            f"{compress['achieved_GBps']:.0f} GB/s")

    prefill, prefill_wide = None, []
    if not args.no_prefill:
        prefill = prefill_case(torch, kvarn, synth, SequenceCache, 128, 32, 8, 15488, 512, 5)
        log(f"prefill 15488 tokens: {prefill['ms']:.2f} ms ({prefill['algorithmic_TOPS']:.0f} TOPS)")
        for dw, hq, hkv in ((256, 16, 4), (512, 8, 1)):
            info = prefill_case(torch, kvarn, synth, SequenceCache, dw, hq, hkv, 4096, 512, 3)
            prefill_wide.append(info)
            log(f"prefill head_dim {dw}, 4096 tokens: {info['ms']:.2f} ms")

    floors = None
    if not args.no_floors:
        floors = floors_case(torch)
        log(f"floors: read 1 GiB {floors['read_1GiB']['GBps']:.0f} GB/s, read 16.75 MB "
            f"{floors['read_16.75MB']['us_per_launch']:.2f} us, fp16 MFMA "
            f"{floors['mfma_f16_16x16x32']['T_ops_per_s']:.0f} TFLOP/s, int8 "
            f"{floors['mfma_i8_16x16x64']['T_ops_per_s']:.0f} TOPS, empty launch {floors['empty_launch_us']:.2f} us")

    if args.calibration_copy:
        src = torch.empty(64 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 64 MiB device to device")

    ms_step = head["us_per_step"] * 1e-3
    alg = head["algorithmic_bytes"]
    achieved = head["achieved_GBps"]
    line = {
        "metric": "KV tokens attended/s (8B-shape decode @16k) + achieved HBM GB/s; prefill t/s",
        "value": head["kv_tokens_per_s"],
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "timed_regions": R,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic: seeded N(0,1) K/V/Q, lognormal per-channel K scales, 1% outlier "
                "channels at 10x",
        "config": {"workload": f"qwen3-8b-shape single-layer decode, batch 1, context {head['context']} "
                               f"({head['tiles']} tiles + {head['window']} window), Hq 32, Hkv 8, head_dim 128",
                   "layers_cycled": head["layers_cycled"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "kvarn_decode_attention (decode_split_kernel + decode_combine_kernel, "
                               "timed together as one call)",
                     "algorithmic_bytes_per_launch": alg, "launch_us": ms_step * 1e3,
                     "measured_read_floor_GBps": (floors or {}).get("read_16.75MB", {}).get("GBps")},
        "hbm_GBps": achieved,
        "decode_contexts": [head] + extra,
        "decode_f16_scales": dec16,
        "decode_k6v5": dec65,
        "verify": verify,
        "qwen3_0.6b_64_steps": q06,
        "wide_heads_batch16_steps": wide,
        "compress": compress,
        "prefill": prefill,
        "prefill_wide_heads": prefill_wide,
        "floors": floors,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
