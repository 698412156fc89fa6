#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Headline workload: Qwen3-8B-shaped single-layer batch-1 decode at a context of
15488 tokens (119 compressed 128-token tiles + a 256-token FP32 window; 32
query heads, 8 KV heads, head_dim 128).  One step = one kvarn_decode_attention
launch that rotates the query, scores and aggregates every tile on the matrix
cores and the window on the vector units, and combines the split partials with
LSE weights and one inverse WHT.  To keep
the caches honest the timed loop cycles through enough distinct layers (records
+ windows + queries) to exceed the 256 MB last-level cache, all resident in HBM
before timing starts; the step sequence is captured once in a HIP graph.

The same JSON line carries: the decode attention launch's achieved HBM
bandwidth against the 8 TB/s peak (roofline), chunked-prefill throughput of
the 15488-token prompt (512-token chunks), compression throughput, and the CPU
oracle timed on a bounded sample of the decode workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LLC_BYTES = 256 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_bytes(T, n_w, Hq, Hkv, d, tile_bytes):
    """Algorithmic bytes of one decode attention launch: every record and window
    row read once, the query read once, the output written once."""
    return T * Hkv * tile_bytes + 2 * n_w * Hkv * d * 4 + 2 * Hq * d * 4 + Hq * d * 4


def time_graph(torch, g, replays):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(replays):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--context", type=int, default=15488)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the KVarN path here runs on a single MI355X)", flush=True)
        sys.exit(2)

    import torch
    from quantized_attention_tok_amd import kvarn, synth
    from quantized_attention_tok_amd.cache import SequenceCache

    dev = "cuda:0"
    kvarn.lib()  # fails loudly if the HIP library is missing
    d, Hq, Hkv, W = 128, 32, 8, 256
    ctx = args.context
    T = kvarn.visible_tiles(ctx - 1, W)
    n_w = ctx - 128 * T
    tb = kvarn.tile_bytes(d)
    scale = 1.0 / math.sqrt(d)
    per_layer = T * Hkv * tb + 2 * n_w * Hkv * d * 4
    L = max(8, int(math.ceil(2 * LLC_BYTES / per_layer)))
    steps = int(math.ceil(args.steps / L)) * L
    warm = int(math.ceil(max(args.warmup, 1) / L)) * L
    log(f"context {ctx}: {T} tiles + {n_w} window tokens; {L} layers of {per_layer / 2**20:.1f} MiB")

    # ---- inputs resident in HBM ----
    K, V = synth.make_kv(2, ctx, Hkv, d, synth.outliers_for(d, 0.01))
    kd = torch.from_numpy(K).to(dev)
    vd = torch.from_numpy(V).to(dev)
    rec0 = torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev)
    kvarn.compress_tile(kd, vd, rec0, T)
    recs = [rec0.clone() for _ in range(L)]
    kw = [kd[128 * T:].clone()[None] for _ in range(L)]
    vw = [vd[128 * T:].clone()[None] for _ in range(L)]
    qs = torch.from_numpy(synth.make_q(2, L, Hq, d)).to(dev).reshape(L, 1, Hq, d)
    qr = torch.empty_like(qs)
    outs = torch.empty_like(qs)
    ws_bytes = kvarn.decode_workspace_bytes(qs[0], qs[0], recs[0], [0], [T], kw[0], vw[0], [n_w], scale)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(l):
        # one launch: query rotation, tile and window partials, LSE combine,
        # inverse WHT (q_rot=None makes the kernel rotate q itself)
        kvarn.decode_attention(qs[l], None, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                               out=outs[l], workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for l in range(L):
            step(l)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g_step = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        for l in range(L):
            step(l)

    time_graph(torch, g_step, warm // L)
    ms = time_graph(torch, g_step, steps // L)
    ms_step = ms / steps
    # per-launch kernel time: HIP events bracketing each launch on its stream
    n_ev = 4 * L
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    for i in range(n_ev):
        ev[i][0].record()
        step(i % L)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms_attn = sorted(a.elapsed_time(e) for a, e in ev)[n_ev // 2]
    alg = decode_bytes(T, n_w, Hq, Hkv, d, tb)
    achieved = alg / (ms_attn * 1e-3) / 1e9
    value = ctx / (ms_step * 1e-3)
    log(f"step {ms_step * 1e3:.2f} us (graph), launch {ms_attn * 1e3:.2f} us (events, median), "
        f"{achieved:.0f} GB/s algorithmic")

    # ---- compression throughput (the prompt's 119 x 8 tile-heads in one launch) ----
    recc = torch.empty_like(rec0)
    g_c = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        kvarn.compress_tile(kd, vd, recc, T)
    torch.cuda.synchronize()
    with torch.cuda.graph(g_c):
        kvarn.compress_tile(kd, vd, recc, T)
    time_graph(torch, g_c, 3)
    n_c = 20
    ms_c = time_graph(torch, g_c, n_c) / n_c
    c_bytes = T * Hkv * (2 * 128 * d * 4 + tb)
    compress = {"tile_heads_per_s": T * Hkv / (ms_c * 1e-3), "ms_per_launch": ms_c,
                "achieved_GBps": c_bytes / (ms_c * 1e-3) / 1e9}
    log(f"compress {T * Hkv} tile-heads: {ms_c:.3f} ms")

    # ---- chunked prefill of the 15488-token prompt ----
    prefill = None
    if not args.no_prefill:
        n, chunk = 15488, 512
        Kp, Vp = synth.make_kv(4, n, Hkv, d, synth.outliers_for(d, 0.01))
        Qp = synth.make_q(4, n, Hq, d)
        kp, vp, qp = (torch.from_numpy(x).to(dev) for x in (Kp, Vp, Qp))
        pre_ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)

        def run_prefill():
            cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=dev)
            for p0 in range(0, n, chunk):
                c = min(chunk, n - p0)
                cache.append(kp[p0:p0 + c], vp[p0:p0 + c])
                q_c = qp[p0:p0 + c]
                q_r = kvarn.rotate_query(q_c)
                rb = 128 * kvarn.visible_tiles(p0, W)
                kvarn.prefill_attention(q_c, q_r, cache.records, cache.n_tiles, cache.k[rb:],
                                        cache.v[rb:], rb, p0, W, scale, workspace=pre_ws)
            return cache

        run_prefill()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 2
        for _ in range(reps):
            run_prefill()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / reps
        prefill = {"tokens_per_s": n / sec, "ms": sec * 1e3, "prompt": n, "chunk": chunk}
        log(f"prefill {n} tokens: {sec * 1e3:.1f} ms")

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        import oracle
        recs_np = rec0.cpu().numpy()
        q_np = qs[0, 0].cpu().numpy()
        lim = threadpool_limits(1) if threadpool_limits else None
        t0 = time.perf_counter()
        kh, vh = oracle.dequant_records(recs_np, d)
        oracle.decode(q_np, kh, vh, T, K[128 * T:], V[128 * T:], scale)
        sec = time.perf_counter() - t0
        if lim is not None:
            lim.unregister()
        cpu = {"value": ctx / sec, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"one decode step of the 8B-shaped layer at context {ctx}: dequantise "
                         f"{T * Hkv} records to fp64 and attend 32 heads over {ctx} keys "
                         f"({sec:.1f} s on one host core)"}
        log(f"cpu oracle: {sec:.1f} s per decode step")

    line = {
        "metric": "KV tokens attended/s (8B-shape decode @16k) + achieved HBM GB/s; prefill t/s",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: seeded N(0,1) K/V/Q, lognormal per-channel K scales, 1% outlier "
                "channels at 10x",
        "config": {"workload": f"qwen3-8b-shape single-layer decode, batch 1, context {ctx} "
                               f"({T} tiles + {n_w} window), Hq 32, Hkv 8, head_dim 128",
                   "layers_cycled": L},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_fused_kernel (kvarn_decode_attention, one launch)",
                     "algorithmic_bytes_per_launch": alg, "launch_us": ms_attn * 1e3},
        "hbm_GBps": achieved,
        "prefill": prefill,
        "compress": compress,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
