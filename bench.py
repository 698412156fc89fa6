#!/usr/bin/env python3
"""Benchmark of the KVarN hot path on one MI355X.

Headline workload: Qwen3-8B-shaped single-layer batch-1 decode at a context of
15488 tokens (119 compressed 128-token tiles + a 256-token FP32 window; 32
query heads, 8 KV heads, head_dim 128).  One step = one kvarn_decode_attention
call: the split kernel (query rotation, every tile on the matrix cores, the
window tokens) and the log-sum-exp combine with its inverse WHT.  To keep the
caches honest the timed loop cycles through enough distinct layers (records +
windows + queries) to exceed twice the 256 MB last-level cache, all resident
in HBM before timing starts; the step sequence is captured once in a HIP
graph and timed with events on the replay stream, so the per-step time is the
device time of the two kernels back to back.

The same JSON line carries: the decode call's achieved algorithmic HBM
bandwidth against the 8 TB/s peak (roofline), decode at contexts 4096 and
32768, chunked-prefill throughput of the 15488-token prompt in 512-token
chunks (compress + rotate + prefill attention, one graph), compression
throughput, and the CPU oracle timed on a bounded sample of the decode
workload (cpu_baseline).

--calibration-copy adds one device-to-device copy of a known size, for
scaling hardware byte counters taken over the same run.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_MFMA_PEAK_TOPS = 5000.0
LLC_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "quantized_attention_tok_amd", "csrc")
DECODE_SOURCES = ["decode_split.hip", "kvarn_mfma.h", "kvarn_launch.h", "kvarn_device.h", "kvarn_api.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_ctx15488.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def decode_bytes(T, n_w, Hq, Hkv, d, tile_bytes):
    """Algorithmic bytes of one decode call: every record and window row read
    once, the query read once, the output written once."""
    return T * Hkv * tile_bytes + 2 * n_w * Hkv * d * 4 + Hq * d * 4 + Hq * d * 4


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


def graph_ms(torch, fn, n_inner, reps):
    """Capture fn() (n_inner steps) in a graph; return ms per step over reps replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / (reps * n_inner), g


def decode_case(torch, kvarn, synth, ctx, steps, warmup, seed=2, f16=False, kbits=4, vbits=2):
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
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run():
        for l in range(L):
            if k4v2:   # q_rot=None: the split kernel rotates q itself
                kvarn.decode_attention(qs[l], None, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                                       out=outs[l], workspace=ws, f16_scales=f16)
            else:      # the vector-unit kernels take a rotated query
                kvarn.rotate_query(qs[l], out=qr)
                kvarn.decode_attention(qs[l], qr, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                                       out=outs[l], workspace=ws, f16_scales=f16, kbits=kbits,
                                       vbits=vbits)

    reps = max(1, int(math.ceil(steps / L)))
    warm = max(1, int(math.ceil(warmup / L)))
    _, g = graph_ms(torch, run, L, 1)
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / (reps * L)
    alg = decode_bytes(T, n_w, Hq, Hkv, d, tb)
    info = {"context": ctx, "tiles": T, "window": n_w, "scales": "f16" if f16 else "f32",
            "key_bits": kbits, "value_bits": vbits, "record_bytes": tb, "layers_cycled": L,
            "us_per_step": ms * 1e3,
            "kv_tokens_per_s": ctx / (ms * 1e-3), "algorithmic_bytes": alg,
            "achieved_GBps": alg / (ms * 1e-3) / 1e9}
    return info, reps * L, warm * L, (K, V, rec0, T, n_w, qs, scale)


def wide_batch_case(torch, kvarn, synth, name, reps=10):
    """The batched wide-head decode workload: 16 sequences whose contexts are
    uniform in 1k-32k tokens in whole compressed tiles, each with a 256-token
    FP32 window; one step = the query rotation and one decode call for the
    batch, the records alternating between two copies (more than the LLC)."""
    w = synth.WORKLOADS[name]
    d, Hq, Hkv, W, B = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window, w.batch
    dev = "cuda:0"
    tiles = [int(t) for t in synth.ragged_contexts(w.seed, B, w.extra["ctx_lo"], w.extra["ctx_hi"], W)]
    tb = kvarn.tile_bytes(d)
    rec_start = [int(x) for x in np.cumsum([0] + tiles[:-1])]
    pool = torch.empty(sum(tiles), Hkv, tb, dtype=torch.uint8, device=dev)
    kw = torch.empty(B, W, Hkv, d, device=dev)
    vw = torch.empty_like(kw)
    for b in range(B):
        K, V = synth.batch_sequence_kv(w, b, 128 * tiles[b] + W)
        kd = torch.from_numpy(K).to(dev)
        vd = torch.from_numpy(V).to(dev)
        kvarn.compress_tile(kd, vd, pool[rec_start[b]:rec_start[b] + tiles[b]], tiles[b])
        kw[b] = kd[128 * tiles[b]:]
        vw[b] = vd[128 * tiles[b]:]
        del K, V, kd, vd
    pools = [pool, pool.clone()]
    q = torch.from_numpy(synth.make_q(w.seed, B, Hq, d)).to(dev)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    wins = [W] * B
    ws = torch.zeros(max(16, kvarn.decode_workspace_bytes(q, None, pool, rec_start, tiles, kw, vw, wins, scale)),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run():
        for p in pools:   # q_rot=None: the tile kernel rotates the queries itself
            kvarn.decode_attention(q, None, p, rec_start, tiles, kw, vw, wins, scale, out=out, workspace=ws)

    ms, _ = graph_ms(torch, run, len(pools), reps)
    alg = sum(decode_bytes(t, W, Hq, Hkv, d, tb) for t in tiles)
    kv_tokens = sum(128 * t + W for t in tiles)
    return {"head_dim": d, "n_q_heads": Hq, "n_kv_heads": Hkv, "batch": B, "tiles": tiles, "window": W,
            "us_per_step": ms * 1e3, "kv_tokens_per_s": kv_tokens / (ms * 1e-3), "algorithmic_bytes": alg,
            "achieved_GBps": alg / (ms * 1e-3) / 1e9, "includes": "query rotation, decode attention"}


def verify_case(torch, kvarn, synth, ctx, width, reps=20, seed=2, f16=False):
    """Multi-query verify of `width` draft rows at the 8B decode shape: one call
    reads every record once for all rows (the workload of a decode step)."""
    d, Hq, Hkv, W = 128, 32, 8, 256
    dev = "cuda:0"
    T = kvarn.visible_tiles(ctx - 1, W)
    n_w = ctx - 128 * T
    tb = kvarn.tile_bytes(d, f16)
    scale = 1.0 / math.sqrt(d)
    per_layer = T * Hkv * tb + 2 * n_w * Hkv * d * 4
    L = max(8, int(math.ceil(2 * LLC_BYTES / per_layer)))
    K, V = synth.make_kv(seed, ctx, Hkv, d, synth.outliers_for(d, 0.01))
    kd = torch.from_numpy(K).to(dev)
    vd = torch.from_numpy(V).to(dev)
    rec0 = torch.empty(T, Hkv, tb, dtype=torch.uint8, device=dev)
    kvarn.compress_tile(kd, vd, rec0, T, f16_scales=f16)
    recs = [rec0.clone() for _ in range(L)]
    kw = [kd[128 * T:].clone()[None] for _ in range(L)]
    vw = [vd[128 * T:].clone()[None] for _ in range(L)]
    qs = torch.from_numpy(synth.make_q(seed, L * width, Hq, d)).to(dev).reshape(L, 1, width, Hq, d)
    outs = torch.empty_like(qs)
    ws_bytes = kvarn.decode_workspace_bytes(qs[0], None, recs[0], [0], [T], kw[0], vw[0], [n_w], scale,
                                            f16_scales=f16)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def run():
        for l in range(L):
            kvarn.decode_attention(qs[l], None, recs[l], [0], [T], kw[l], vw[l], [n_w], scale,
                                   out=outs[l], workspace=ws, f16_scales=f16)

    ms, _ = graph_ms(torch, run, L, reps)
    return {"width": width, "context": ctx, "us_per_call": ms * 1e3,
            "query_rows_per_s": width / (ms * 1e-3), "layers_cycled": L,
            "algorithmic_bytes": decode_bytes(T, n_w, Hq, Hkv, d, tb)}


def prefill_case(torch, kvarn, synth, SequenceCache, d, Hq, Hkv, n, chunk, reps, W=256):
    """Chunked prefill of an n-token prompt in one graph: raw row copies, tile
    compression, query rotation (inside the prefill kernel at head_dim 128)
    and prefill attention for every chunk."""
    dev = "cuda:0"
    Kp, Vp = synth.make_kv(4, n, Hkv, d, synth.outliers_for(d, 0.01))
    Qp = synth.make_q(4, n, Hq, d)
    kp, vp, qp = (torch.from_numpy(x).to(dev) for x in (Kp, Vp, Qp))
    outp = torch.empty_like(qp)
    cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=dev)
    ws = None
    if d != 128:   # the vector-unit prefill keeps split partials in a workspace
        big = max(kvarn.prefill_workspace_bytes(qp[p0:p0 + min(chunk, n - p0)], qp[p0:p0 + min(chunk, n - p0)],
                                                cache.records, n // 128, cache.k, cache.v, 0, p0, W, 1.0)
                  for p0 in range(0, n, chunk))
        ws = torch.zeros(max(big, 16), dtype=torch.uint8, device=dev)

    def run_prefill():
        cache.n_tokens = cache.n_tiles = 0
        for p0 in range(0, n, chunk):
            c = min(chunk, n - p0)
            cache.append(kp[p0:p0 + c], vp[p0:p0 + c])
            q_c = qp[p0:p0 + c]
            q_r = None   # K4V2 records: the kernels rotate the rows themselves
            rb = 128 * kvarn.visible_tiles(p0, W)
            kvarn.prefill_attention(q_c, q_r, cache.records, cache.n_tiles, cache.k[rb:],
                                    cache.v[rb:], rb, p0, W, 1.0 / math.sqrt(d), out=outp[p0:p0 + c],
                                    workspace=ws)

    ms_p, _ = graph_ms(torch, run_prefill, 1, reps)
    pairs = n * (n + 1) // 2                            # causal (query, key) pairs per head
    ops = 2 * 2 * d * pairs * Hq                         # Q.K and P.V multiply-adds as 2 ops each
    return {"head_dim": d, "n_q_heads": Hq, "n_kv_heads": Hkv, "tokens_per_s": n / (ms_p * 1e-3),
            "ms": ms_p, "prompt": n, "chunk": chunk, "algorithmic_TOPS": ops / (ms_p * 1e-3) / 1e12,
            "int8_mfma_frac": ops / (ms_p * 1e-3) / 1e12 / INT8_MFMA_PEAK_TOPS,
            "includes": "raw row copies, tile compression, query rotation, prefill attention"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--context", type=int, default=15488)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra-contexts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy", action="store_true")
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

    head, steps, warm, keep = decode_case(torch, kvarn, synth, args.context, args.steps, args.warmup)
    log(f"decode context {head['context']}: {head['us_per_step']:.2f} us per call, "
        f"{head['achieved_GBps']:.0f} GB/s algorithmic")
    extra = []
    if not args.no_extra_contexts:
        for c in (4096, 32768):
            if c != args.context:
                info, _, _, _ = decode_case(torch, kvarn, synth, c, 320, 32)
                extra.append(info)
                log(f"decode context {c}: {info['us_per_step']:.2f} us per call, "
                    f"{info['achieved_GBps']:.0f} GB/s algorithmic")

    # ---- the same decode over records with f16 scales ----
    dec16 = None
    if not args.no_extra_contexts:
        dec16, _, _, _ = decode_case(torch, kvarn, synth, args.context, 320, 32, f16=True)
        log(f"decode context {args.context}, f16 scales: {dec16['us_per_step']:.2f} us per call, "
            f"{dec16['achieved_GBps']:.0f} GB/s algorithmic")
    # ---- and over K6V5 records (vector-unit kernels, query rotation in the step) ----
    dec65 = None
    if not args.no_extra_contexts:
        dec65, _, _, _ = decode_case(torch, kvarn, synth, args.context, 160, 16, kbits=6, vbits=5)
        log(f"decode context {args.context}, 6-bit keys / 5-bit values: {dec65['us_per_step']:.2f} us "
            f"per call, {dec65['achieved_GBps']:.0f} GB/s algorithmic")

    # ---- multi-query verify (width 8) at the same context ----
    verify = verify_case(torch, kvarn, synth, args.context, 8)
    verify["vs_decode_call"] = verify["us_per_call"] / head["us_per_step"]
    log(f"verify width 8 at context {args.context}: {verify['us_per_call']:.2f} us per call "
        f"({verify['vs_decode_call']:.2f} decode calls)")

    # ---- batched decode at the wide heads: 16 sequences, contexts 1k-32k ----
    wide_batch = []
    if not args.no_extra_contexts:
        for name in ("wide_d256", "wide_d512"):
            info = wide_batch_case(torch, kvarn, synth, name)
            wide_batch.append(info)
            log(f"batched decode head_dim {info['head_dim']} ({info['batch']} sequences, "
                f"{sum(info['tiles'])} tiles): {info['us_per_step']:.1f} us per step, "
                f"{info['achieved_GBps']:.0f} GB/s algorithmic")

    # ---- compression throughput (the prompt's 119 x 8 tile-heads in one launch) ----
    K, V, rec0, T, n_w, qs, scale = keep
    kd = torch.from_numpy(K).to(dev)
    vd = torch.from_numpy(V).to(dev)
    recc = torch.empty_like(rec0)
    ms_c, _ = graph_ms(torch, lambda: kvarn.compress_tile(kd, vd, recc, T), 1, 20)
    c_bytes = T * Hkv * (2 * 128 * d * 4 + kvarn.tile_bytes(d))
    compress = {"tile_heads": T * Hkv, "us_per_launch": ms_c * 1e3,
                "tile_heads_per_s": T * Hkv / (ms_c * 1e-3), "achieved_GBps": c_bytes / (ms_c * 1e-3) / 1e9}
    log(f"compress {T * Hkv} tile-heads: {ms_c * 1e3:.1f} us")

    # ---- chunked prefill of the 15488-token prompt (one graph of all chunks) ----
    prefill = None
    prefill_wide = []
    if not args.no_prefill:
        prefill = prefill_case(torch, kvarn, synth, SequenceCache, 128, Hq, Hkv, 15488, 512, 3)
        log(f"prefill {prefill['prompt']} tokens: {prefill['ms']:.2f} ms")
        for dw, hq, hkv in ((256, 16, 4), (512, 8, 1)):
            info = prefill_case(torch, kvarn, synth, SequenceCache, dw, hq, hkv, 4096, 512, 2)
            prefill_wide.append(info)
            log(f"prefill head_dim {dw}, {info['prompt']} tokens: {info['ms']:.2f} ms")

    if args.calibration_copy:
        src = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 64 MiB device to device")

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.no_cpu_baseline:
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:  # pragma: no cover
            threadpool_limits = None
        import oracle
        recs_np = rec0.cpu().numpy()
        q_all = qs[:, 0].cpu().numpy()
        lim = threadpool_limits(1) if threadpool_limits else None
        # whole decode steps (dequantise every record, attend every head), each with
        # the next layer's query, until about 10 s of one core's work
        n_steps, t0 = 0, time.perf_counter()
        while n_steps < 2 or (n_steps < 200 and time.perf_counter() - t0 < 10.0):
            kh, vh = oracle.dequant_records(recs_np, d)
            oracle.decode(q_all[n_steps % q_all.shape[0]], kh, vh, T, K[128 * T:], V[128 * T:], scale)
            n_steps += 1
        sec = time.perf_counter() - t0
        if lim is not None:
            lim.unregister()
        ctx = head["context"]
        cpu = {"value": n_steps * ctx / sec, "unit": "KV tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_steps} decode steps of the 8B-shaped layer at context {ctx}, each: "
                         f"dequantise {T * Hkv} records to fp64 and attend 32 heads over {ctx} keys "
                         f"({sec:.1f} s on one host core)"}
        log(f"cpu oracle: {n_steps} decode steps in {sec:.1f} s")

    ms_step = head["us_per_step"] * 1e-3
    alg = head["algorithmic_bytes"]
    achieved = head["achieved_GBps"]
    traffic = measured_traffic()
    line = {
        "metric": "KV tokens attended/s (8B-shape decode @16k) + achieved HBM GB/s; prefill t/s",
        "value": head["kv_tokens_per_s"],
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
        "config": {"workload": f"qwen3-8b-shape single-layer decode, batch 1, context {head['context']} "
                               f"({head['tiles']} tiles + {head['window']} window), Hq 32, Hkv 8, head_dim 128",
                   "layers_cycled": head["layers_cycled"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kvarn_decode_attention: decode_split_kernel + decode_combine_kernel",
                     "algorithmic_bytes_per_launch": alg, "launch_us": ms_step * 1e3},
        "hbm_GBps": achieved,
        "decode_contexts": [head] + extra,
        "decode_f16_scales": dec16,
        "decode_k6v5": dec65,
        "prefill": prefill,
        "prefill_wide_heads": prefill_wide,
        "verify": verify,
        "decode_wide_heads_batch16": wide_batch,
        "compress": compress,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
