"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's
callers.  This module holds none of the method's arithmetic: it only draws
random K, V and Q arrays and describes workload shapes.

Input recipe (stands in for the pages' Qwen3-0.6B / Qwen3-8B activations on
wikitext-2, which are not available here):
  K[t, h, c] = g * sigma[h, c] * o[h, c],  g ~ N(0, 1),
      sigma ~ lognormal(0, 1) fixed per (kv head, channel) for the sequence,
      o = 10 on seeded outlier channels (4 per head, or ceil(1% of d)), else 1;
  V ~ N(0, 1);  Q ~ N(0, 1);  all fp32.
Generator: numpy PCG64, sub-streams from SeedSequence(seed).spawn().
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TILE = 128


@dataclass(frozen=True)
class Workload:
    name: str
    head_dim: int
    n_q_heads: int
    n_kv_heads: int
    window: int
    n_outliers: int
    seed: int
    contexts: tuple = ()          # total KV length per sequence
    batch: int = 1
    steps: int = 0                # decode steps to run
    chunk: int = 0                # prefill chunk length
    extra: dict = field(default_factory=dict)


def outliers_for(d: int, fraction: float | None = None, count: int | None = None) -> int:
    if count is not None:
        return count
    return int(math.ceil(fraction * d))


# The five workloads.  Context conventions: for the decode workloads the
# context is the total KV length (compressed tiles + FP32 window).
WORKLOADS = {
    "tiny": Workload("tiny", 128, 1, 1, window=0, n_outliers=4, seed=0, contexts=(512,), steps=1),
    # 24 compressed tiles + a 256-token window, then 64 appended decode steps
    "qwen3_0.6b_decode": Workload("qwen3_0.6b_decode", 128, 16, 8, window=256, n_outliers=4,
                                  seed=1, contexts=(3072 + 256,), steps=64),
    "qwen3_8b_decode": Workload("qwen3_8b_decode", 128, 32, 8, window=256,
                                n_outliers=outliers_for(128, 0.01), seed=2,
                                contexts=(4096, 15488, 32768), steps=1),
    "wide_d256": Workload("wide_d256", 256, 16, 4, window=256, n_outliers=4, seed=3, batch=16,
                          extra={"ctx_lo": 1024, "ctx_hi": 32768}),
    "wide_d512": Workload("wide_d512", 512, 8, 1, window=256, n_outliers=4, seed=3, batch=16,
                          extra={"ctx_lo": 1024, "ctx_hi": 32768}),
    "qwen3_8b_prefill": Workload("qwen3_8b_prefill", 128, 32, 8, window=256,
                                 n_outliers=outliers_for(128, 0.01), seed=4,
                                 contexts=(15488,), chunk=512),
}


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def channel_profile(seed: int, n_kv: int, d: int, n_outliers: int):
    """Per-(kv head, channel) scale sigma * o used for K."""
    rs, ro = _streams(seed, 2)
    sigma = np.exp(rs.standard_normal((n_kv, d))).astype(np.float32)
    mult = np.ones((n_kv, d), np.float32)
    for h in range(n_kv):
        idx = ro.choice(d, size=n_outliers, replace=False)
        mult[h, idx] = 10.0
    return (sigma * mult).astype(np.float32)


def make_kv(seed: int, n_tokens: int, n_kv: int, d: int, n_outliers: int,
            profile: np.ndarray | None = None):
    """K, V: [n_tokens][n_kv][d] fp32 with the outlier-channel recipe."""
    if profile is None:
        profile = channel_profile(seed, n_kv, d, n_outliers)
    _, _, rk, rv = _streams(seed, 4)
    K = (rk.standard_normal((n_tokens, n_kv, d), dtype=np.float32) * profile[None]).astype(np.float32)
    V = rv.standard_normal((n_tokens, n_kv, d), dtype=np.float32)
    return K, V


def make_q(seed: int, n_rows: int, n_q: int, d: int):
    """Q: [n_rows][n_q][d] fp32 N(0, 1)."""
    rq = _streams(seed + 1000, 1)[0]
    return rq.standard_normal((n_rows, n_q, d), dtype=np.float32)


def batch_sequence_kv(w: Workload, b: int, n_tokens: int):
    """K, V of sequence b of a batched workload, from streams of its own."""
    return make_kv(w.seed * 1000 + b, n_tokens, w.n_kv_heads, w.head_dim, w.n_outliers)


def ragged_contexts(seed: int, batch: int, lo: int, hi: int, window: int):
    """Per-sequence compressed-tile counts for a ragged batch: a context drawn
    uniformly in [lo, hi] tokens and rounded to whole tiles, plus the window."""
    r = _streams(seed + 2000, 1)[0]
    ctx = r.integers(lo, hi + 1, size=batch)
    tiles = np.maximum(1, np.rint(ctx / TILE).astype(np.int64))
    return tiles


def window_offsets(seed: int, batch: int):
    """Per-sequence window fill beyond the W-token minimum at the start of a
    stepped run, uniform in [0, 128): over 128 appended tokens every sequence
    then promotes exactly one tile, at a step of its own."""
    r = _streams(seed + 3000, 1)[0]
    return r.integers(0, TILE, size=batch)
