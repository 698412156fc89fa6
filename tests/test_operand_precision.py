"""Which matrix-core operand format can carry the contractions of attention
over the records within the 1e-4 bar (CPU emulation, no GPU).

Issue #433 item 1 (SharpInference KVarN follow-ups) proposes an int8
tensor-core K-score GEMM against the 4-bit channel-major tile.  The codes are
exact in int8 (and in fp16), but the float operand of each contraction is not:
  scores:  sum_c q~_c zK[t][c]   with q~ = q' * kscale  (one row per query head)
  values:  sum_t w_t zV[t][c]    with w = p * vscale    (one row per query head)
A matrix-core format writes the float row as a sum of narrow terms that share
one power-of-two scale per row (per query head and tile); each term meets the
exact integer codes and accumulates exactly (int32) or in fp32.

This test emulates those formats on the 8B-shaped prefill workload (seeded
synthetic K/V with lognormal channel scales and 1% outlier channels, records
from the oracle) and measures the attention output against the exact fp64
evaluation of the same records:
  * one int8 term (7 bits below the row maximum) and two int8 terms (14 bits)
    miss the bar: with outlier channels and a softmax that spans many orders
    of magnitude, most elements sit far below their row's maximum;
  * three int8 terms pass, and so does the fp16 hi + lo pair the kernels use
    (each term keeps 11 significant bits relative to the element itself).
On gfx950 a 16x16x64 int8 matrix op takes the issue time of a 16x16x32 fp16
one, so three int8 terms cost 3/4 of the matrix time of the fp16 pair; that
caps a contraction at 1/3 of the int8 peak (fp16 pair: 1/4).
"""
import math

import numpy as np
import pytest

import oracle
from quantized_attention_tok_amd import synth

TAU_BAR = 1e-4


def _row_exponent(y):
    amax = np.max(np.abs(y), axis=-1, keepdims=True)
    return np.floor(np.log2(np.where(amax > 0, amax, 1.0)))


def int8_terms(y, nterms):
    """y as nterms int8 terms under one power-of-two scale per row: the row
    maximum maps into [64, 128); each term rounds the remainder (x 128) to
    the nearest integer in [-127, 127]."""
    s = 2.0 ** (6 - _row_exponent(y))
    r = np.asarray(y, np.float64) * s
    approx, f = np.zeros_like(r), 1.0
    for _ in range(nterms):
        t = np.clip(np.rint(r), -127, 127)
        approx += t / f
        r = (r - t) * 128.0
        f *= 128.0
    return approx / s


def fp16_terms(y, nterms):
    """y as fp16 terms under one power-of-two scale per row (maximum in
    [2^13, 2^14)): hi = fp16(y), lo = fp16(y - hi)."""
    s = (2.0 ** (13 - _row_exponent(y))).astype(np.float32)
    r = (np.asarray(y, np.float32) * s).astype(np.float32)
    approx = np.zeros(r.shape, np.float64)
    for _ in range(nterms):
        t = r.astype(np.float16)
        approx += t.astype(np.float64)
        r = (r - t.astype(np.float32)).astype(np.float32)
    return approx / s


FORMATS = {
    "exact": None,
    "int8x1": lambda y: int8_terms(y, 1),
    "int8x2": lambda y: int8_terms(y, 2),
    "int8x3": lambda y: int8_terms(y, 3),
    "fp16x1": lambda y: fp16_terms(y, 1),
    "fp16x2": lambda y: fp16_terms(y, 2),
}


@pytest.fixture(scope="module")
def workload():
    """The first 4096 tokens of the 8B-shaped prefill prompt (every tile has the
    distribution of the full 15488-token prompt's tiles)."""
    w = synth.WORKLOADS["qwen3_8b_prefill"]
    d, Hq, Hkv, W, n = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window, 4096
    K, V = synth.make_kv(w.seed, n, Hkv, d, w.n_outliers)
    Q = synth.make_q(w.seed, n, Hq, d)
    T = oracle.visible_tiles(n - 1, W)
    recs = oracle.compress_tiles(K, V, T)
    codes = [[oracle.unpack_codes(recs[j, h], d) for h in range(Hkv)] for j in range(T)]
    scales = [[oracle.record_scales(recs[j, h], d) for h in range(Hkv)] for j in range(T)]
    return dict(d=d, Hq=Hq, Hkv=Hkv, W=W, K=K, V=V, Q=Q, codes=codes, scales=scales,
                H=oracle.hadamard_f64(d))


def attention_row(wl, p, hq, qk_fmt, pv_fmt):
    """Output of query head hq at prompt position p (the decode view at p),
    with the two tile contractions in the given formats and everything else
    in fp64: scores tau * ktok_t (sum_c q~_c zK + sum_c q'_c kmin_c), values
    vchan_c (sum_t w_t zV + sum_t p_t vmin_t), window tokens raw."""
    d, G = wl["d"], wl["Hq"] // wl["Hkv"]
    kv, tau = hq // G, 1.0 / math.sqrt(d)
    T = oracle.visible_tiles(p, wl["W"])
    qrot = oracle.wht_f32(wl["Q"][p, hq][None])[0]
    S = []
    for j in range(T):
        sc, (zK, _) = wl["scales"][j][kv], wl["codes"][j][kv]
        qt = (qrot * sc["kscale"]).astype(np.float32)
        qa = qt.astype(np.float64) if qk_fmt is None else qk_fmt(qt)
        bias = float(np.dot(qrot.astype(np.float64), sc["kmin"].astype(np.float64)))
        S.append(tau * sc["ktok"].astype(np.float64) * (zK.astype(np.float64) @ qa + bias))
    lo = 128 * T
    kw = wl["K"][lo:p + 1, kv].astype(np.float64)
    vw = wl["V"][lo:p + 1, kv].astype(np.float64)
    Sw = tau * (kw @ wl["Q"][p, hq].astype(np.float64))
    m = max([s.max() for s in S] + [Sw.max()])
    o_rot, l = np.zeros(d), 0.0
    for j in range(T):
        sc, (_, zV) = wl["scales"][j][kv], wl["codes"][j][kv]
        pj = np.exp(S[j] - m)
        l += pj.sum()
        w = (pj.astype(np.float32) * sc["vscale"][:, 0]).astype(np.float32)
        wa = w.astype(np.float64) if pv_fmt is None else pv_fmt(w)
        u = float(np.dot(pj, sc["vmin"][:, 0].astype(np.float64)))
        o_rot += sc["vchan"].astype(np.float64) * (wa @ zV.astype(np.float64) + u)
    pw = np.exp(Sw - m)
    l += pw.sum()
    return (wl["H"] @ o_rot + pw @ vw) / l


ROWS = (700, 1500, 2600, 3500, 4095)


def rel_error(wl, qk, pv, heads=range(0, 32, 3)):
    num = den = 0.0
    for p in ROWS:
        for hq in heads:
            ref = attention_row(wl, p, hq, None, None)
            got = attention_row(wl, p, hq, FORMATS[qk], FORMATS[pv])
            num += float(np.sum((got - ref) ** 2))
            den += float(np.sum(ref ** 2))
    return math.sqrt(num / den)


def test_emulated_formats_reduce_to_exact():
    # the emulation itself: the exact format is the fp64 evaluation, and the
    # term decompositions converge to the float row as terms are added
    y = np.random.default_rng(0).standard_normal((4, 128)).astype(np.float32) * np.float32(3.0)
    y[:, 5] *= np.float32(1e3)
    errs = [np.max(np.abs(int8_terms(y, k) - y)) for k in (1, 2, 3, 4)]
    assert all(b < a for a, b in zip(errs, errs[1:]))
    assert np.max(np.abs(fp16_terms(y, 2) - y) / np.abs(y)) < 2.0 ** -20


@pytest.mark.parametrize("qk,pv,passes", [
    ("int8x1", "exact", False), ("int8x2", "exact", False), ("exact", "int8x2", False),
    ("int8x3", "int8x3", True), ("fp16x1", "exact", False), ("exact", "fp16x1", False),
    ("fp16x2", "fp16x2", True)])
def test_operand_format_against_the_bar(workload, qk, pv, passes):
    err = rel_error(workload, qk, pv)
    print(f"scores {qk}, values {pv}: rel L2 {err:.2e}")
    if passes:
        assert err < TAU_BAR / 10      # inside the bar with an order of magnitude to spare
    else:
        assert err > TAU_BAR           # fails the bar
