"""Pins of the CPU oracle to facts outside itself: closed forms, textbook and
library special cases, invariants the pages state, and the one numeric figure
the pages print that fixes the record size.  CPU only."""
import decimal
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from quantized_attention_tok_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
DIMS = [128, 256, 512]


# --------------------------------------------------------------------------
# Walsh-Hadamard rotation (issue #180, Algorithm step 1: orthonormal, so it
# preserves attention scores)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", DIMS)
def test_wht_scale_is_correctly_rounded(d):
    decimal.getcontext().prec = 60
    exact = decimal.Decimal(1) / decimal.Decimal(d).sqrt()
    c = oracle.wht_scale(d)
    # the neighbours of c in fp32 must both be farther from the exact value
    up = np.nextafter(c, np.float32(1))
    dn = np.nextafter(c, np.float32(0))
    err = abs(decimal.Decimal(float(c)) - exact)
    assert err <= abs(decimal.Decimal(float(up)) - exact)
    assert err <= abs(decimal.Decimal(float(dn)) - exact)


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_matches_library(d):
    H = oracle.hadamard_f64(d)
    assert np.array_equal(H, scipy.linalg.hadamard(d) / np.sqrt(d))
    assert np.allclose(H @ H, np.eye(d), atol=1e-13)
    e0 = np.zeros(d); e0[0] = 1
    assert np.allclose(H @ e0, np.full(d, 1 / np.sqrt(d)), atol=1e-15)


@pytest.mark.parametrize("d", DIMS)
def test_wht_f32_matches_library_transform(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((8, d)).astype(np.float32) * 3
    y = oracle.wht_f32(x)
    ref = x.astype(np.float64) @ (scipy.linalg.hadamard(d) / np.sqrt(d)).T
    bound = (math.log2(d) + 2) * np.finfo(np.float32).eps * np.abs(x).sum(1, keepdims=True) / np.sqrt(d)
    assert np.all(np.abs(y - ref) <= bound)


@pytest.mark.parametrize("d", DIMS)
def test_wht_integer_inputs_single_final_scale(d):
    # Integer inputs make every butterfly exact, so the result must be the
    # exact integer transform times c_d with one rounding: this pins a single
    # scale at the end (not a 1/sqrt(2) per stage).
    rng = np.random.default_rng(1 + d)
    x = rng.integers(-50, 50, size=(4, d)).astype(np.float32)
    exact = (x.astype(np.float64) @ scipy.linalg.hadamard(d).T).astype(np.float32)
    want = exact * oracle.wht_scale(d)
    assert np.array_equal(oracle.wht_f32(x), want)


@pytest.mark.parametrize("d", DIMS)
def test_wht_self_inverse_and_preserves_dot(d):
    rng = np.random.default_rng(7 + d)
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    qq = oracle.wht_f32(oracle.wht_f32(q))
    assert np.max(np.abs(qq - q)) <= 4 * math.log2(d) * np.finfo(np.float32).eps * np.abs(q).max() * 4
    dot = float(np.dot(q.astype(np.float64), k))
    dot_rot = float(np.dot(oracle.wht_f32(q).astype(np.float64), oracle.wht_f32(k)))
    assert abs(dot - dot_rot) <= 1e-5 * np.linalg.norm(q) * np.linalg.norm(k)


# --------------------------------------------------------------------------
# Pairwise summation order
# --------------------------------------------------------------------------

def test_pairwise_sum_worked_cases():
    e = np.float32(2.0 ** -24)
    # contiguous halves: (1 + e) + (e + e) = 1 + 2^-23 ; a sequential sum gives 1
    assert oracle.pairwise_sum_f32(np.array([1, e, e, e], np.float32)) == np.float32(1 + 2.0 ** -23)
    # contiguous halves: (1 + e) + (0 + e) = 1 ; pairing 0 with 2 would give 1 + 2^-23
    assert oracle.pairwise_sum_f32(np.array([1, e, 0, e], np.float32)) == np.float32(1.0)


@pytest.mark.parametrize("n", [128, 256, 512])
def test_pairwise_sum_error_bound(n):
    rng = np.random.default_rng(n)
    y = (rng.standard_normal(n) * np.exp(rng.standard_normal(n) * 2)).astype(np.float32)
    exact = math.fsum(float(v) for v in y)
    got = float(oracle.pairwise_sum_f32(y))
    assert abs(got - exact) <= math.log2(n) * np.finfo(np.float32).eps * np.abs(y.astype(np.float64)).sum()


# --------------------------------------------------------------------------
# Sinkhorn (issue #180, Algorithm step 2: dual-axis alternation of per-channel
# and per-token std normalisation)
# --------------------------------------------------------------------------

def _rotated_tile(seed, d, n_out):
    K, V = synth.make_kv(seed, 128, 1, d, n_out)
    return oracle.wht_f32(K[:, 0]), oracle.wht_f32(V[:, 0])


@pytest.mark.parametrize("d,n_out", [(128, 4), (128, 2), (256, 4), (512, 4)])
def test_sinkhorn_drives_both_axes_to_unit_spread(d, n_out):
    for X in _rotated_tile(10 + d + n_out, d, n_out):
        r, s = oracle.sinkhorn_f32(X, 8)
        Y = X.astype(np.float64) / (r[:, None].astype(np.float64) * s[None, :])
        row = np.abs(np.log(np.sqrt(np.mean(Y * Y, axis=1))))
        col = np.abs(np.log(np.sqrt(np.mean(Y * Y, axis=0))))
        assert row.max() < 1e-6
        assert col.max() < 1e-5


def test_sinkhorn_converges_geometrically():
    X, _ = _rotated_tile(3, 128, 2)
    errs = []
    for it in (1, 2, 4, 8):
        r, s = oracle.sinkhorn_f32(X, it)
        Y = X.astype(np.float64) / (r[:, None].astype(np.float64) * s[None, :])
        errs.append(np.abs(np.log(np.mean(Y * Y, axis=0))).max())
    assert errs[0] > errs[1] > errs[2] > errs[3]
    assert errs[3] < 1e-5


@pytest.mark.parametrize("d", DIMS)
def test_sinkhorn_rank_one_sign_pattern_closed_form(d):
    # X = u_t v_c eps_tc with eps = +-1 normalises to eps after one iteration:
    # s_c = v_c sqrt(mean u^2), r_t = u_t / sqrt(mean u^2).
    rng = np.random.default_rng(d)
    u = np.exp(rng.standard_normal(128)).astype(np.float32)
    v = np.exp(rng.standard_normal(d)).astype(np.float32)
    eps = np.where(rng.random((128, d)) < 0.5, -1.0, 1.0).astype(np.float32)
    X = (u[:, None] * v[None, :] * eps).astype(np.float32)
    r, s = oracle.sinkhorn_f32(X, 8)
    mu = np.sqrt(np.mean(u.astype(np.float64) ** 2))
    assert np.allclose(s, v * mu, rtol=2e-6)
    assert np.allclose(r, u / mu, rtol=2e-6)
    Xn = oracle.normalise_f32(X, r, s)
    assert np.allclose(Xn, eps, rtol=0, atol=4e-6)


def test_sinkhorn_power_of_two_equivariance():
    # The channel step comes first, so scaling one channel by 2^k scales its
    # s_c by exactly 2^k and changes no other bit (codes included).
    X, V = _rotated_tile(5, 128, 4)
    r, s = oracle.sinkhorn_f32(X, 8)
    Y = X.copy()
    Y[:, 17] *= np.float32(8.0)
    r2, s2 = oracle.sinkhorn_f32(Y, 8)
    assert s2[17] == s[17] * 8
    mask = np.ones(128, bool); mask[17] = False
    assert np.array_equal(s2[mask], s[mask]) and np.array_equal(r2, r)
    assert np.array_equal(oracle.normalise_f32(Y, r2, s2), oracle.normalise_f32(X, r, s))
    # A token scaled by 2^k reaches the same normalised tile (the fixed point is
    # unique up to the r/s gauge), to the fp32 convergence floor.
    Z = X.copy()
    Z[40, :] *= np.float32(0.25)
    r3, s3 = oracle.sinkhorn_f32(Z, 8)
    assert np.allclose(oracle.normalise_f32(Z, r3, s3), oracle.normalise_f32(X, r, s),
                       rtol=2e-5, atol=1e-6)


@pytest.mark.parametrize("d", [128, 512])
def test_sinkhorn_matches_independent_fp64_alternation(d):
    # The literal alternation in fp64: Y <- Y / colrms(Y), then Y <- Y / rowrms(Y),
    # accumulating the divisors; same fixed point and iterates as the oracle.
    X, _ = _rotated_tile(21, d, 4)
    Y = X.astype(np.float64)
    racc = np.ones(128); sacc = np.ones(d)
    for _ in range(8):
        cs = np.sqrt(np.mean(Y * Y, axis=0)); Y /= cs[None, :]; sacc *= cs
        rs = np.sqrt(np.mean(Y * Y, axis=1)); Y /= rs[:, None]; racc *= rs
    r, s = oracle.sinkhorn_f32(X, 8)
    # the oracle reports s from the last channel step alone: the fp64 divisor
    # product, divided by the token factors common to every channel
    assert np.allclose(r * s[0], racc * sacc[0], rtol=2e-5)
    assert np.allclose(s / s[0], sacc / sacc[0], rtol=2e-5)
    assert np.allclose(np.outer(r, s), np.outer(racc, sacc), rtol=2e-5)


def test_sinkhorn_degenerate_zero_column_and_row():
    X, _ = _rotated_tile(9, 128, 4)
    X = X.copy()
    X[:, 5] = 0
    X[77, :] = 0
    r, s = oracle.sinkhorn_f32(X, 8)
    assert np.all(np.isfinite(r)) and np.all(np.isfinite(s))
    assert s[5] == 1.0 and r[77] == 1.0
    assert np.all(np.isfinite(oracle.normalise_f32(X, r, s)))


# --------------------------------------------------------------------------
# Asymmetric RTN (issue #180, Algorithm step 3; codes in [0,15] and [0,3])
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 2])
def test_rtn_range_endpoints_and_error_bound(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    for _ in range(20):
        x = (rng.standard_normal(128) * rng.exponential()).astype(np.float32)
        lo, dl, z = oracle.rtn_group(x, bits)
        assert lo == x.min() and z.min() == 0 and z.max() == L
        assert z[np.argmin(x)] == 0 and z[np.argmax(x)] == L
        deq = lo.astype(np.float64) + z * np.float64(dl)
        assert np.all(np.abs(deq - x) <= dl / 2 * (1 + 1e-5) + 1e-30)


@pytest.mark.parametrize("bits", [4, 2])
def test_rtn_arithmetic_progression_round_trips(bits):
    L = (1 << bits) - 1
    lo, step = np.float32(-1.5), np.float32(0.125)
    k = np.arange(L + 1)
    x = (lo + k * step).astype(np.float32)
    glo, dl, z = oracle.rtn_group(np.resize(x, 128), bits)
    assert glo == lo and dl == step
    assert np.array_equal(np.unique(z), k)


def test_rtn_ties_round_to_even_and_constant_group():
    x = np.zeros(128, np.float32)
    x[0], x[1] = 0.0, 15.0    # lo = 0, delta = 1 exactly
    x[2], x[3], x[4] = 2.5, 3.5, 14.5
    lo, dl, z = oracle.rtn_group(x, 4)
    assert dl == 1.0 and (z[2], z[3], z[4]) == (2, 4, 14)
    lo, dl, z = oracle.rtn_group(np.full(128, 0.75, np.float32), 2)
    assert lo == np.float32(0.75) and dl == 0 and not z.any()


# --------------------------------------------------------------------------
# Record layout and size (PR #434 commit list: channel-major K, token-major V,
# 2-bit bit packing; "Measured" table: capacity figure)
# --------------------------------------------------------------------------

def test_record_size_reproduces_capacity_figure():
    pin = json.load(open(os.path.join(HERE, "golden", "capacity_pin.json")))
    d, W = pin["head_dim"], pin["window"]
    fp32_token = 2 * d * 4
    budget = pin["fp32_context"] * fp32_token
    tiles = (budget - W * fp32_token) // oracle.tile_bytes(d)
    assert tiles * 128 + W == pin["kvarn_context"]
    # a layout with two more f32 vectors per tile-head would not reproduce it
    alt = oracle.tile_bytes(d) + 2 * 128 * 4
    assert ((budget - W * fp32_token) // alt) * 128 + W != pin["kvarn_context"]
    assert [oracle.tile_bytes(x) for x in DIMS] == [15360, 30208, 59904]


@pytest.mark.parametrize("d", DIMS)
def test_layout_sections_aligned_and_contiguous(d):
    off = oracle.layout(d)
    vals = list(off.values())
    assert vals == sorted(vals) and all(v % 16 == 0 for v in vals)
    assert off["vcode"] - off["kcode"] == d * 128 // 2
    assert off["ktok"] - off["vcode"] == d * 128 // 4
    assert off["end"] == oracle.tile_bytes(d)


def test_packing_nibble_and_crumb_order():
    K, V = synth.make_kv(11, 128, 1, 128, 4)
    rec = oracle.compress_tile(K[:, 0], V[:, 0])
    zK, zV = oracle.unpack_codes(rec, 128)
    off = oracle.layout(128)
    for c in (0, 3, 127):
        for j in (0, 5, 63):
            b = rec[off["kcode"] + 64 * c + j]
            assert b & 15 == zK[2 * j, c] and b >> 4 == zK[2 * j + 1, c]
    for t in (0, 64, 127):
        for j in (0, 9, 31):
            b = int(rec[off["vcode"] + 32 * t + j])
            assert [(b >> (2 * i)) & 3 for i in range(4)] == list(zV[t, 4 * j:4 * j + 4])
    assert zK.max() <= 15 and zV.max() <= 3


@pytest.mark.parametrize("d", DIMS)
def test_codes_match_rtn_of_normalised_tile(d):
    K, V = synth.make_kv(12 + d, 128, 1, d, 4)
    rec = oracle.compress_tile(K[:, 0], V[:, 0])
    zK, zV = oracle.unpack_codes(rec, d)
    sc = oracle.record_scales(rec, d)
    X = oracle.wht_f32(K[:, 0])
    r, s = oracle.sinkhorn_f32(X, 8)
    Xn = oracle.normalise_f32(X, r, s)
    for c in (0, d // 3, d - 1):
        lo, dl, z = oracle.rtn_group(Xn[:, c], 4)
        assert np.array_equal(z, zK[:, c])
        assert sc["kscale"][c] == dl * s[c] and sc["kmin"][c] == lo * s[c]
    assert np.array_equal(sc["ktok"], r)
    Xv = oracle.wht_f32(V[:, 0])
    rv, sv = oracle.sinkhorn_f32(Xv, 8)
    Xvn = oracle.normalise_f32(Xv, rv, sv)
    for t in (0, 77):
        for g in range(d // 128):
            lo, dl, z = oracle.rtn_group(Xvn[t, 128 * g:128 * (g + 1)], 2)
            assert np.array_equal(z, zV[t, 128 * g:128 * (g + 1)])
            assert sc["vscale"][t, g] == dl * rv[t] and sc["vmin"][t, g] == lo * rv[t]
    assert np.array_equal(sc["vchan"], sv)


# --------------------------------------------------------------------------
# Dequantised cache and attention
# --------------------------------------------------------------------------

def _lossless_tile(d, seed):
    """Raw K whose rotated tile is u_t v_c eps_tc: it sits on the 4-bit and
    2-bit grids after normalisation, so compression is exact up to fp32
    rounding."""
    rng = np.random.default_rng(seed)
    u = np.exp(0.5 * rng.standard_normal(128))
    v = np.exp(rng.standard_normal(d))
    eps = np.where(rng.random((128, d)) < 0.5, -1.0, 1.0)
    Xrot = u[:, None] * v[None, :] * eps
    H = oracle.hadamard_f64(d)
    return (Xrot @ H.T).astype(np.float32)


@pytest.mark.parametrize("d", DIMS)
def test_lossless_tile_round_trips_through_record(d):
    K = _lossless_tile(d, 30 + d)
    V = _lossless_tile(d, 31 + d)
    rec = oracle.compress_tile(K, V)
    kh, vh = oracle.dequant(rec, d)
    assert np.linalg.norm(kh - K) / np.linalg.norm(K) < 2e-5
    assert np.linalg.norm(vh - V) / np.linalg.norm(V) < 2e-5


def test_attention_special_cases_and_lossless_equivalence():
    d, G = 128, 4
    rng = np.random.default_rng(5)
    K = _lossless_tile(d, 40)[:, None, :]
    V = _lossless_tile(d, 41)[:, None, :]
    rec = oracle.compress_tile(K[:, 0], V[:, 0])[None, None]
    kh, vh = oracle.dequant_records(rec, d)
    q = rng.standard_normal((G, d)).astype(np.float32)
    empty = np.zeros((0, 1, d), np.float32)
    tau = 1 / np.sqrt(d)
    out = oracle.decode(q, kh, vh, 1, empty, empty, tau)
    # textbook attention on the raw (uncompressed) tile
    s = tau * (q.astype(np.float64) @ K[:, 0].astype(np.float64).T)
    p = np.exp(s - s.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    ref = p @ V[:, 0].astype(np.float64)
    assert np.linalg.norm(out - ref) / np.linalg.norm(ref) < 1e-5
    # q = 0: plain mean of the visible values
    out0 = oracle.decode(np.zeros((1, d), np.float32), kh, vh, 1, empty, empty, tau)
    assert np.allclose(out0[0], vh[:, 0].mean(0), atol=1e-12)
    # one dominant key
    qd = (kh[37, 0] * 1e3).astype(np.float32)[None]
    outd = oracle.decode(qd, kh, vh, 1, empty, empty, tau)
    assert np.allclose(outd[0], vh[37, 0], atol=1e-9)


def test_attention_python_and_c_agree_and_rotated_identity():
    d = 128
    K, V = synth.make_kv(13, 256, 1, d, 4)
    rec = oracle.compress_tile(K[:128, 0], V[:128, 0])
    kd, vd = oracle.dequant_rotated(rec, d)
    kh, vh = oracle.dequant(rec, d)
    rng = np.random.default_rng(0)
    q = rng.standard_normal(d)
    H = oracle.hadamard_f64(d)
    # q . khat == (H q) . k'   (orthogonal rotation; colibri PR #399 review note)
    assert np.allclose(kh @ q, kd @ (H @ q), rtol=1e-12, atol=1e-12)
    keys = np.concatenate([kh, K[128:, 0]]); vals = np.concatenate([vh, V[128:, 0]])
    o1, l1 = oracle.attend(q, keys, vals, 0.1)
    o2, l2 = oracle.attend_c(q, keys, vals, 0.1)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14) and abs(l1 - l2) < 1e-12
    # window-only attention (no tiles) is plain softmax attention on raw K, V
    empty = np.zeros((0, 1, d))
    q32 = q.astype(np.float32)
    out = oracle.decode(q32[None], empty, empty, 0, K[:, :1], V[:, :1], 0.1)
    s = 0.1 * (K[:, 0].astype(np.float64) @ q32.astype(np.float64))
    p = np.exp(s - s.max()); p /= p.sum()
    assert np.allclose(out[0], p @ V[:, 0], rtol=1e-12, atol=1e-14)


def test_sinkhorn_reduces_reconstruction_error_on_outlier_keys():
    # sanity (comparative): normalisation helps per-channel 4-bit keys
    K, V = synth.make_kv(14, 128, 1, 128, 4)
    err = []
    for iters in (0, 8):
        rec = oracle.compress_tile(K[:, 0], V[:, 0], iters)
        kh, vh = oracle.dequant(rec, 128)
        err.append(np.linalg.norm(vh - V[:, 0]) / np.linalg.norm(V[:, 0]))
    assert err[1] < err[0]


def test_visible_tile_rule_fits_the_workloads():
    # FP32 window of W tokens, promote the oldest 128 when it reaches W + 128
    assert oracle.visible_tiles(511, 0) == 4                         # tiny: 512 tokens, window 0
    for total, tiles in [(4096, 30), (15488, 119), (32768, 254)]:
        assert oracle.visible_tiles(total - 1, 256) == tiles
        assert total - 128 * tiles == 256
    # 24 tiles + 256 window + 64 appended tokens: no promotion inside the run
    assert oracle.visible_tiles(3072 + 256 + 63, 256) == 24
    assert oracle.visible_tiles(3072 + 256 + 127, 256) == 25
    assert oracle.visible_tiles(254, 256) == 0


def test_verify_rows_are_prefill_views_and_last_row_is_decode():
    """gmlx PR #116 commit list (verify widths 2-8 attend the records): row i of
    a width-w verify over (T tiles, n_w window tokens) is the chunked-prefill
    output at position 128 T + n_w - w + i under the window rule with
    W' = n_w - w + 1 (each such row sees exactly T tiles), computed through
    visible_tiles and raw-token slicing rather than window prefixes; the last
    row is the ordinary decode query."""
    d, Hq, Hkv, T, n_w, w = 128, 4, 2, 2, 11, 5
    K, V = synth.make_kv(61, 128 * T + n_w, Hkv, d, 2)
    q = synth.make_q(61, w, Hq, d)
    recs = oracle.compress_tiles(K, V, T)
    kh, vh = oracle.dequant_records(recs, d)
    scale = 1 / np.sqrt(d)
    got = oracle.verify(q, kh, vh, T, K[128 * T:], V[128 * T:], scale)
    Wp = n_w - w + 1
    for i in range(w):
        pos = 128 * T + n_w - w + i
        assert oracle.visible_tiles(pos, Wp) == T
        ref = oracle.prefill_row(q[i], pos, Wp, kh, vh, K, V, scale)
        assert np.allclose(got[i], ref, rtol=0, atol=1e-13)
    last = oracle.decode(q[w - 1], kh, vh, T, K[128 * T:], V[128 * T:], scale)
    assert np.array_equal(got[w - 1], last)
    # an earlier row differs from the full-window decode (it must not see later drafts)
    full0 = oracle.decode(q[0], kh, vh, T, K[128 * T:], V[128 * T:], scale)
    assert np.linalg.norm(got[0] - full0) > 1e-6


# --------------------------------------------------------------------------
# f16 scales in the record (SharpInference issue #433 item 3)
# --------------------------------------------------------------------------

def test_f16_rounding_matches_numpy_half_conversion():
    """The oracle's binary32 -> binary16 conversion is IEEE round-to-nearest-even:
    numpy's float16 cast is the library reference, on edge values and on random
    values from subnormal to overflow range."""
    edge = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11), 6.1e-5, 1.0 + 2.0 ** -11,
            1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 1e-30, float("inf"), -float("inf")]
    rng = np.random.default_rng(5)
    rand = (rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 18, 20000))).astype(np.float32)
    for x in list(np.float32(edge)) + list(rand):
        with np.errstate(over="ignore"):   # overflow to infinity is one of the cases
            want = int(np.array([x], np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f32_to_f16_bits(x) == want, (x, hex(want))
        assert oracle.f16_bits_to_f32(want) == float(np.array([want], np.uint16).view(np.float16)[0].astype(np.float32))
    nan = oracle.f32_to_f16_bits(float("nan"))
    assert (nan & 0x7c00) == 0x7c00 and (nan & 0x3ff) != 0


@pytest.mark.parametrize("d", [128, 256, 512])
def test_f16_record_same_codes_rounded_scales_and_size(d):
    K, V = synth.make_kv(77 + d, 128, 1, d, 4)
    r32 = oracle.compress_tile(K[:, 0], V[:, 0])
    r16 = oracle.compress_tile(K[:, 0], V[:, 0], f16=True)
    assert r16.size == oracle.tile_bytes(d, True) == 106 * d + 256
    z32 = oracle.unpack_codes(r32, d)
    z16 = oracle.unpack_codes(r16, d)
    assert np.array_equal(z32[0], z16[0]) and np.array_equal(z32[1], z16[1])
    s32 = oracle.record_scales(r32, d)
    s16 = oracle.record_scales(r16, d, f16=True)
    for name in s32:
        assert np.array_equal(s32[name].astype(np.float16).astype(np.float32), s16[name]), name
    if d == 128:   # the pages' saving: 120 -> 108 bytes per token per KV head
        assert oracle.tile_bytes(128) // 128 == 120 and oracle.tile_bytes(128, True) // 128 == 108


def test_f16_record_dequant_within_half_rounding_of_f32_record():
    """k' = ktok (z kscale + kmin): each of the three stored factors moves by at
    most 2^-11 relative when rounded to f16, so every dequantised element moves
    by at most (1 + 2^-11)^2 - 1 relative to the sum of its term magnitudes."""
    d = 128
    K, V = synth.make_kv(88, 128, 1, d, 4)
    r32 = oracle.compress_tile(K[:, 0], V[:, 0])
    r16 = oracle.compress_tile(K[:, 0], V[:, 0], f16=True)
    k32, v32 = oracle.dequant_rotated(r32, d)
    k16, v16 = oracle.dequant_rotated(r16, d, f16=True)
    s = oracle.record_scales(r32, d)
    zK, zV = oracle.unpack_codes(r32, d)
    eps = (1 + 2.0 ** -11) ** 2 - 1 + 1e-12
    magk = np.abs(s["ktok"])[:, None] * (zK * np.abs(s["kscale"])[None] + np.abs(s["kmin"])[None])
    magv = np.abs(s["vchan"])[None] * (zV * np.abs(s["vscale"][:, :1]) + np.abs(s["vmin"][:, :1]))
    assert np.all(np.abs(k16 - k32) <= eps * magk)
    assert np.all(np.abs(v16 - v32) <= eps * magv)
    assert np.any(k16 != k32)


# --------------------------------------------------------------------------
# configurable key / value widths (gmlx PR #116 commit list: k6v5-style arms)
# --------------------------------------------------------------------------

WIDTHS = [(6, 5), (3, 1), (8, 8), (2, 3), (5, 4), (1, 7)]


@pytest.mark.parametrize("d", [128, 256, 512])
@pytest.mark.parametrize("f16", [False, True])
def test_bit_stream_packer_and_reader_agree_with_the_k4v2_nibble_code(d, f16):
    """At 4/2 bits the LSB-first bit stream is the nibble / crumb record: the
    bit-level writer and reader reproduce the hand-packed bytes and codes."""
    K, V = synth.make_kv(90 + d, 128, 1, d, 4)
    r = oracle.compress_tile(K[:, 0], V[:, 0], f16=f16)
    assert np.array_equal(oracle.compress_tile_bits(K[:, 0], V[:, 0], f16=f16), r)
    a, b = oracle.unpack_codes(r, d), oracle.unpack_codes_bits(r, d)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_width_record_sizes_closed_form():
    for d in (128, 256, 512):
        for kb in range(1, 9):
            for vb in range(1, 9):
                codes = 128 * d * (kb + vb) // 8
                assert oracle.tile_bytes(d, False, kb, vb) == codes + 4 * (128 + 5 * d)
                assert oracle.tile_bytes(d, True, kb, vb) == codes + 2 * (128 + 5 * d)
        assert oracle.tile_bytes(d, False, 0, 2) == 0 and oracle.tile_bytes(d, False, 4, 9) == 0
    assert oracle.tile_bytes(128, False, 4, 2) == 116 * 128 + 512


@pytest.mark.parametrize("kb,vb", WIDTHS)
def test_width_codes_are_little_endian_bit_streams(kb, vb):
    """Rebuild both code sections from the codes with Python integers: key
    channel c is sum_t zK[t][c] 2^(kb t), value token t is sum_c zV[t][c]
    2^(vb c), each stored little-endian."""
    d = 256
    K, V = synth.make_kv(7 * kb + vb, 128, 1, d, 4)
    rec = oracle.compress_tile(K[:, 0], V[:, 0], kbits=kb, vbits=vb)
    off = oracle.layout(d, False, kb, vb)
    zK, zV = oracle.unpack_codes(rec, d, kb, vb)
    for c in (0, 1, 77, d - 1):
        n = sum(int(zK[t, c]) << (kb * t) for t in range(128))
        want = n.to_bytes(16 * kb, "little")
        assert bytes(rec[off["kcode"] + 16 * kb * c: off["kcode"] + 16 * kb * (c + 1)]) == want
    for t in (0, 5, 127):
        n = sum(int(zV[t, c]) << (vb * c) for c in range(d))
        lo = off["vcode"] + t * d * vb // 8
        assert bytes(rec[lo: lo + d * vb // 8]) == n.to_bytes(d * vb // 8, "little")
    assert off["ktok"] == 16 * d * (kb + vb)


@pytest.mark.parametrize("kb,vb", WIDTHS)
def test_width_rtn_uses_every_level_and_stays_within_half_a_step(kb, vb):
    """RTN with 2^b - 1 levels: every key channel and value token group holds
    code 0 (its minimum) and code 2^b - 1 (its maximum); every dequantised
    element of the rotated tile is within half a step (r s delta / 2) of the
    rotated input."""
    d = 128
    K, V = synth.make_kv(11 * kb + vb, 128, 1, d, 4)
    rec = oracle.compress_tile(K[:, 0], V[:, 0], kbits=kb, vbits=vb)
    zK, zV = oracle.unpack_codes(rec, d, kb, vb)
    assert np.all(zK.min(axis=0) == 0) and np.all(zK.max(axis=0) == 2 ** kb - 1)
    assert np.all(zV.min(axis=1) == 0) and np.all(zV.max(axis=1) == 2 ** vb - 1)
    s = oracle.record_scales(rec, d, False, kb, vb)
    kd, vd = oracle.dequant_rotated(rec, d, False, kb, vb)
    Xk = oracle.wht_f32(K[:, 0]).astype(np.float64)
    Xv = oracle.wht_f32(V[:, 0]).astype(np.float64)
    stepk = s["ktok"][:, None].astype(np.float64) * s["kscale"][None].astype(np.float64)
    stepv = s["vchan"][None].astype(np.float64) * s["vscale"][:, :1].astype(np.float64)
    assert np.all(np.abs(kd - Xk) <= 0.5 * stepk * (1 + 1e-4) + 1e-6 * np.abs(Xk))
    assert np.all(np.abs(vd - Xv) <= 0.5 * stepv * (1 + 1e-4) + 1e-6 * np.abs(Xv))


def test_width_error_falls_with_every_added_bit():
    """Each extra bit roughly halves the step: the relative L2 error of the
    dequantised keys and values falls by more than 1.5x per bit."""
    d = 128
    K, V = synth.make_kv(123, 128, 1, d, 4)
    Xk = oracle.wht_f32(K[:, 0]).astype(np.float64)
    Xv = oracle.wht_f32(V[:, 0]).astype(np.float64)
    ek, ev = [], []
    for b in range(1, 9):
        rec = oracle.compress_tile(K[:, 0], V[:, 0], kbits=b, vbits=b)
        kd, vd = oracle.dequant_rotated(rec, d, False, b, b)
        ek.append(np.linalg.norm(kd - Xk) / np.linalg.norm(Xk))
        ev.append(np.linalg.norm(vd - Xv) / np.linalg.norm(Xv))
    for i in range(1, 8):
        assert ek[i] < ek[i - 1] / 1.5 and ev[i] < ev[i - 1] / 1.5, (i, ek, ev)
