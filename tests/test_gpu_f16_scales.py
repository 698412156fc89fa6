"""GPU parity of the record with f16 scales (SharpInference issue #433 item 3,
"f16 scales in the packed tile layout"): the compressor writes the same codes
as the fp32 record and each scale rounded to the nearest binary16, byte for
byte as the oracle does; decode, verify and prefill read that record and stay
within 1e-4 relative L2 of the fp64 oracle on the f16-scale dequantised
cache."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from poison import nan_bytes, nan_like
from quantized_attention_tok_amd import kvarn, synth
from quantized_attention_tok_amd.cache import SequenceCache

pytestmark = pytest.mark.gpu
TOL = 1e-4
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvarn.lib()
    yield
    torch.cuda.synchronize()


def gpu_compress16(K, V, n_tiles):
    d, n_kv = K.shape[2], K.shape[1]
    rec = torch.zeros(max(n_tiles, 1), n_kv, kvarn.tile_bytes(d, True), dtype=torch.uint8, device=DEV)
    kvarn.compress_tile(to_dev(K), to_dev(V), rec, n_tiles, f16_scales=True)
    torch.cuda.synchronize()
    return rec[:n_tiles].cpu().numpy()


@pytest.mark.parametrize("d,n_kv,n_tiles", [(128, 2, 4), (256, 2, 3), (512, 1, 3)])
def test_compress_f16_bytes_identical_with_degenerate_tiles(d, n_kv, n_tiles):
    say("compress f16", d, n_kv, n_tiles)
    K, V = synth.make_kv(500 + d, 128 * n_tiles, n_kv, d, 4)
    K[:, 0, 3] = 0.0                        # all-zero channel
    V[128:256, 0, :] = 1.5                  # constant value tile
    K[256:384, n_kv - 1, :] *= np.float32(1e-6)   # scales in the f16 subnormal range
    V[256:384, n_kv - 1, :] *= np.float32(1e4)    # scales near the top of the f16 range
    got = gpu_compress16(K, V, n_tiles)
    want = oracle.compress_tiles(K, V, n_tiles, f16=True)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} bytes differ, first at {mism[:5].tolist()}"
    # the codes are those of the fp32 record
    lay16, lay32 = oracle.layout(d, True), oracle.layout(d)
    ref32 = oracle.compress_tiles(K, V, n_tiles)
    assert np.array_equal(got[..., :lay16["ktok"]], ref32[..., :lay32["ktok"]])


def test_decode_f16_8b_shape_and_cache_size():
    say("decode f16 8b 15488")
    d, Hq, Hkv, W, ctx = 128, 32, 8, 256, 15488
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(2, ctx, Hkv, d, 2)
    q = synth.make_q(2, 1, Hq, d)
    recs = gpu_compress16(K, V, T)
    assert recs.shape[-1] == 13824
    want = oracle.compress_tiles(K, V, T, f16=True)
    assert np.array_equal(recs, want)          # every record byte-identical to the oracle's
    kh, vh = oracle.dequant_records(want, d, f16=True)
    scale = 1 / math.sqrt(d)
    qd = to_dev(q)
    for q_rot in (kvarn.rotate_query(qd), None):   # both query paths of the matrix-core decode
        out = kvarn.decode_attention(qd, q_rot, to_dev(recs), [0], [T], to_dev(K[128 * T:][None]),
                                     to_dev(V[128 * T:][None]), [ctx - 128 * T], scale,
                                     f16_scales=True)
        torch.cuda.synchronize()
        ref = oracle.decode(q[0], kh, vh, T, K[128 * T:], V[128 * T:], scale)
        err = rel_l2(out.cpu().numpy()[0], ref)
        say("rel_l2", err)
        assert err < TOL


@pytest.mark.parametrize("d,Hq,Hkv", [(256, 16, 4), (512, 8, 1)])
def test_decode_f16_wide_heads_ragged_batch(d, Hq, Hkv):
    say("decode f16 ragged", d)
    B, W = 4, 256
    rng = np.random.default_rng(600 + d)
    tiles = [int(x) for x in rng.integers(1, 9, size=B)]
    wins = [int(x) for x in rng.integers(W, W + 128, size=B)]
    cap = max(wins)
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    recs_all, rec_start, KV, row = [], [], [], 0
    for b in range(B):
        K, V = synth.make_kv(610 + 3 * b + d, 128 * tiles[b] + wins[b], Hkv, d, 4)
        recs_all.append(gpu_compress16(K, V, tiles[b]))
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all)
    q = synth.make_q(620 + d, B, Hq, d)
    qd = to_dev(q)
    scale = 1 / math.sqrt(d)
    out = kvarn.decode_attention(qd, kvarn.rotate_query(qd), to_dev(recs), rec_start, tiles,
                                 to_dev(kw), to_dev(vw), wins, scale, f16_scales=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        mine = recs[rec_start[b]:rec_start[b] + tiles[b]]
        assert np.array_equal(mine, oracle.compress_tiles(K, V, tiles[b], f16=True))
        kh, vh = oracle.dequant_records(mine, d, f16=True)
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        err = rel_l2(got[b], ref)
        assert err < TOL, (b, err)


def test_verify_f16_ragged_batch():
    say("verify f16 ragged")
    d, B, Hq, Hkv, w = 128, 3, 16, 4, 6
    tiles, wins = [4, 0, 2], [50, w, 17]
    recs_all, rec_start, KV, row = [], [], [], 0
    cap = max(wins)
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    for b in range(B):
        K, V = synth.make_kv(700 + 5 * b, 128 * tiles[b] + wins[b], Hkv, d, 2)
        if tiles[b]:
            recs_all.append(gpu_compress16(K, V, tiles[b]))
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all)
    q = synth.make_q(710, B * w, Hq, d).reshape(B, w, Hq, d)
    scale = 1 / math.sqrt(d)
    out = kvarn.decode_attention(to_dev(q), None, to_dev(recs), rec_start, tiles, to_dev(kw),
                                 to_dev(vw), wins, scale, f16_scales=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        if tiles[b]:
            mine = recs[rec_start[b]:rec_start[b] + tiles[b]]
            assert np.array_equal(mine, oracle.compress_tiles(K, V, tiles[b], f16=True))
            kh, vh = oracle.dequant_records(mine, d, f16=True)
        else:
            kh = vh = np.zeros((0, Hkv, d))
        lo = 128 * tiles[b]
        ref = oracle.verify(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        for i in range(w):
            err = rel_l2(got[b, i], ref[i])
            assert err < TOL, (b, i, err)


def _prefill16(K, V, Q, W, chunk, Hkv, d, poison=False):
    n = K.shape[0]
    cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=DEV, f16_scales=True)
    outs = []
    scale = 1 / math.sqrt(d)
    for p0 in range(0, n, chunk):
        c = min(chunk, n - p0)
        cache.append(to_dev(K[p0:p0 + c]), to_dev(V[p0:p0 + c]))
        qd = to_dev(Q[p0:p0 + c])
        qr = kvarn.rotate_query(qd)
        raw_base = 128 * kvarn.visible_tiles(p0, W)
        extra = {}
        if poison:   # NaN-filled output and workspace
            nb = kvarn.prefill_workspace_bytes(qd, qr, cache.records, cache.n_tiles, cache.k[raw_base:],
                                               cache.v[raw_base:], raw_base, p0, W, scale, f16_scales=True)
            extra = {"out": nan_like(qd), "workspace": nan_bytes(nb)}
        outs.append(kvarn.prefill_attention(qd, qr, cache.records, cache.n_tiles,
                                            cache.k[raw_base:], cache.v[raw_base:], raw_base, p0, W,
                                            scale, f16_scales=True, **extra))
    torch.cuda.synchronize()
    return torch.cat(outs).cpu().numpy(), cache.records[:cache.n_tiles].cpu().numpy()


@pytest.mark.parametrize("d,Hq,Hkv,n", [(128, 8, 2, 1100), (256, 16, 4, 700), (512, 8, 1, 500)])
def test_prefill_f16_every_row(d, Hq, Hkv, n):
    say("prefill f16", d, n)
    W = 256
    K, V = synth.make_kv(800 + d, n, Hkv, d, 2)
    Q = synth.make_q(800 + d, n, Hq, d)
    out, recs = _prefill16(K, V, Q, W, 256, Hkv, d)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0], f16=True))
    kh, vh = oracle.dequant_records(recs, d, f16=True)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in range(n)])
    err = rel_l2(out, ref)
    say("rel_l2", err)
    assert err < TOL
    # an odd chunk (odd row counts in every chunk and the tail), NaN-filled buffers
    out2, recs2 = _prefill16(K, V, Q, W, 77, Hkv, d, poison=True)
    assert np.array_equal(recs2, recs)
    err2 = rel_l2(out2, ref)
    say("odd chunk rel_l2", err2, "vs chunk 256", rel_l2(out2, out))
    assert err2 < TOL and rel_l2(out2, out) < 1e-5
