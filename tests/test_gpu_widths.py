"""GPU parity of records with other code widths (gmlx PR #116 commit list:
mixed-width "k6v5"-style arms, key and value widths chosen on their own): the
compressor writes the oracle's bit-stream record byte for byte; decode and
prefill over those records (vector-unit kernels) stay within 1e-4 relative L2
of the fp64 oracle on the same dequantised cache."""
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


def gpu_compress(K, V, n_tiles, kb, vb, f16=False):
    d, n_kv = K.shape[2], K.shape[1]
    rec = torch.zeros(max(n_tiles, 1), n_kv, kvarn.tile_bytes(d, f16, kb, vb), dtype=torch.uint8,
                      device=DEV)
    kvarn.compress_tile(to_dev(K), to_dev(V), rec, n_tiles, f16_scales=f16, kbits=kb, vbits=vb)
    torch.cuda.synchronize()
    return rec[:n_tiles].cpu().numpy()


@pytest.mark.parametrize("d,kb,vb,f16", [(128, 6, 5, False), (128, 3, 1, False), (128, 8, 8, True),
                                         (256, 2, 3, False), (256, 5, 4, True), (512, 1, 7, False),
                                         (512, 8, 8, False), (512, 6, 5, True)])
def test_compress_widths_bytes_identical_with_degenerate_tiles(d, kb, vb, f16):
    say("compress widths", d, kb, vb, f16)
    n_kv, n_tiles = 2, 3
    K, V = synth.make_kv(1000 + d + 10 * kb + vb, 128 * n_tiles, n_kv, d, 4)
    K[:, 0, 5] = 0.0                        # all-zero channel
    V[128:256, 1, :] = 0.75                 # constant value tile
    K[256:384, 1, :] *= np.float32(1e-3)
    got = gpu_compress(K, V, n_tiles, kb, vb, f16)
    want = oracle.compress_tiles(K, V, n_tiles, f16=f16, kbits=kb, vbits=vb)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} bytes differ, first at {mism[:5].tolist()}"


@pytest.mark.parametrize("kb,vb,f16", [(6, 5, False), (3, 1, True)])
def test_decode_widths_8b_shape(kb, vb, f16):
    say("decode widths 8b 4096", kb, vb, f16)
    d, Hq, Hkv, W, ctx = 128, 32, 8, 256, 4096
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(3, ctx, Hkv, d, 2)
    q = synth.make_q(3, 1, Hq, d)
    recs = gpu_compress(K, V, T, kb, vb, f16)
    want = oracle.compress_tiles(K, V, T, f16=f16, kbits=kb, vbits=vb)
    assert np.array_equal(recs, want)          # every record byte-identical to the oracle's
    kh, vh = oracle.dequant_records(want, d, f16, kb, vb)
    scale = 1 / math.sqrt(d)
    qd = to_dev(q)
    qr, rd = kvarn.rotate_query(qd), to_dev(recs)
    kwd, vwd = to_dev(K[128 * T:][None]), to_dev(V[128 * T:][None])
    # NaN-filled workspace and output: every partial the combine reads must be written
    ws = nan_bytes(kvarn.decode_workspace_bytes(qd, qr, rd, [0], [T], kwd, vwd, [ctx - 128 * T], scale,
                                                f16_scales=f16, kbits=kb, vbits=vb))
    out = kvarn.decode_attention(qd, qr, rd, [0], [T], kwd, vwd, [ctx - 128 * T], scale, out=nan_like(qd),
                                 workspace=ws, f16_scales=f16, kbits=kb, vbits=vb)
    torch.cuda.synchronize()
    ref = oracle.decode(q[0], kh, vh, T, K[128 * T:], V[128 * T:], scale)
    err = rel_l2(out.cpu().numpy()[0], ref)
    say("rel_l2", err)
    assert err < TOL


@pytest.mark.parametrize("d,Hq,Hkv,kb,vb", [(256, 16, 4, 3, 1), (512, 8, 1, 8, 8), (128, 16, 2, 2, 3)])
def test_decode_widths_ragged_batch(d, Hq, Hkv, kb, vb):
    say("decode widths ragged", d, kb, vb)
    B = 3
    tiles, wins = [5, 1, 3], [200, 17, 256]
    cap = max(wins)
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    recs_all, rec_start, KV, row = [], [], [], 0
    for b in range(B):
        K, V = synth.make_kv(1100 + 7 * b + d, 128 * tiles[b] + wins[b], Hkv, d, 4)
        recs_all.append(gpu_compress(K, V, tiles[b], kb, vb))
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all)
    q = synth.make_q(1200 + d, B, Hq, d)
    qd = to_dev(q)
    scale = 1 / math.sqrt(d)
    out = kvarn.decode_attention(qd, kvarn.rotate_query(qd), to_dev(recs), rec_start, tiles,
                                 to_dev(kw), to_dev(vw), wins, scale, kbits=kb, vbits=vb)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        mine = recs[rec_start[b]:rec_start[b] + tiles[b]]
        assert np.array_equal(mine, oracle.compress_tiles(K, V, tiles[b], kbits=kb, vbits=vb))
        kh, vh = oracle.dequant_records(mine, d, False, kb, vb)
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        assert rel_l2(got[b], ref) < TOL, b


@pytest.mark.parametrize("d,Hq,Hkv,kb,vb,n", [(128, 8, 2, 6, 5, 900), (256, 8, 2, 2, 3, 600)])
def test_prefill_widths_every_row(d, Hq, Hkv, kb, vb, n):
    say("prefill widths", d, kb, vb, n)
    W = 256
    K, V = synth.make_kv(1300 + d, n, Hkv, d, 2)
    Q = synth.make_q(1300 + d, n, Hq, d)
    cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=DEV, kbits=kb, vbits=vb)
    scale = 1 / math.sqrt(d)
    outs = []
    for p0 in range(0, n, 256):
        c = min(256, n - p0)
        cache.append(to_dev(K[p0:p0 + c]), to_dev(V[p0:p0 + c]))
        qd = to_dev(Q[p0:p0 + c])
        raw_base = 128 * kvarn.visible_tiles(p0, W)
        outs.append(kvarn.prefill_attention(qd, kvarn.rotate_query(qd), cache.records, cache.n_tiles,
                                            cache.k[raw_base:], cache.v[raw_base:], raw_base, p0, W,
                                            scale, kbits=kb, vbits=vb))
    torch.cuda.synchronize()
    out = torch.cat(outs).cpu().numpy()
    recs = cache.records[:cache.n_tiles].cpu().numpy()
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0], kbits=kb, vbits=vb))
    kh, vh = oracle.dequant_records(recs, d, False, kb, vb)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, scale) for p in range(n)])
    err = rel_l2(out, ref)
    say("rel_l2", err)
    assert err < TOL


def test_verify_with_other_widths_is_rejected_before_launch():
    say("verify widths rejected")
    d, Hq, Hkv = 128, 8, 2
    q = torch.zeros(1, 2, Hq, d, device=DEV)
    rec = torch.zeros(1, Hkv, kvarn.tile_bytes(d, False, 6, 5), dtype=torch.uint8, device=DEV)
    kw = torch.zeros(1, 8, Hkv, d, device=DEV)
    with pytest.raises(kvarn.KVarNError) as e:
        kvarn.decode_attention(q, q, rec, [0], [1], kw, kw, [8], 0.1, kbits=6, vbits=5)
    assert e.value.status == 2
