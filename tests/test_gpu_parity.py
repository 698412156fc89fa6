"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Records must be byte-identical; attention must be within
1e-4 relative L2 of the fp64 oracle on the dequantised cache."""
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


def gpu_compress(K, V, n_tiles):
    d, n_kv = K.shape[2], K.shape[1]
    rec = torch.zeros(max(n_tiles, 1), n_kv, kvarn.tile_bytes(d), dtype=torch.uint8, device=DEV)
    kvarn.compress_tile(to_dev(K), to_dev(V), rec, n_tiles)
    torch.cuda.synchronize()
    return rec[:n_tiles].cpu().numpy()


# --------------------------------------------------------------------------
# compression: byte parity
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d,n_kv,n_tiles,n_out", [(128, 1, 4, 4), (128, 8, 6, 2), (256, 4, 3, 4),
                                                  (512, 1, 3, 4), (512, 2, 2, 4)])
def test_compress_bytes_identical(d, n_kv, n_tiles, n_out):
    say("compress", d, n_kv, n_tiles)
    K, V = synth.make_kv(100 + d + n_kv, 128 * n_tiles, n_kv, d, n_out)
    got = gpu_compress(K, V, n_tiles)
    want = oracle.compress_tiles(K, V, n_tiles)
    mism = np.argwhere(got != want)
    assert mism.size == 0, f"{len(mism)} bytes differ, first at {mism[:5].tolist()}"


def test_compress_strided_input_and_degenerate_tiles():
    say("compress degenerate")
    d, n_kv = 128, 2
    K, V = synth.make_kv(7, 128 * 4, n_kv, d, 4)
    K[:, 0, 5] = 0.0                        # all-zero channel in head 0
    K[128 + 17, 1, :] = 0.0                 # all-zero token
    V[256:384, 0, :] = 1.5                  # constant tile
    K[384:512, 1, :] *= np.float32(1e-30)   # tiny (subnormal squares)
    V[384:512, 1, ::3] = 0.0
    # strided: heads interleaved with a padding head
    Kp = np.zeros((128 * 4, n_kv + 1, d), np.float32); Kp[:, :n_kv] = K
    Vp = np.zeros((128 * 4, n_kv + 1, d), np.float32); Vp[:, :n_kv] = V
    rec = torch.zeros(4, n_kv, kvarn.tile_bytes(d), dtype=torch.uint8, device=DEV)
    kd, vd = to_dev(Kp), to_dev(Vp)
    kvarn.compress_tile(kd[:, :n_kv], vd[:, :n_kv], rec, 4)
    torch.cuda.synchronize()
    want = oracle.compress_tiles(K, V, 4)
    assert np.array_equal(rec.cpu().numpy(), want)


def test_compress_prefill_prompt_all_tiles():
    # the full 8B-shaped prompt: 119 tiles x 8 KV heads = 952 records
    say("compress 952 records")
    K, V = synth.make_kv(4, 15488, 8, 128, 2)
    got = gpu_compress(K, V, 119)
    want = oracle.compress_tiles(K, V, 119)
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# query rotation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [128, 256, 512])
def test_rotate_query_matches_oracle_transform(d):
    say("rotate", d)
    q = synth.make_q(d, 37, 3, d)
    got = kvarn.rotate_query(to_dev(q))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.wht_f32(q))


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------

def run_decode(q, recs, n_tiles, kw, vw, scale, poison=False, **kw_args):
    """q [B][Hq][d]; recs [rows][Hkv][bytes] (numpy); kw/vw [B][cap][Hkv][d].
    poison: the workspace and the output start as NaN."""
    qd = to_dev(q)
    qr = kvarn.rotate_query(qd)
    rd = to_dev(recs) if recs is not None and recs.size else None
    rec_start, n_win = kw_args.pop("rec_start"), kw_args.pop("n_win")
    kwd, vwd = to_dev(kw), to_dev(vw)
    if poison:
        nb = kvarn.decode_workspace_bytes(qd, qr, rd, rec_start, n_tiles, kwd, vwd, n_win, scale,
                                          max_tiles=kw_args.get("max_tiles"),
                                          max_win=kw_args.get("max_win"))
        assert nb > 0
        kw_args["workspace"] = nan_bytes(nb)
        kw_args["out"] = nan_like(qd)
    out = kvarn.decode_attention(qd, qr, rd, rec_start, n_tiles, kwd, vwd, n_win, scale, **kw_args)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_decode_tiny_tiles_only():
    say("decode tiny")
    d = 128
    K, V = synth.make_kv(0, 512, 1, d, 4)
    q = synth.make_q(0, 1, 1, d)
    recs = gpu_compress(K, V, 4)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, 4))
    kh, vh = oracle.dequant_records(recs, d)
    empty = np.zeros((1, 1, 1, d), np.float32)
    got = run_decode(q, recs, [4], empty, empty, 1 / math.sqrt(d), rec_start=[0], n_win=[0])
    ref = oracle.decode(q[0], kh, vh, 4, np.zeros((0, 1, d)), np.zeros((0, 1, d)), 1 / math.sqrt(d))
    assert rel_l2(got[0], ref) < TOL


@pytest.mark.parametrize("ctx", [4096, 15488, 32768])
def test_decode_8b_shape(ctx):
    say("decode 8b", ctx)
    d, Hq, Hkv, W = 128, 32, 8, 256
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(2, ctx, Hkv, d, 2)
    q = synth.make_q(2, 1, Hq, d)
    recs = gpu_compress(K, V, T)
    want = oracle.compress_tiles(K, V, T)
    assert np.array_equal(recs, want)          # every record byte-identical to the oracle's
    kh, vh = oracle.dequant_records(want, d)
    kw = K[128 * T:][None]
    vw = V[128 * T:][None]
    scale = 1 / math.sqrt(d)
    got = run_decode(q, recs, [T], kw, vw, scale, poison=True, rec_start=[0], n_win=[ctx - 128 * T])
    ref = oracle.decode(q[0], kh, vh, T, K[128 * T:], V[128 * T:], scale)
    err = rel_l2(got[0], ref)
    say("rel_l2", err)
    assert err < TOL


def test_decode_qwen06b_64_steps_with_appends():
    say("decode 0.6b steps")
    d, Hq, Hkv, W = 128, 16, 8, 256
    steps = 64
    n0 = 3072 + 256
    K, V = synth.make_kv(1, n0 + steps, Hkv, d, 4)
    Q = synth.make_q(1, steps, Hq, d)
    cache = SequenceCache(Hkv, d, W, capacity=n0 + steps + 128, device=DEV)
    cache.append(to_dev(K[:n0]), to_dev(V[:n0]))
    assert cache.n_tiles == 24 and cache.n_win == 256
    recs_all = cache.records[:24].cpu().numpy()
    assert np.array_equal(recs_all, oracle.compress_tiles(K, V, 24))
    kh, vh = oracle.dequant_records(recs_all, d)
    scale = 1 / math.sqrt(d)
    worst = 0.0
    for s in range(steps):
        cache.append(to_dev(K[n0 + s:n0 + s + 1]), to_dev(V[n0 + s:n0 + s + 1]))
        qd = to_dev(Q[s:s + 1])
        qr = kvarn.rotate_query(qd)
        out = kvarn.decode_attention(qd, qr, cache.records, [0], [cache.n_tiles],
                                     cache.k[None], cache.v[None], [cache.n_win], scale,
                                     win_start=[128 * cache.n_tiles])
        if s % 9 == 0 or s == steps - 1:
            lo = 128 * cache.n_tiles
            ref = oracle.decode(Q[s], kh, vh, cache.n_tiles, K[lo:n0 + s + 1], V[lo:n0 + s + 1], scale)
            worst = max(worst, rel_l2(out[0].cpu().numpy(), ref))
    assert cache.n_tiles == 24
    assert worst < TOL


@pytest.mark.parametrize("d,Hq,Hkv", [(256, 16, 4), (512, 8, 1)])
def test_decode_ragged_batch_with_promotions(d, Hq, Hkv):
    say("decode ragged", d)
    B, W = 6, 256
    rng = np.random.default_rng(d)
    tiles0 = rng.integers(1, 12, size=B)          # small contexts keep the oracle quick
    caches, KV = [], []
    for b in range(B):
        n = int(128 * tiles0[b] + W + rng.integers(0, 128))
        K, V = synth.make_kv(300 + 10 * b + d, n + 140, Hkv, d, 4)
        c = SequenceCache(Hkv, d, W, capacity=n + 300, device=DEV)
        c.append(to_dev(K[:n]), to_dev(V[:n]))
        caches.append(c)
        KV.append((K, V, n))
    scale = 1 / math.sqrt(d)
    # one shared record pool and window buffer, as the ABI takes them
    steps = 140
    for s in range(steps):
        for b in range(B):
            K, V, n = KV[b]
            caches[b].append(to_dev(K[n + s:n + s + 1]), to_dev(V[n + s:n + s + 1]))
        if s not in (0, 70, steps - 1):
            continue
        rows = max(c.n_tiles for c in caches)
        pool = torch.zeros(B * rows, Hkv, kvarn.tile_bytes(d), dtype=torch.uint8, device=DEV)
        cap = max(c.n_win for c in caches)
        kw = torch.zeros(B, cap, Hkv, d, device=DEV)
        vw = torch.zeros_like(kw)
        for b, c in enumerate(caches):
            pool[b * rows:b * rows + c.n_tiles] = c.records[:c.n_tiles]
            k_, v_ = c.window_views()
            kw[b, :c.n_win] = k_
            vw[b, :c.n_win] = v_
        q = synth.make_q(d + s, B, Hq, d)
        qd = to_dev(q)
        qr = kvarn.rotate_query(qd)
        rs, nts, nws = [b * rows for b in range(B)], [c.n_tiles for c in caches], [c.n_win for c in caches]
        ws = nan_bytes(kvarn.decode_workspace_bytes(qd, qr, pool, rs, nts, kw, vw, nws, scale))
        out = kvarn.decode_attention(qd, qr, pool, rs, nts, kw, vw, nws, scale, out=nan_like(qd), workspace=ws)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        errs = []
        for b, c in enumerate(caches):
            K, V, n = KV[b]
            recs = c.records[:c.n_tiles].cpu().numpy()
            assert np.array_equal(recs, oracle.compress_tiles(K, V, c.n_tiles))
            kh, vh = oracle.dequant_records(recs, d)
            lo = 128 * c.n_tiles
            ref = oracle.decode(q[b], kh, vh, c.n_tiles, K[lo:n + s + 1], V[lo:n + s + 1], scale)
            errs.append(rel_l2(out[b], ref))
        say("step", s, "max rel_l2", max(errs))
        assert max(errs) < TOL
    assert all(c.n_tiles > t for c, t in zip(caches, tiles0))   # every sequence promoted


def test_decode_split_plan_invariance_and_determinism():
    say("decode splits")
    d, Hq, Hkv, W = 128, 32, 8, 256
    ctx = 8192
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(9, ctx, Hkv, d, 2)
    q = synth.make_q(9, 1, Hq, d)
    recs = gpu_compress(K, V, T)
    kw, vw = K[128 * T:][None], V[128 * T:][None]
    want = oracle.compress_tiles(K, V, T)
    assert np.array_equal(recs, want)
    kh, vh = oracle.dequant_records(want, d)
    ref = oracle.decode(q[0], kh, vh, T, K[128 * T:], V[128 * T:], 0.1)
    outs = []
    for max_tiles in (T, T + 5, 4 * T):
        outs.append(run_decode(q, recs, [T], kw, vw, 0.1, poison=True, rec_start=[0],
                               n_win=[ctx - 128 * T], max_tiles=max_tiles, max_win=ctx - 128 * T + 70))
    # Every plan against the fp64 oracle at the attention bar.
    errs = [rel_l2(o[0], ref) for o in outs]
    # Plans differ only in how many split partials there are and in the order
    # the combine folds them (the same fp32 terms summed in another order):
    # any split count gives the same result within 1e-6.
    diffs = [rel_l2(outs[i], outs[0]) for i in (1, 2)]
    say("plans vs oracle", errs, "plan vs plan", diffs)
    assert max(errs) < TOL
    assert max(diffs) < 1e-6
    again = run_decode(q, recs, [T], kw, vw, 0.1, poison=True, rec_start=[0], n_win=[ctx - 128 * T],
                       max_tiles=T + 5, max_win=ctx - 128 * T + 70)
    assert np.array_equal(again, outs[1])


# --------------------------------------------------------------------------
# chunked prefill
# --------------------------------------------------------------------------

def prefill_run(K, V, Q, W, chunk, Hkv, d, rotate=True, poison=False, no_ws=False):
    """Feed the prompt in chunks: compress due tiles, rotate (or leave the
    rotation to the kernel), attend.  poison: every chunk's output (and
    workspace, where the call takes one) starts as NaN.  no_ws: no workspace
    (head_dim 128: the single-launch kernel)."""
    n = K.shape[0]
    cache = SequenceCache(Hkv, d, W, capacity=n + 128, device=DEV)
    outs = []
    scale = 1 / math.sqrt(d)
    for p0 in range(0, n, chunk):
        c = min(chunk, n - p0)
        cache.append(to_dev(K[p0:p0 + c]), to_dev(V[p0:p0 + c]))
        qd = to_dev(Q[p0:p0 + c])
        qr = kvarn.rotate_query(qd) if rotate else None
        t_first = kvarn.visible_tiles(p0, W)
        raw_base = 128 * t_first
        extra = {"no_workspace": True} if no_ws else {}
        if poison:
            nb = kvarn.prefill_workspace_bytes(qd, qr, cache.records, cache.n_tiles, cache.k[raw_base:],
                                               cache.v[raw_base:], raw_base, p0, W, scale)
            extra.update({"out": nan_like(qd)} if no_ws else {"out": nan_like(qd), "workspace": nan_bytes(nb)})
        o = kvarn.prefill_attention(qd, qr, cache.records, cache.n_tiles, cache.k[raw_base:],
                                    cache.v[raw_base:], raw_base, p0, W, scale, **extra)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.cat(outs).cpu().numpy(), cache.records[:cache.n_tiles].cpu().numpy()


def test_prefill_small_prompt_every_row():
    say("prefill small")
    d, Hq, Hkv, W = 128, 8, 2, 256
    n = 1100
    K, V = synth.make_kv(21, n, Hkv, d, 2)
    Q = synth.make_q(21, n, Hq, d)
    out, recs = prefill_run(K, V, Q, W, 256, Hkv, d, poison=True)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0]))
    kh, vh = oracle.dequant_records(recs, d)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in range(n)])
    assert rel_l2(out, ref) < TOL
    # without a workspace: the single-launch kernel (half-tile waves, no splits).
    # Every score is the same to the bit; the two differ in the running maximum
    # each partial's value weights w = p vscale are taken against before their
    # fp16 hi / lo split (about 2^-22 relative each) and in the fp32 merge order
    out1, _ = prefill_run(K, V, Q, W, 256, Hkv, d, poison=True, no_ws=True)
    err1 = rel_l2(out1, ref)
    say("split vs single launch", rel_l2(out1, out), "single vs oracle", err1)
    assert err1 < TOL
    assert rel_l2(out1, out) < 5e-6


@pytest.mark.parametrize("W,chunk,Hq,Hkv,n,rotate", [(0, 100, 8, 8, 620, True), (1, 17, 4, 2, 300, False),
                                                     (100, 333, 16, 2, 800, True), (384, 1, 8, 1, 410, False),
                                                     (128, 1000, 8, 4, 700, False),
                                                     # 288-row chunks at 32/8 heads: 72 workgroups, 3 shares
                                                     (256, 288, 32, 8, 600, False)])
def test_prefill_windows_ragged_chunks_and_gqa_every_row(W, chunk, Hq, Hkv, n, rotate):
    """Windows 0, 1 and not a multiple of 128, chunks that cut 16-row column
    blocks and tiles anywhere (down to one row, up to the whole prompt), and
    query/KV head ratios 1, 2, 4 and 8 on the head_dim-128 matrix-core kernel
    (4 shares, and 3 at 288-row chunks of 32/8 heads; the 15488-token test
    covers 1 and 2); with the rotated query given or rotated inside the
    kernel."""
    say("prefill window/chunk/gqa", W, chunk, Hq, Hkv, n, rotate)
    d = 128
    K, V = synth.make_kv(60 + W + chunk, n, Hkv, d, 2)
    Q = synth.make_q(60 + W + chunk, n, Hq, d)
    out, recs = prefill_run(K, V, Q, W, chunk, Hkv, d, rotate)
    assert recs.shape[0] == oracle.visible_tiles(n - 1, W)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0]))
    kh, vh = oracle.dequant_records(recs, d)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in range(n)])
    err = rel_l2(out, ref)
    say("rel_l2", err)
    assert err < TOL


def test_prefill_raw_magnitude_jumps_every_row():
    """Raw window rows whose magnitude jumps by orders of magnitude between and
    inside 64-token staging steps, a query block far from unit scale, and the
    same rows later inside compressed tiles: every row within the bar on its own."""
    say("prefill raw magnitudes")
    d, Hq, Hkv, W = 128, 8, 2, 256
    n = 900
    K, V = synth.make_kv(23, n, Hkv, d, 2)
    Q = synth.make_q(23, n, Hq, d)
    V[520:584] *= np.float32(1e4)
    V[600:630, 1] *= np.float32(1e-3)
    K[650:700] *= np.float32(1e-3)
    K[700:740, 0] *= np.float32(6.0)
    V[760:800] *= np.float32(3e5)
    Q[820:880] *= np.float32(40.0)
    out, recs = prefill_run(K, V, Q, W, 256, Hkv, d)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0]))
    kh, vh = oracle.dequant_records(recs, d)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in range(n)])
    num = np.linalg.norm((out.astype(np.float64) - ref).reshape(n, -1), axis=1)
    rel = num / np.linalg.norm(ref.reshape(n, -1), axis=1)
    say("per-row rel rms", float(np.sqrt(np.mean(rel ** 2))), "max", float(rel.max()))
    assert np.sqrt(np.mean(rel ** 2)) < TOL and rel.max() < 10 * TOL



@pytest.mark.parametrize("d,Hq,Hkv", [(256, 16, 4), (512, 8, 1), (256, 4, 4), (512, 4, 2), (256, 16, 2), (256, 8, 4)])
def test_prefill_wide_heads_every_row_and_rechunk(d, Hq, Hkv):
    say("prefill wide", d)
    W, n = 256, 700
    K, V = synth.make_kv(40 + d, n, Hkv, d, 4)
    Q = synth.make_q(40 + d, n, Hq, d)
    out, recs = prefill_run(K, V, Q, W, 256, Hkv, d)
    assert np.array_equal(recs, oracle.compress_tiles(K, V, recs.shape[0]))
    kh, vh = oracle.dequant_records(recs, d)
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in range(n)])
    err = rel_l2(out, ref)
    say("rel_l2", err)
    assert err < TOL
    # another chunking (and queries rotated inside the kernels): the same tiles,
    # rows within the split-plan rounding of each other
    out2, recs2 = prefill_run(K, V, Q, W, 128, Hkv, d, rotate=False)
    assert np.array_equal(recs2, recs)
    assert rel_l2(out2, out) < 1e-5
    # an odd chunk (77 rows, so chunks and the tail have odd row counts: the
    # one-row-per-workgroup tile kernel) with NaN-filled outputs and workspaces
    out3, recs3 = prefill_run(K, V, Q, W, 77, Hkv, d, rotate=False, poison=True)
    assert np.array_equal(recs3, recs)
    err3 = rel_l2(out3, ref)
    say("odd chunk rel_l2", err3, "vs even chunk", rel_l2(out3, out))
    assert err3 < TOL
    assert rel_l2(out3, out) < 1e-5

def test_prefill_8b_prompt_sampled_rows_and_rechunk_identity():
    say("prefill 8b")
    d, Hq, Hkv, W = 128, 32, 8, 256
    n = 15488
    K, V = synth.make_kv(4, n, Hkv, d, 2)
    Q = synth.make_q(4, n, Hq, d)
    out512, recs512 = prefill_run(K, V, Q, W, 512, Hkv, d)
    assert recs512.shape[0] == 119
    for chunk in (256, 1024):
        out_c, recs_c = prefill_run(K, V, Q, W, chunk, Hkv, d)
        assert np.array_equal(recs_c, recs512)          # tiles are schedule-independent
        # the chunk size sets the split plan (4, 2, 1 tile-and-raw shares at 256,
        # 512, 1024 rows): each share's running maximum, fp16 hi / lo value weights
        # and fp32 sums over up to 121 tiles; within 5e-6 (measured 2.1e-6)
        say("chunk", chunk, "vs 512", rel_l2(out_c, out512))
        assert rel_l2(out_c, out512) < 5e-6
    # the bench's form: the kernel rotates the query rows itself, with the rounding
    # of the separate rotation, so the output is the same to the bit
    out_k, _ = prefill_run(K, V, Q, W, 512, Hkv, d, rotate=False)
    assert np.array_equal(out_k, out512)
    want = oracle.compress_tiles(K, V, 119)
    assert np.array_equal(recs512, want)       # every record byte-identical to the oracle's
    kh, vh = oracle.dequant_records(want, d)
    rows = sorted(set(list(range(0, 1024, 37)) + [383, 384, 511, 512, 639, 640, 8191, 8192, n - 1]
                      + list(range(0, n, 61))[:60]))
    ref = np.stack([oracle.prefill_row(Q[p], p, W, kh, vh, K, V, 1 / math.sqrt(d)) for p in rows])
    err = rel_l2(out512[rows], ref)
    say("prefill sampled rel_l2", err)
    assert err < TOL



# --------------------------------------------------------------------------
# multi-query verify: q_len rows per sequence, row i sees window [0, n_w - w + i]
# --------------------------------------------------------------------------

def _verify_batch(seed, B, Hq, Hkv, tiles, wins, w):
    d = 128
    recs_all, rec_start, KV = [], [], []
    cap = max(wins)
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros((B, cap, Hkv, d), np.float32)
    row = 0
    for b in range(B):
        K, V = synth.make_kv(seed + 7 * b, 128 * tiles[b] + wins[b], Hkv, d, 2)
        if tiles[b]:
            recs_all.append(oracle.compress_tiles(K, V, tiles[b]))
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all) if recs_all else np.zeros((0, Hkv, kvarn.tile_bytes(d)), np.uint8)
    q = synth.make_q(seed, B * w, Hq, d).reshape(B, w, Hq, d)
    return recs, rec_start, kw, vw, KV, q


@pytest.mark.parametrize("Hq,Hkv,w,with_rot", [(16, 8, 2, True), (8, 2, 5, False), (16, 2, 8, True),
                                                (4, 4, 8, False)])
def test_decode_multi_query_verify_ragged_batch(Hq, Hkv, w, with_rot):
    say("verify ragged", Hq, Hkv, w, with_rot)
    d, B = 128, 3
    tiles = [3, 0, 1]
    wins = [40, w, 23]   # the second sequence: no tiles and only the drafts
    recs, rec_start, kw, vw, KV, q = _verify_batch(900 + w, B, Hq, Hkv, tiles, wins, w)
    scale = 1 / math.sqrt(d)
    qd = to_dev(q)
    qr = kvarn.rotate_query(qd) if with_rot else None
    rd = to_dev(recs) if recs.size else None
    kwd, vwd = to_dev(kw), to_dev(vw)
    ws = nan_bytes(kvarn.decode_workspace_bytes(qd, qr, rd, rec_start, tiles, kwd, vwd, wins, scale))
    out = kvarn.decode_attention(qd, qr, rd, rec_start, tiles, kwd, vwd, wins, scale, out=nan_like(qd),
                                 workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        if tiles[b]:
            kh, vh = oracle.dequant_records(recs[rec_start[b]:rec_start[b] + tiles[b]], d)
        else:
            kh = vh = np.zeros((0, Hkv, d))
        lo = 128 * tiles[b]
        ref = oracle.verify(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        for i in range(w):
            err = rel_l2(got[b, i], ref[i])
            assert err < TOL, (b, i, err)


def test_decode_multi_query_verify_8b_shape():
    say("verify 8b 15488 w8")
    d, Hq, Hkv, W, ctx, w = 128, 32, 8, 256, 15488, 8
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(4, ctx, Hkv, d, 2)
    q = synth.make_q(4, w, Hq, d)[None]
    recs = gpu_compress(K, V, T)
    want = oracle.compress_tiles(K, V, T)
    assert np.array_equal(recs, want)
    kh, vh = oracle.dequant_records(want, d)
    n_w = ctx - 128 * T
    scale = 1 / math.sqrt(d)
    qd, rd = to_dev(q), to_dev(recs)
    kwd, vwd = to_dev(K[128 * T:][None]), to_dev(V[128 * T:][None])
    ws = nan_bytes(kvarn.decode_workspace_bytes(qd, None, rd, [0], [T], kwd, vwd, [n_w], scale))
    out = kvarn.decode_attention(qd, None, rd, [0], [T], kwd, vwd, [n_w], scale, out=nan_like(qd), workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[0]
    ref = oracle.verify(q[0], kh, vh, T, K[128 * T:], V[128 * T:], scale)
    err = max(rel_l2(got[i], ref[i]) for i in range(w))
    say("rel_l2", err)
    assert err < TOL
    # the last verify row is the ordinary decode query of the full window
    one = run_decode(q[0, w - 1:w], recs, [T], K[128 * T:][None], V[128 * T:][None], scale,
                     rec_start=[0], n_win=[n_w])
    assert rel_l2(one[0], got[w - 1]) < 2 * TOL

def test_decode_inkernel_rotation_and_workspace_reuse():
    say("decode q_rot=None, reused workspace")
    d, Hq, Hkv, W = 128, 32, 8, 256
    ctx = 2048 + 256 + 77
    T = oracle.visible_tiles(ctx - 1, W)
    K, V = synth.make_kv(31, ctx, Hkv, d, 2)
    recs = gpu_compress(K, V, T)
    want = oracle.compress_tiles(K, V, T)
    assert np.array_equal(recs, want)
    kh, vh = oracle.dequant_records(want, d)
    qd_all = synth.make_q(31, 3, Hq, d)
    kw = to_dev(K[128 * T:][None]); vw = to_dev(V[128 * T:][None]); rd = to_dev(recs)
    nb = kvarn.decode_workspace_bytes(to_dev(qd_all[:1]), None, rd, [0], [T], kw, vw, [ctx - 128 * T], 0.1)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    outs = []
    for r in range(3):
        qd = to_dev(qd_all[r:r + 1])
        outs.append(kvarn.decode_attention(qd, None, rd, [0], [T], kw, vw, [ctx - 128 * T], 0.1,
                                           workspace=ws))
    torch.cuda.synchronize()
    for r in range(3):
        ref = oracle.decode(qd_all[r], kh, vh, T, K[128 * T:], V[128 * T:], 0.1)
        assert rel_l2(outs[r][0].cpu().numpy(), ref) < TOL
    # with an explicit rotated query the result is the same to rounding
    qd = to_dev(qd_all[:1])
    o2 = kvarn.decode_attention(qd, kvarn.rotate_query(qd), rd, [0], [T], kw, vw, [ctx - 128 * T], 0.1,
                                workspace=ws)
    torch.cuda.synchronize()
    assert rel_l2(o2[0].cpu().numpy(), outs[0][0].cpu().numpy()) < 1e-6


@pytest.mark.parametrize("with_rot", [True, False])
def test_decode_batch_at_the_limit_mixed_views(with_rot):
    """KVARN_MAX_BATCH = 64 sequences in one call (the per-sequence argument
    arrays at their size): tile-only, window-only and mixed sequences, records
    from a shared pool at scattered rows, windows at per-sequence offsets."""
    say("decode batch 64", with_rot)
    d, Hq, Hkv, B = 128, 8, 2, 64
    rng = np.random.default_rng(64)
    tiles = [int(x) for x in rng.integers(0, 4, size=B)]
    wins = [int(x) for x in rng.integers(0, 41, size=B)]
    for b in range(B):
        if tiles[b] + wins[b] == 0:
            wins[b] = 1
    tiles[0], wins[0] = 3, 0      # tiles only
    tiles[1], wins[1] = 0, 33     # window only
    recs_all, rec_start, KV = [], [], []
    row = 5                        # the pool starts with unused rows
    pool = [np.zeros((5, Hkv, kvarn.tile_bytes(d)), np.uint8)]
    cap = max(wins) + 7
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    win_start = []
    for b in range(B):
        K, V = synth.make_kv(5000 + b, 128 * tiles[b] + wins[b], Hkv, d, 2)
        if tiles[b]:
            pool.append(oracle.compress_tiles(K, V, tiles[b]))
        rec_start.append(row)
        row += tiles[b]
        ws = b % 7                 # window rows start at a per-sequence offset
        kw[b, ws:ws + wins[b]] = K[128 * tiles[b]:]
        vw[b, ws:ws + wins[b]] = V[128 * tiles[b]:]
        win_start.append(ws)
        KV.append((K, V))
    recs = np.concatenate(pool)
    q = synth.make_q(6000, B, Hq, d)
    scale = 1 / math.sqrt(d)
    qd = to_dev(q)
    qr = kvarn.rotate_query(qd) if with_rot else None
    out = kvarn.decode_attention(qd, qr, to_dev(recs), rec_start, tiles, to_dev(kw), to_dev(vw),
                                 wins, scale, win_start=win_start)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(B):
        K, V = KV[b]
        if tiles[b]:
            kh, vh = oracle.dequant_records(recs[rec_start[b]:rec_start[b] + tiles[b]], d)
        else:
            kh = vh = np.zeros((0, Hkv, d))
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        worst = max(worst, rel_l2(got[b], ref))
    say("worst rel_l2", worst)
    assert worst < TOL


@pytest.mark.parametrize("Hq,Hkv,with_rot", [(16, 2, True), (32, 4, False), (8, 8, True), (4, 4, False)])
def test_decode_gqa_8_and_1_ragged_batch(Hq, Hkv, with_rot):
    """The head_dim-128 matrix-core decode with 8 query heads per KV head (all
    eight in one MFMA column block) and with one, over a ragged batch: long and
    short tile runs, windows from 1 token to past a 16-token split, a sequence
    with tiles only; both query paths."""
    say("decode gqa", Hq, Hkv, with_rot)
    d = 128
    tiles, wins = [40, 1, 7, 0], [300, 1, 0, 17]
    B = len(tiles)
    recs_all, rec_start, KV, row = [], [], [], 0
    cap = max(wins)
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    for b in range(B):
        K, V = synth.make_kv(7000 + 11 * b + Hq, 128 * tiles[b] + wins[b], Hkv, d, 2)
        if tiles[b]:
            recs_all.append(gpu_compress(K, V, tiles[b]))
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all)
    q = synth.make_q(7100 + Hq, B, Hq, d)
    scale = 1 / math.sqrt(d)
    qd = to_dev(q)
    out = kvarn.decode_attention(qd, kvarn.rotate_query(qd) if with_rot else None, to_dev(recs), rec_start,
                                 tiles, to_dev(kw), to_dev(vw), wins, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        if tiles[b]:
            mine = recs[rec_start[b]:rec_start[b] + tiles[b]]
            assert np.array_equal(mine, oracle.compress_tiles(K, V, tiles[b]))
            kh, vh = oracle.dequant_records(mine, d)
        else:
            kh = vh = np.zeros((0, Hkv, d))
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        err = rel_l2(got[b], ref)
        assert err < TOL, (b, err)


@pytest.mark.parametrize("d,Hq,Hkv,kbits,vbits,noalloc", [(128, 32, 8, 4, 2, False), (128, 16, 2, 4, 2, True),
                                                          (256, 16, 4, 4, 2, False), (128, 8, 2, 6, 5, False)])
def test_decode_appends_the_newest_token_in_the_call(d, Hq, Hkv, kbits, vbits, noalloc):
    """k_new / v_new: the call stores the newest token's rows as window token
    n_win - 1 of each sequence and attends them. Paths: the head_dim-128 K4V2
    split kernel (in the same launch, with the workspace and without), and the
    copy launch before the head_dim-256 and the vector-unit decode. The window
    rows start as NaN. The output must equal, to the bit, the same decode
    over a window that already holds the rows; every other window row must be
    untouched; ragged windows and window starts."""
    say("decode append", d, Hq, Hkv, kbits, vbits, noalloc)
    tiles, wins, starts = [6, 0, 3], [1, 40, 17], [0, 5, 2]
    B = len(tiles)
    k4v2 = (kbits, vbits) == (4, 2)
    cap = max(w + s for w, s in zip(wins, starts)) + 3
    kw = np.zeros((B, cap, Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    recs_all, rec_start, row = [], [], 0
    for b in range(B):
        K, V = synth.make_kv(8100 + 13 * b + d, 128 * tiles[b] + wins[b], Hkv, d, 2)
        if tiles[b]:
            recs_all.append(oracle.compress_tiles(K, V, tiles[b], kbits=kbits, vbits=vbits))
        rec_start.append(row)
        row += tiles[b]
        kw[b, starts[b]:starts[b] + wins[b]] = K[128 * tiles[b]:]
        vw[b, starts[b]:starts[b] + wins[b]] = V[128 * tiles[b]:]
    recs = to_dev(np.concatenate(recs_all))
    q = to_dev(synth.make_q(8200 + d, B, Hq, d))
    scale = 1 / math.sqrt(d)
    qr = None if k4v2 else kvarn.rotate_query(q)
    # the newest token of each sequence, and a window whose row for it is NaN
    last = [starts[b] + wins[b] - 1 for b in range(B)]
    k_new = to_dev(np.stack([kw[b, last[b]] for b in range(B)]))
    v_new = to_dev(np.stack([vw[b, last[b]] for b in range(B)]))
    kw_full, vw_full = to_dev(kw), to_dev(vw)
    kw_gap, vw_gap = kw_full.clone(), vw_full.clone()
    for b in range(B):
        kw_gap[b, last[b]] = float("nan")
        vw_gap[b, last[b]] = float("nan")
    args = dict(win_start=starts, kbits=kbits, vbits=vbits)
    want = kvarn.decode_attention(q, qr, recs, rec_start, tiles, kw_full, vw_full, wins, scale, **args)
    if noalloc:
        got = kvarn.decode_attention_noalloc(q, qr, recs, rec_start, tiles, kw_gap, vw_gap, wins, scale,
                                             nan_like(q), k_new=k_new, v_new=v_new, **args)
    else:
        nb = kvarn.decode_workspace_bytes(q, qr, recs, rec_start, tiles, kw_gap, vw_gap, wins, scale,
                                          kbits=kbits, vbits=vbits)
        got = kvarn.decode_attention(q, qr, recs, rec_start, tiles, kw_gap, vw_gap, wins, scale,
                                     out=nan_like(q), workspace=nan_bytes(nb), k_new=k_new, v_new=v_new,
                                     **args)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert torch.equal(kw_gap, kw_full) and torch.equal(vw_gap, vw_full)


@pytest.mark.parametrize("d,Hq,Hkv,f16", [(256, 4, 4, False), (256, 8, 4, True), (256, 16, 2, False),
                                          (512, 4, 4, True), (512, 4, 2, False), (512, 8, 2, False)])
def test_decode_wide_every_group_size_ragged(d, Hq, Hkv, f16):
    """Head_dim 256 / 512 over K4V2 records for each query group size G = Hq / Hkv
    (1, 2, 4, 8 heads in the matrix-core operand rows), in a ragged batch with a
    window-only sequence and one without window tokens; then the same records
    with every window empty (no window splits at all)."""
    say("decode wide group sizes", d, Hq, Hkv, f16)
    tiles, wins = [9, 0, 4, 1], [200, 37, 0, 256]
    B = len(tiles)
    kw = np.zeros((B, max(wins), Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    recs_all, rec_start, KV, row = [], [], [], 0
    for b in range(B):
        K, V = synth.make_kv(900 + 7 * b + d + Hq, 128 * tiles[b] + wins[b], Hkv, d, 4)
        if tiles[b]:
            rec = torch.zeros(tiles[b], Hkv, kvarn.tile_bytes(d, f16), dtype=torch.uint8, device=DEV)
            kvarn.compress_tile(to_dev(K), to_dev(V), rec, tiles[b], f16_scales=f16)
            torch.cuda.synchronize()
            recs_all.append(rec.cpu().numpy())
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    recs = np.concatenate(recs_all)
    q = synth.make_q(950 + d + Hq, B, Hq, d)
    qd = to_dev(q)
    scale = 1 / math.sqrt(d)
    deq = {}
    for b in range(B):
        K, V = KV[b]
        if tiles[b]:
            mine = recs[rec_start[b]:rec_start[b] + tiles[b]]
            assert np.array_equal(mine, oracle.compress_tiles(K, V, tiles[b], f16=f16))
            deq[b] = oracle.dequant_records(mine, d, f16=f16)
        else:
            deq[b] = (np.zeros((0, Hkv, d)), np.zeros((0, Hkv, d)))
    out = kvarn.decode_attention(qd, kvarn.rotate_query(qd), to_dev(recs), rec_start, tiles, to_dev(kw),
                                 to_dev(vw), wins, scale, f16_scales=f16)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        K, V = KV[b]
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], deq[b][0], deq[b][1], tiles[b], K[lo:], V[lo:], scale)
        err = rel_l2(got[b], ref)
        assert err < TOL, (b, err)
    # q_rot None: the tile kernel rotates the queries itself (same butterflies)
    out = kvarn.decode_attention(qd, None, to_dev(recs), rec_start, tiles, to_dev(kw), to_dev(vw), wins,
                                 scale, f16_scales=f16)
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), got) < 1e-6
    # tiles only: every window empty
    keep = [b for b in range(B) if tiles[b]]
    out = kvarn.decode_attention(qd[keep], kvarn.rotate_query(qd[keep]), to_dev(recs),
                                 [rec_start[b] for b in keep], [tiles[b] for b in keep], to_dev(kw[keep]),
                                 to_dev(vw[keep]), [0] * len(keep), scale, f16_scales=f16)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for i, b in enumerate(keep):
        K, V = KV[b]
        empty = K[:0]
        ref = oracle.decode(q[b], deq[b][0], deq[b][1], tiles[b], empty, V[:0], scale)
        err = rel_l2(got[i], ref)
        assert err < TOL, (b, err)


@pytest.mark.parametrize("d,Hq,Hkv", [(256, 4, 4), (512, 4, 2)])
def test_decode_wide_multi_tile_splits_small_groups(d, Hq, Hkv):
    """Head_dim 256 / 512 with query group sizes 1 and 2 in a batch large enough
    that the split plan puts two or more tiles in a split (each wave's softmax
    state then runs over several tiles): every sequence agrees with its own
    single-sequence call (one tile per split) to 1e-5, and the two shortest
    sequences with the oracle."""
    say("decode wide multi-tile splits", d, Hq, Hkv)
    B = 8
    tiles = [70, 3, 66, 5, 80, 71, 69, 75] if Hkv == 4 else [140, 3, 131, 5, 150, 142, 139, 145]
    wins = [256, 40, 130, 255, 1, 200, 64, 99]
    assert B * Hkv * max(tiles) > 2048          # over the decode plan's workgroup target: 2+ tiles per split
    recs_all, rec_start, KV, row = [], [], [], 0
    kw = np.zeros((B, max(wins), Hkv, d), np.float32)
    vw = np.zeros_like(kw)
    for b in range(B):
        K, V = synth.make_kv(1500 + 11 * b + d, 128 * tiles[b] + wins[b], Hkv, d, 4)
        rec = torch.zeros(tiles[b], Hkv, kvarn.tile_bytes(d), dtype=torch.uint8, device=DEV)
        kvarn.compress_tile(to_dev(K), to_dev(V), rec, tiles[b])
        recs_all.append(rec)
        rec_start.append(row)
        row += tiles[b]
        kw[b, :wins[b]] = K[128 * tiles[b]:]
        vw[b, :wins[b]] = V[128 * tiles[b]:]
        KV.append((K, V))
    pool = torch.cat(recs_all)
    q = synth.make_q(1600 + d, B, Hq, d)
    qd = to_dev(q)
    qr = kvarn.rotate_query(qd)
    scale = 1 / math.sqrt(d)
    kwd, vwd = to_dev(kw), to_dev(vw)
    out = kvarn.decode_attention(qd, qr, pool, rec_start, tiles, kwd, vwd, wins, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        one = kvarn.decode_attention(qd[b:b + 1], qr[b:b + 1], recs_all[b], [0], [tiles[b]], kwd[b:b + 1],
                                     vwd[b:b + 1], [wins[b]], scale)
        torch.cuda.synchronize()
        err = rel_l2(got[b], one.cpu().numpy()[0])
        assert err < 1e-5, (b, err)
    for b in (1, 3):
        K, V = KV[b]
        recs = recs_all[b].cpu().numpy()
        assert np.array_equal(recs, oracle.compress_tiles(K, V, tiles[b]))
        kh, vh = oracle.dequant_records(recs, d)
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        err = rel_l2(got[b], ref)
        assert err < TOL, (b, err)


@pytest.mark.parametrize("name", ["wide_d256", "wide_d512"])
def test_decode_wide_batch16_full_size_sampled(name):
    """The batched wide-head workload at its full size (16 sequences, contexts
    uniform in 1k-32k tokens in whole tiles, a 256-token window each), in the
    one call the benchmark times: a sampled record of every sequence byte for
    byte against the oracle; the two shortest sequences (which the oracle can
    compress whole in seconds) every record and the output against the fp64
    oracle; the three longest against one-sequence calls of their own (the
    batch changes only the split plan, so they agree to rounding)."""
    w = synth.WORKLOADS[name]
    d, Hq, Hkv, W, B = w.head_dim, w.n_q_heads, w.n_kv_heads, w.window, w.batch
    say("wide batch", name)
    tiles = [int(t) for t in synth.ragged_contexts(w.seed, B, w.extra["ctx_lo"], w.extra["ctx_hi"], W)]
    tb = kvarn.tile_bytes(d)
    rec_start = [int(x) for x in np.cumsum([0] + tiles[:-1])]
    pool = torch.empty(sum(tiles), Hkv, tb, dtype=torch.uint8, device=DEV)
    kw = torch.empty(B, W, Hkv, d, device=DEV)
    vw = torch.empty_like(kw)
    order = sorted(range(B), key=lambda b: tiles[b])
    short, long_ = order[:2], order[-3:]
    keep = {}
    pick = np.random.default_rng(w.seed)
    for b in range(B):
        K, V = synth.batch_sequence_kv(w, b, 128 * tiles[b] + W)
        kd, vd = to_dev(K), to_dev(V)
        kvarn.compress_tile(kd, vd, pool[rec_start[b]:rec_start[b] + tiles[b]], tiles[b])
        kw[b] = kd[128 * tiles[b]:]
        vw[b] = vd[128 * tiles[b]:]
        torch.cuda.synchronize()
        j = int(pick.integers(0, tiles[b]))
        got_rec = pool[rec_start[b] + j:rec_start[b] + j + 1].cpu().numpy()
        want_rec = oracle.compress_tiles(K[128 * j:128 * (j + 1)], V[128 * j:128 * (j + 1)], 1)
        assert np.array_equal(got_rec, want_rec), (b, j)
        if b in short:
            keep[b] = (K, V)
        del K, V, kd, vd
    say("tiles", tiles)
    q = synth.make_q(w.seed, B, Hq, d)
    qd = to_dev(q)
    scale = 1 / math.sqrt(d)
    out = kvarn.decode_attention(qd, kvarn.rotate_query(qd), pool, rec_start, tiles, kw, vw, [W] * B, scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in short:
        K, V = keep[b]
        want = oracle.compress_tiles(K, V, tiles[b])
        assert np.array_equal(pool[rec_start[b]:rec_start[b] + tiles[b]].cpu().numpy(), want), b
        kh, vh = oracle.dequant_records(want, d)
        lo = 128 * tiles[b]
        ref = oracle.decode(q[b], kh, vh, tiles[b], K[lo:], V[lo:], scale)
        err = rel_l2(got[b], ref)
        say("sequence", b, "tiles", tiles[b], "rel_l2", err)
        assert err < TOL, (b, err)
    for b in long_:
        qb = qd[b:b + 1].contiguous()
        one = kvarn.decode_attention(qb, kvarn.rotate_query(qb), pool, [rec_start[b]], [tiles[b]], kw[b:b + 1],
                                     vw[b:b + 1], [W], scale)
        torch.cuda.synchronize()
        diff = rel_l2(one.cpu().numpy()[0], got[b])
        say("sequence", b, "tiles", tiles[b], "batch vs alone", diff)
        assert diff < 1e-5, (b, diff)
