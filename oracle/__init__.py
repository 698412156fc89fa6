"""Plain CPU oracle for the KVarN hot path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.

Compression (fp32, fixed operation order) lives in ``kvarn_oracle.c``; this
module wraps it and evaluates attention in fp64 as the textbook definition:
softmax over the dequantised, unrotated cache plus the raw FP32 window.

Method sources (cited by page and section):
  * SharpInference issue #180 "Implement KVarN ...", "Algorithm (per
    128-token tile)" steps 1-4 (rotation, dual-axis normalisation, RTN,
    read-time scale folding, preset k4v2 g128).
  * SharpInference PR #434 "KVarN ... CPU + CUDA (#180)", commit list
    (FP32 window as staging with whole-tile promotion; chunked prefill with a
    single streaming softmax over compressed tiles plus the FP32 window and a
    deferred inverse WHT).
  * SharpInference issue #433 (follow-ups), item 2: split-tile decode with an
    LSE combine, inverse WHT after combining the rotated tile partials.
  * gmlx PR #116 "KVarN variance-normalized KV cache", commit list:
    speculative-verify widths 2-8 attend the compressed records (verify
    rows are decode queries).
  * gmlx PR #116 commit list: mixed-width "k6v5"-style arms and key/value
    widths chosen on their own (RTN with 2^b - 1 levels; the codes of every
    width are an LSB-first bit stream, which for 4/2 bits is the nibble and
    crumb order of the K4V2 record).
  * colibri PR #399, maintainer's "Ready for review" comment: for an
    orthogonal rotation, q . xhat == rotate(q) . c and the weighted value sum
    is the unrotation of the weighted code sum.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

TILE = 128
_HERE = os.path.dirname(os.path.abspath(__file__))
# KVARN_ORACLE_SANITIZED=1 loads the AddressSanitizer/UBSan build of the same
# C source (the sanitizer runtimes must be preloaded into the process).
_SANITIZED = os.environ.get("KVARN_ORACLE_SANITIZED") == "1"
_LIB_PATH = os.path.join(_HERE, "libkvarn_oracle_san.so" if _SANITIZED else "libkvarn_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build(sanitize=_SANITIZED)
    lib = ctypes.CDLL(_LIB_PATH)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_tile_bytes.restype = ctypes.c_longlong
    lib.oracle_tile_bytes.argtypes = [ctypes.c_int]
    lib.oracle_tile_bytes_fmt.restype = ctypes.c_longlong
    lib.oracle_tile_bytes_fmt.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.oracle_layout.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_longlong)]
    lib.oracle_layout_fmt.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_longlong)]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_wht_scale.restype = ctypes.c_float
    lib.oracle_wht_scale.argtypes = [ctypes.c_int]
    lib.oracle_wht_f32.argtypes = [f32p, ctypes.c_int]
    lib.oracle_pairwise_sum_f32.restype = ctypes.c_float
    lib.oracle_pairwise_sum_f32.argtypes = [f32p, ctypes.c_int]
    lib.oracle_sinkhorn_f32.argtypes = [f32p, ctypes.c_int, ctypes.c_int, f32p, f32p]
    lib.oracle_normalise_f32.argtypes = [f32p, ctypes.c_int, f32p, f32p, f32p]
    lib.oracle_rtn_group.argtypes = [f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     f32p, f32p, u8p, ctypes.c_int]
    lib.oracle_compress_tile.restype = ctypes.c_int
    lib.oracle_compress_tile.argtypes = [f32p, f32p, ctypes.c_longlong, ctypes.c_int,
                                         ctypes.c_int, u8p]
    lib.oracle_compress_tile_fmt.restype = ctypes.c_int
    lib.oracle_compress_tile_fmt.argtypes = [f32p, f32p, ctypes.c_longlong, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, u8p]
    lib.oracle_unpack_codes.argtypes = [u8p, ctypes.c_int, u8p, u8p]
    i = ctypes.c_int
    lib.oracle_tile_bytes_w.restype = ctypes.c_longlong
    lib.oracle_tile_bytes_w.argtypes = [i, i, i, i]
    lib.oracle_layout_w.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_longlong)]
    lib.oracle_compress_tile_w.restype = ctypes.c_int
    lib.oracle_compress_tile_w.argtypes = [f32p, f32p, ctypes.c_longlong, i, i, i, i, i, u8p]
    lib.oracle_unpack_codes_w.argtypes = [u8p, i, i, i, u8p, u8p]
    lib.oracle_dequant_f64_w.argtypes = [u8p, i, i, i, i, i, f64p, f64p]
    lib.oracle_dequant_f64.argtypes = [u8p, ctypes.c_int, ctypes.c_int, f64p, f64p]
    lib.oracle_dequant_f64_fmt.argtypes = [u8p, ctypes.c_int, ctypes.c_int, ctypes.c_int, f64p, f64p]
    lib.oracle_attend_f64.argtypes = [f64p, f64p, f64p, ctypes.c_longlong, ctypes.c_int,
                                      ctypes.c_double, f64p, f64p]
    _lib = lib
    return lib


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


# --------------------------------------------------------------------------
# sizes and layout
# --------------------------------------------------------------------------

def _k4v2(kbits, vbits):
    return kbits == 4 and vbits == 2


def tile_bytes(d: int, f16: bool = False, kbits: int = 4, vbits: int = 2) -> int:
    """Bytes of one (tile, kv-head) record: 116*d + 512 with fp32 scales, or
    106*d + 256 with f16 scales (SharpInference issue #433 item 3), for 4-bit
    keys and 2-bit values; 16*d*(kbits + vbits) code bytes in general.  0 if
    d or a width is unsupported."""
    if _k4v2(kbits, vbits):
        return int(_load().oracle_tile_bytes_fmt(d, 1 if f16 else 0))
    return int(_load().oracle_tile_bytes_w(d, 1 if f16 else 0, kbits, vbits))


def layout(d: int, f16: bool = False, kbits: int = 4, vbits: int = 2) -> dict:
    """Byte offsets of the record sections."""
    off = (ctypes.c_longlong * 9)()
    if _k4v2(kbits, vbits):
        _load().oracle_layout_fmt(d, 1 if f16 else 0, off)
    else:
        _load().oracle_layout_w(d, 1 if f16 else 0, kbits, vbits, off)
    names = ["kcode", "vcode", "ktok", "kscale", "kmin", "vchan", "vscale", "vmin", "end"]
    return dict(zip(names, [int(x) for x in off]))


def f32_to_f16_bits(x: float) -> int:
    """The oracle's binary32 -> binary16 rounding (nearest, ties to even)."""
    return int(_load().oracle_f32_to_f16(float(np.float32(x))))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(int(h)))


def visible_tiles(pos: int, window: int) -> int:
    """Compressed tiles visible to the query at 0-based position ``pos``.

    The FP32 window keeps at least ``window`` tokens; when it reaches
    window+128 the oldest 128 are promoted as one tile (PR #434 commit list:
    "the FP32 window is the staging; whole-tile promotion").  So after token
    ``pos`` the cache holds max(0, floor((pos + 1 - window) / 128)) tiles.
    """
    return max(0, (pos + 1 - window) // TILE)


# --------------------------------------------------------------------------
# fp32 building blocks (exposed for the pins)
# --------------------------------------------------------------------------

def wht_scale(d: int) -> np.float32:
    return np.float32(_load().oracle_wht_scale(d))


def wht_f32(x: np.ndarray) -> np.ndarray:
    """Row-wise fp32 WHT (stages h = 1, 2, ..., d/2, then scale)."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    d = x.shape[-1]
    flat = x.reshape(-1, d)
    lib = _load()
    for i in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[i])
        lib.oracle_wht_f32(_p(row, ctypes.c_float), d)
        flat[i] = row
    return flat.reshape(x.shape)


def pairwise_sum_f32(y: np.ndarray) -> np.float32:
    y = np.ascontiguousarray(y, dtype=np.float32)
    return np.float32(_load().oracle_pairwise_sum_f32(_p(y, ctypes.c_float), y.size))


def sinkhorn_f32(X: np.ndarray, iters: int = 8):
    """Per-token spread r[128] and per-channel spread s[d] of a rotated tile."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    d = X.shape[1]
    r = np.zeros(TILE, np.float32)
    s = np.zeros(d, np.float32)
    _load().oracle_sinkhorn_f32(_p(X, ctypes.c_float), d, iters,
                                _p(r, ctypes.c_float), _p(s, ctypes.c_float))
    return r, s


def normalise_f32(X, r, s):
    X = np.ascontiguousarray(X, dtype=np.float32)
    r = np.ascontiguousarray(r, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.zeros_like(X)
    _load().oracle_normalise_f32(_p(X, ctypes.c_float), X.shape[1], _p(r, ctypes.c_float),
                                 _p(s, ctypes.c_float), _p(out, ctypes.c_float))
    return out


def rtn_group(x: np.ndarray, bits: int):
    """Asymmetric RTN of one group: returns (lo, delta, codes)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    lo = np.zeros(1, np.float32)
    dl = np.zeros(1, np.float32)
    z = np.zeros(x.size, np.uint8)
    _load().oracle_rtn_group(_p(x, ctypes.c_float), x.size, 1, (1 << bits) - 1,
                             _p(lo, ctypes.c_float), _p(dl, ctypes.c_float),
                             _p(z, ctypes.c_uint8), 1)
    return np.float32(lo[0]), np.float32(dl[0]), z


# --------------------------------------------------------------------------
# compression
# --------------------------------------------------------------------------

def _tiles_in(k_tile, v_tile):
    k = np.ascontiguousarray(k_tile, dtype=np.float32)
    v = np.ascontiguousarray(v_tile, dtype=np.float32)
    assert k.shape == v.shape and k.shape[0] == TILE
    return k, v, k.shape[1]


def compress_tile_bits(k_tile: np.ndarray, v_tile: np.ndarray, iters: int = 8, f16: bool = False,
                       kbits: int = 4, vbits: int = 2) -> np.ndarray:
    """compress_tile packed by the bit-stream writer (any widths, 4/2 included)."""
    k, v, d = _tiles_in(k_tile, v_tile)
    rec = np.zeros(int(_load().oracle_tile_bytes_w(d, 1 if f16 else 0, kbits, vbits)), np.uint8)
    rc = _load().oracle_compress_tile_w(_p(k, ctypes.c_float), _p(v, ctypes.c_float), d, d, iters,
                                        1 if f16 else 0, kbits, vbits, _p(rec, ctypes.c_uint8))
    if rc != 0:
        raise ValueError(f"unsupported head_dim {d} or widths {kbits}/{vbits}")
    return rec


def compress_tile(k_tile: np.ndarray, v_tile: np.ndarray, iters: int = 8,
                  f16: bool = False, kbits: int = 4, vbits: int = 2) -> np.ndarray:
    """One (tile, kv head): raw fp32 K and V tiles [128][d] -> record bytes.
    With f16 the six scale vectors are stored rounded to half precision
    (nearest, ties to even); the codes are those of the fp32 record.  Keys
    take kbits-bit codes, values vbits-bit codes (K4V2 by default, packed
    nibble by nibble; other widths by the bit-stream writer)."""
    if not _k4v2(kbits, vbits):
        return compress_tile_bits(k_tile, v_tile, iters, f16, kbits, vbits)
    k, v, d = _tiles_in(k_tile, v_tile)
    rec = np.zeros(tile_bytes(d, f16), np.uint8)
    rc = _load().oracle_compress_tile_fmt(_p(k, ctypes.c_float), _p(v, ctypes.c_float), d, d,
                                          iters, 1 if f16 else 0, _p(rec, ctypes.c_uint8))
    if rc != 0:
        raise ValueError(f"unsupported head_dim {d}")
    return rec


def compress_tiles(K: np.ndarray, V: np.ndarray, n_tiles: int, iters: int = 8,
                   f16: bool = False, kbits: int = 4, vbits: int = 2) -> np.ndarray:
    """K, V: [n_tokens][n_kv][d] raw fp32.  Returns records [n_tiles][n_kv][bytes]
    for the first n_tiles whole tiles."""
    n_kv, d = K.shape[1], K.shape[2]
    out = np.zeros((n_tiles, n_kv, tile_bytes(d, f16, kbits, vbits)), np.uint8)
    for j in range(n_tiles):
        for h in range(n_kv):
            out[j, h] = compress_tile(K[TILE * j:TILE * (j + 1), h], V[TILE * j:TILE * (j + 1), h],
                                      iters, f16, kbits, vbits)
    return out


def unpack_codes_bits(rec: np.ndarray, d: int, kbits: int = 4, vbits: int = 2):
    """zK[t][c], zV[t][c] read by the bit-stream reader (any widths)."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    zK = np.zeros((TILE, d), np.uint8)
    zV = np.zeros((TILE, d), np.uint8)
    _load().oracle_unpack_codes_w(_p(rec, ctypes.c_uint8), d, kbits, vbits, _p(zK, ctypes.c_uint8),
                                  _p(zV, ctypes.c_uint8))
    return zK, zV


def unpack_codes(rec: np.ndarray, d: int, kbits: int = 4, vbits: int = 2):
    if not _k4v2(kbits, vbits):
        return unpack_codes_bits(rec, d, kbits, vbits)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    zK = np.zeros((TILE, d), np.uint8)
    zV = np.zeros((TILE, d), np.uint8)
    _load().oracle_unpack_codes(_p(rec, ctypes.c_uint8), d, _p(zK, ctypes.c_uint8),
                                _p(zV, ctypes.c_uint8))
    return zK, zV


def record_scales(rec: np.ndarray, d: int, f16: bool = False, kbits: int = 4,
                  vbits: int = 2) -> dict:
    """The six scale vectors of a record as fp32 numpy arrays."""
    off = layout(d, f16, kbits, vbits)
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    ng = d // 128
    w, dt = (2, np.float16) if f16 else (4, np.float32)

    def get(a, n):
        return rec[off[a]:off[a] + w * n].view(dt).astype(np.float32)
    return {
        "ktok": get("ktok", TILE), "kscale": get("kscale", d), "kmin": get("kmin", d),
        "vchan": get("vchan", d), "vscale": get("vscale", TILE * ng).reshape(TILE, ng),
        "vmin": get("vmin", TILE * ng).reshape(TILE, ng),
    }


# --------------------------------------------------------------------------
# dequantised cache and attention (fp64)
# --------------------------------------------------------------------------

def hadamard_f64(d: int) -> np.ndarray:
    """Orthonormal Sylvester Hadamard: H[i][j] = (-1)^popcount(i & j) / sqrt(d)."""
    i = np.arange(d)
    parity = np.zeros((d, d), np.int64)
    x = i[:, None] & i[None, :]
    while np.any(x):
        parity ^= x & 1
        x >>= 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(d)


def dequant_rotated(rec: np.ndarray, d: int, f16: bool = False, kbits: int = 4, vbits: int = 2):
    """k'[t][c], v'[t][c] in the rotated domain (fp64), from the stored codes
    and folded scales."""
    rec = np.ascontiguousarray(rec, dtype=np.uint8)
    kd = np.zeros((TILE, d), np.float64)
    vd = np.zeros((TILE, d), np.float64)
    if _k4v2(kbits, vbits):
        _load().oracle_dequant_f64_fmt(_p(rec, ctypes.c_uint8), d, 1 if f16 else 0, 1,
                                       _p(kd, ctypes.c_double), _p(vd, ctypes.c_double))
    else:
        _load().oracle_dequant_f64_w(_p(rec, ctypes.c_uint8), d, 1 if f16 else 0, kbits, vbits, 1,
                                     _p(kd, ctypes.c_double), _p(vd, ctypes.c_double))
    return kd, vd


def dequant(rec: np.ndarray, d: int, f16: bool = False, kbits: int = 4, vbits: int = 2):
    """khat = H k', vhat = H v' (fp64, raw domain)."""
    kd, vd = dequant_rotated(rec, d, f16, kbits, vbits)
    H = hadamard_f64(d)
    return kd @ H.T, vd @ H.T


def dequant_records(records: np.ndarray, d: int, f16: bool = False, kbits: int = 4,
                    vbits: int = 2):
    """records [T][n_kv][bytes] -> khat, vhat [T*128][n_kv][d] fp64."""
    T, n_kv = records.shape[0], records.shape[1]
    kh = np.zeros((T * TILE, n_kv, d))
    vh = np.zeros((T * TILE, n_kv, d))
    H = hadamard_f64(d)
    for j in range(T):
        for h in range(n_kv):
            kd, vd = dequant_rotated(records[j, h], d, f16, kbits, vbits)
            kh[TILE * j:TILE * (j + 1), h] = kd @ H.T
            vh[TILE * j:TILE * (j + 1), h] = vd @ H.T
    return kh, vh


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Textbook softmax attention in fp64 for one query over n keys:
    s_j = scale * q.k_j, p = softmax(s) (max-subtracted), out = sum p_j v_j.
    Returns (out[d], lse)."""
    q = np.asarray(q, np.float64)
    s = scale * (np.asarray(keys, np.float64) @ q)
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    return (p @ np.asarray(vals, np.float64)) / l, m + np.log(l)


def attend_c(q, keys, vals, scale):
    """The same definition, as a plain C loop (cross-check of ``attend``)."""
    q = np.ascontiguousarray(q, np.float64)
    keys = np.ascontiguousarray(keys, np.float64)
    vals = np.ascontiguousarray(vals, np.float64)
    out = np.zeros(q.shape[-1])
    lse = np.zeros(1)
    _load().oracle_attend_f64(_p(q, ctypes.c_double), _p(keys, ctypes.c_double),
                              _p(vals, ctypes.c_double), keys.shape[0], q.shape[-1], scale,
                              _p(out, ctypes.c_double), _p(lse, ctypes.c_double))
    return out, float(lse[0])


def decode(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, n_tiles: int,
           k_win: np.ndarray, v_win: np.ndarray, scale: float) -> np.ndarray:
    """One decode query per head over n_tiles compressed tiles plus the window.

    q: [Hq][d] raw query.  khat/vhat: dequantised tiles [>=128*n_tiles][Hkv][d].
    k_win/v_win: raw FP32 window [n_w][Hkv][d].  Query head h reads KV head
    h // (Hq/Hkv).  Returns out [Hq][d] fp64.
    """
    Hq, d = q.shape
    Hkv = k_win.shape[1] if k_win.size else khat.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, d))
    nt = TILE * n_tiles
    for h in range(Hq):
        kv = h // G
        keys = np.concatenate([khat[:nt, kv], np.asarray(k_win[:, kv], np.float64)], axis=0)
        vals = np.concatenate([vhat[:nt, kv], np.asarray(v_win[:, kv], np.float64)], axis=0)
        out[h], _ = attend(q[h], keys, vals, scale)
    return out


def prefill_row(q_row: np.ndarray, pos: int, window: int, khat: np.ndarray,
                vhat: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Prefill output at position ``pos``: the decode view at that position,
    i.e. tiles [0, T(pos)) compressed plus raw tokens [128*T(pos), pos].
    q_row: [Hq][d]; K, V: raw [n_tokens][Hkv][d]."""
    T = visible_tiles(pos, window)
    lo = TILE * T
    return decode(q_row, khat, vhat, T, K[lo:pos + 1], V[lo:pos + 1], scale)


def verify(q: np.ndarray, khat: np.ndarray, vhat: np.ndarray, n_tiles: int,
           k_win: np.ndarray, v_win: np.ndarray, scale: float) -> np.ndarray:
    """Multi-query verify (gmlx PR #116 commit list, verify widths 2-8): the
    w = q.shape[0] newest window tokens are the query rows; row i is the
    decode query of window token n_w - w + i and sees the n_tiles tiles plus
    window tokens [0, n_w - w + i].  q: [w][Hq][d]; k_win/v_win: the raw
    window [n_w][Hkv][d].  Returns out [w][Hq][d] fp64."""
    w = q.shape[0]
    n_w = k_win.shape[0]
    assert n_w >= w
    return np.stack([decode(q[i], khat, vhat, n_tiles, k_win[:n_w - w + i + 1],
                            v_win[:n_w - w + i + 1], scale) for i in range(w)])
