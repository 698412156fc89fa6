"""Thin ctypes binding of libkvarn.so (include/kvarn.h).

Argument marshalling only: tensors become device pointers and strides, the
current torch stream becomes the hipStream_t, and a non-zero status raises.
Every step of the computation runs in the HIP kernels; there is no CPU path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvarn.so")
TILE = 128

KVARN_OK = 0
SCALES_F16 = 0x10000   # head_dim flag: records with f16 scales


def KEY_BITS(b: int) -> int:     # head_dim field: key code width 1..8
    return (b & 0xF) << 20


def VALUE_BITS(b: int) -> int:   # head_dim field: value code width 1..8
    return (b & 0xF) << 24
STATUS = {0: "KVARN_OK", 1: "KVARN_E_INVALID", 2: "KVARN_E_UNSUPPORTED", 3: "KVARN_E_ALIGN",
          4: "KVARN_E_WORKSPACE", 5: "KVARN_E_DEVICE"}


class KVarNError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("max_tiles", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_rot", ctypes.c_void_p),
        ("records", ctypes.c_void_p), ("n_record_rows", ctypes.c_int64),
        ("rec_start", ctypes.POINTER(ctypes.c_int64)),
        ("n_tiles", ctypes.POINTER(ctypes.c_int32)),
        ("k_win", ctypes.c_void_p), ("v_win", ctypes.c_void_p),
        ("win_seq_stride", ctypes.c_int64), ("win_tok_stride", ctypes.c_int64),
        ("win_head_stride", ctypes.c_int64),
        ("win_start", ctypes.POINTER(ctypes.c_int64)),
        ("n_win", ctypes.POINTER(ctypes.c_int32)), ("max_win", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("q_len", ctypes.c_int32),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
    ]


class PrefillArgs(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("window", ctypes.c_int32),
        ("pos0", ctypes.c_int64), ("chunk", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q", ctypes.c_void_p), ("q_rot", ctypes.c_void_p),
        ("records", ctypes.c_void_p), ("n_record_rows", ctypes.c_int64),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("tok_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
        ("raw_base", ctypes.c_int64), ("out", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kvarn_status_string.restype = ctypes.c_char_p
    L.kvarn_status_string.argtypes = [ctypes.c_int]
    L.kvarn_tile_bytes.restype = ctypes.c_size_t
    L.kvarn_tile_bytes.argtypes = [i32]
    L.kvarn_compress_tile.restype = ctypes.c_int
    L.kvarn_compress_tile.argtypes = [i32, i32, i32, vp, vp, i64, i64, vp, vp]
    L.kvarn_rotate_query.restype = ctypes.c_int
    L.kvarn_rotate_query.argtypes = [i32, i64, vp, vp, vp]
    L.kvarn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvarn_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
    L.kvarn_decode_attention.restype = ctypes.c_int
    L.kvarn_decode_attention.argtypes = [ctypes.POINTER(DecodeArgs), vp, ctypes.c_size_t, vp]
    L.kvarn_decode_attention_noalloc.restype = ctypes.c_int
    L.kvarn_decode_attention_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), vp]
    L.kvarn_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.kvarn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
    L.kvarn_prefill_attention.restype = ctypes.c_int
    L.kvarn_prefill_attention.argtypes = [ctypes.POINTER(PrefillArgs), vp, ctypes.c_size_t, vp]
    _lib = L
    return L


def _check(fn, st):
    if st != KVARN_OK:
        raise KVarNError(fn, st)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kvarn kernels take device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _hd(d: int, f16_scales: bool = False, kbits: int = 4, vbits: int = 2) -> int:
    """The head_dim format word: d, the f16-scale flag and the code widths."""
    hd = d | SCALES_F16 if f16_scales else d
    if (kbits, vbits) != (4, 2):
        hd |= KEY_BITS(kbits) | VALUE_BITS(vbits)
    return hd


def tile_bytes(head_dim: int, f16_scales: bool = False, kbits: int = 4, vbits: int = 2) -> int:
    return int(lib().kvarn_tile_bytes(_hd(head_dim, f16_scales, kbits, vbits)))


def _check_records(records, d, f16_scales, kbits=4, vbits=2):
    if records is not None and records.dim() == 3:
        assert records.shape[-1] == tile_bytes(d, f16_scales, kbits, vbits), \
            "record size does not match the format"


def compress_tile(k: torch.Tensor, v: torch.Tensor, records: torch.Tensor, n_tiles: int,
                  stream=None, f16_scales: bool = False, kbits: int = 4, vbits: int = 2) -> None:
    """Compress tiles [0, n_tiles) of raw k/v ([tokens][kv_heads][d] views with
    contiguous channels) into records ([n_tiles][kv_heads][tile_bytes] uint8);
    f16_scales selects the record with f16 scales, kbits / vbits the code
    widths (1..8; K4V2 by default)."""
    assert k.shape == v.shape and k.stride() == v.stride() and k.stride(2) == 1
    d, n_kv = k.shape[2], k.shape[1]
    if n_tiles > 0:
        assert k.shape[0] >= TILE * n_tiles
        assert records.numel() >= n_tiles * n_kv * tile_bytes(d, f16_scales, kbits, vbits)
        assert records.dtype == torch.uint8
        _check_records(records, d, f16_scales, kbits, vbits)
    _check("kvarn_compress_tile", lib().kvarn_compress_tile(
        _hd(d, f16_scales, kbits, vbits), n_tiles, n_kv, _ptr(k), _ptr(v), k.stride(0),
        k.stride(1), _ptr(records), _stream(stream)))


def rotate_query(q: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """H q along the last dim of a contiguous fp32 tensor."""
    assert q.is_contiguous() and q.dtype == torch.float32
    if out is None:
        out = torch.empty_like(q)
    d = q.shape[-1]
    _check("kvarn_rotate_query", lib().kvarn_rotate_query(
        d, q.numel() // d, _ptr(q), _ptr(out), _stream(stream)))
    return out


def _decode_args(q, q_rot, records, n_record_rows, rec_start, n_tiles, k_win, v_win, n_win,
                 scale, out, max_tiles=None, max_win=None, win_start=None, f16_scales=False,
                 kbits=4, vbits=2, k_new=None, v_new=None):
    if q.dim() == 4:   # [B][q_len][Hq][d]: multi-query verify rows
        B, w, Hq, d = q.shape
    else:
        (B, Hq, d), w = q.shape, 1
    n_kv = k_win.shape[2] if k_win is not None else records.shape[1]
    rs = (ctypes.c_int64 * B)(*[int(x) for x in rec_start])
    ws = (ctypes.c_int64 * B)(*[int(x) for x in (win_start if win_start is not None else [0] * B)])
    nt = (ctypes.c_int32 * B)(*[int(x) for x in n_tiles])
    nw = (ctypes.c_int32 * B)(*[int(x) for x in n_win])
    a = DecodeArgs()
    _check_records(records, d, f16_scales, kbits, vbits)
    a.head_dim, a.batch, a.n_q_heads, a.n_kv_heads = _hd(d, f16_scales, kbits, vbits), B, Hq, n_kv
    a.softmax_scale = scale
    a.max_tiles = int(max(n_tiles)) if max_tiles is None else int(max_tiles)
    a.q, a.q_rot = _ptr(q), (_ptr(q_rot) if q_rot is not None else None)
    a.records = _ptr(records) if records is not None else None
    a.n_record_rows = n_record_rows
    a.rec_start, a.n_tiles, a.n_win, a.win_start = rs, nt, nw, ws
    a.k_win, a.v_win = _ptr(k_win), _ptr(v_win)
    if k_win is not None:
        a.win_seq_stride, a.win_tok_stride, a.win_head_stride = k_win.stride(0), k_win.stride(1), k_win.stride(2)
    a.max_win = int(max(n_win)) if max_win is None else int(max_win)
    a.out = _ptr(out)
    a.q_len = w
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
    return a, (rs, nt, nw, ws)


def decode_attention(q, q_rot, records, rec_start, n_tiles, k_win, v_win, n_win, scale,
                     out=None, workspace=None, max_tiles=None, max_win=None, stream=None,
                     win_start=None, f16_scales=False, kbits=4, vbits=2, k_new=None, v_new=None):
    """Decode attention for a batch.

    q, q_rot: [B][Hq][d] fp32 (q_rot may be None over K4V2 records: the kernels
    rotate q themselves), or [B][w][Hq][d] for a multi-query verify of width
    w = 2..8 (head_dim 128): row i is the query of window token n_win - w + i
    and sees the tiles and window tokens [0, n_win - w + i].  records: uint8 pool [rows][Hkv][tile_bytes];
    sequence b's tile j is row rec_start[b] + j.  k_win, v_win: [B][cap][Hkv][d]
    raw windows (strided views allowed, channels contiguous); n_tiles, n_win:
    per-sequence counts (host sequences); win_start: first window row of each
    sequence (default 0); f16_scales: the records carry f16 scales; kbits /
    vbits: their code widths; k_new, v_new: [B][Hkv][d] rows of each
    sequence's newest token, stored by the call as window token n_win - 1
    and attended (None: the window already holds them).  Returns out [B][Hq][d]."""
    if out is None:
        out = torch.empty_like(q)
    rows = records.shape[0] if records is not None else 0
    a, keep = _decode_args(q, q_rot, records, rows, rec_start, n_tiles, k_win, v_win, n_win,
                           scale, out, max_tiles, max_win, win_start, f16_scales, kbits, vbits,
                           k_new, v_new)
    need = int(lib().kvarn_decode_workspace_bytes(ctypes.byref(a)))
    if workspace is None:   # scratch: the kernels write every byte they read
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("kvarn_decode_attention", lib().kvarn_decode_attention(
        ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_attention_noalloc(q, q_rot, records, rec_start, n_tiles, k_win, v_win, n_win, scale, out,
                             max_tiles=None, max_win=None, stream=None, win_start=None,
                             f16_scales=False, kbits=4, vbits=2, k_new=None, v_new=None):
    """decode_attention without a workspace: the split partials go to the
    library's own per-GPU scratch array (at most NOALLOC_SCRATCH_BYTES of
    partials; larger calls raise KVARN_E_WORKSPACE).  `out` must be given, so
    the call makes no allocation."""
    rows = records.shape[0] if records is not None else 0
    a, keep = _decode_args(q, q_rot, records, rows, rec_start, n_tiles, k_win, v_win, n_win,
                           scale, out, max_tiles, max_win, win_start, f16_scales, kbits, vbits,
                           k_new, v_new)
    _check("kvarn_decode_attention_noalloc",
           lib().kvarn_decode_attention_noalloc(ctypes.byref(a), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_workspace_bytes(q, q_rot, records, rec_start, n_tiles, k_win, v_win, n_win, scale,
                           max_tiles=None, max_win=None, f16_scales=False, kbits=4,
                           vbits=2) -> int:
    rows = records.shape[0] if records is not None else 0
    a, keep = _decode_args(q, q_rot, records, rows, rec_start, n_tiles, k_win, v_win, n_win,
                           scale, q, max_tiles, max_win, f16_scales=f16_scales, kbits=kbits,
                           vbits=vbits)
    return int(lib().kvarn_decode_workspace_bytes(ctypes.byref(a)))


def _prefill_args(q, q_rot, records, n_record_rows, k, v, raw_base, pos0, window, scale, out,
                  f16_scales=False, kbits=4, vbits=2):
    C, Hq, d = q.shape
    _check_records(records, d, f16_scales, kbits, vbits)
    a = PrefillArgs()
    a.head_dim, a.n_q_heads, a.n_kv_heads, a.window = (_hd(d, f16_scales, kbits, vbits), Hq,
                                                       k.shape[1], window)
    a.pos0, a.chunk, a.softmax_scale = pos0, C, scale
    a.q, a.q_rot = _ptr(q), _ptr(q_rot)
    a.records = _ptr(records) if records is not None else None
    a.n_record_rows = n_record_rows
    a.k, a.v = _ptr(k), _ptr(v)
    a.tok_stride, a.head_stride = k.stride(0), k.stride(1)
    a.raw_base = raw_base
    a.out = _ptr(out)
    return a


def prefill_workspace_bytes(q, q_rot, records, n_record_rows, k, v, raw_base, pos0, window,
                            scale, f16_scales=False, kbits=4, vbits=2) -> int:
    """Workspace bytes of a prefill_attention call with these arguments."""
    a = _prefill_args(q, q_rot, records, n_record_rows, k, v, raw_base, pos0, window, scale, q,
                      f16_scales, kbits, vbits)
    return int(lib().kvarn_prefill_workspace_bytes(ctypes.byref(a)))


def prefill_attention(q, q_rot, records, n_record_rows, k, v, raw_base, pos0, window, scale,
                      out=None, workspace=None, stream=None, f16_scales=False, kbits=4, vbits=2,
                      no_workspace=False):
    """Chunk of C query positions [pos0, pos0+C) of one sequence.

    q, q_rot: [C][Hq][d] (q_rot may be None over K4V2 records: the kernels
    rotate the rows themselves).  records: [rows][Hkv][tile_bytes] (tile j = row j).
    k, v: raw [n][Hkv][d] views whose row i is absolute position raw_base + i;
    f16_scales: the records carry f16 scales; kbits / vbits: their code widths.
    workspace: None allocates what the call needs; no_workspace passes NULL
    (head_dim 128 over K4V2 records only: the single-launch kernel)."""
    assert k.stride(2) == 1 and k.stride() == v.stride()
    if out is None:
        out = torch.empty_like(q)
    a = _prefill_args(q, q_rot, records, n_record_rows, k, v, raw_base, pos0, window, scale, out,
                      f16_scales, kbits, vbits)
    if no_workspace:
        ws_ptr, ws_bytes = None, 0
    else:
        need = int(lib().kvarn_prefill_workspace_bytes(ctypes.byref(a)))
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _check("kvarn_prefill_attention", lib().kvarn_prefill_attention(
        ctypes.byref(a), ws_ptr, ws_bytes, _stream(stream)))
    return out


def visible_tiles(pos: int, window: int) -> int:
    """Host bookkeeping of the promotion rule: tiles held after token pos."""
    ahead = pos + 1 - window
    return ahead // TILE if ahead > 0 else 0
