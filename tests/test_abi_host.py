"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/kvarn.h declares, and rejects bad arguments before
anything is enqueued (no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvarn.h")


@pytest.fixture(scope="module")
def L():
    from quantized_attention_tok_amd import build_lib, kvarn
    if not os.path.exists(kvarn.LIB_PATH):
        build_lib.build()
    return kvarn.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) == 9, names
    for n in names:
        assert hasattr(L, n), n


def test_tile_bytes_and_status_strings(L):
    assert [L.kvarn_tile_bytes(d) for d in (128, 256, 512)] == [15360, 30208, 59904]
    assert L.kvarn_tile_bytes(64) == 0 and L.kvarn_tile_bytes(1024) == 0
    assert L.kvarn_status_string(0) == b"KVARN_OK"
    assert L.kvarn_status_string(4) == b"KVARN_E_WORKSPACE"
    assert L.kvarn_status_string(99) == b"KVARN_E_UNKNOWN"


def test_f16_scale_flag_sizes_match_the_oracle_record(L):
    import oracle
    from quantized_attention_tok_amd import kvarn
    m = re.search(r"#define\s+KVARN_SCALES_F16\s+(0x[0-9a-fA-F]+)", open(HEADER).read())
    assert m and int(m.group(1), 16) == kvarn.SCALES_F16
    F = kvarn.SCALES_F16
    for d in (128, 256, 512):
        assert L.kvarn_tile_bytes(d | F) == oracle.tile_bytes(d, f16=True)
        assert L.kvarn_tile_bytes(d) == oracle.tile_bytes(d)
    assert L.kvarn_tile_bytes(128 | F) == 13824   # 108 bytes per token at d = 128
    assert L.kvarn_tile_bytes(128 | 0x20000) == 0 and L.kvarn_tile_bytes(96 | F) == 0


def test_code_width_fields_and_sizes_match_the_oracle_record(L):
    import oracle
    from quantized_attention_tok_amd import kvarn
    text = open(HEADER).read()
    assert re.search(r"#define\s+KVARN_KEY_BITS\(b\)\s+\(\(\(b\) & 0xF\) << 20\)", text)
    assert re.search(r"#define\s+KVARN_VALUE_BITS\(b\)\s+\(\(\(b\) & 0xF\) << 24\)", text)
    for d in (128, 256, 512):
        for kb in range(1, 9):
            for vb in range(1, 9):
                for f16 in (False, True):
                    hd = kvarn._hd(d, f16, kb, vb)
                    assert L.kvarn_tile_bytes(hd) == oracle.tile_bytes(d, f16, kb, vb), (d, kb, vb, f16)
    # a zero field is the K4V2 default; widths above 8 are unsupported
    assert L.kvarn_tile_bytes(128 | (4 << 20) | (2 << 24)) == L.kvarn_tile_bytes(128)
    assert L.kvarn_tile_bytes(128 | (9 << 20)) == 0 and L.kvarn_tile_bytes(128 | (15 << 24)) == 0
    assert L.kvarn_tile_bytes(128 | (1 << 28)) == 0


# These calls pass fake device pointers that every case must reject before a
# launch; on a machine with a GPU a wrongly accepted case would launch a kernel
# on them, so the module only runs where no GPU is visible.
if os.path.exists("/dev/kfd"):
    pytest.skip("host-only validation checks (fake pointers); a GPU is visible", allow_module_level=True)

FAKE = 0x10000  # aligned but never dereferenced: every call below fails validation first
# A status of KVARN_OK (0) or KVARN_E_DEVICE (5) would mean a launch was
# attempted with FAKE pointers; the tests assert specific validation errors.


def test_compress_validation(L):
    f = L.kvarn_compress_tile
    vp = ctypes.c_void_p
    assert f(100, 1, 1, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE), None) == 2
    assert f(128, -1, 1, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE), None) == 1
    assert f(128, 1, 0, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE), None) == 1
    assert f(128, 1, 1, None, vp(FAKE), 128, 128, vp(FAKE), None) == 1
    assert f(128, 1, 1, vp(FAKE), vp(FAKE), 64, 128, vp(FAKE), None) == 1
    assert f(128, 1, 1, vp(FAKE + 4), vp(FAKE), 128, 128, vp(FAKE), None) == 3
    assert f(128, 1, 1, vp(FAKE), vp(FAKE), 130, 128, vp(FAKE), None) == 3
    assert f(128, 0, 1, None, None, 0, 0, None, None) == 0   # empty is a no-op
    F = 0x10000   # KVARN_SCALES_F16
    assert f(100 | F, 1, 1, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE), None) == 2
    assert f(128 | 0x40000, 1, 1, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE), None) == 2
    assert f(256 | F, 1, 1, vp(FAKE), vp(FAKE), 128, 256, vp(FAKE), None) == 1   # stride < 256
    assert f(128 | F, 1, 1, vp(FAKE), vp(FAKE), 128, 128, vp(FAKE + 8), None) == 3


def test_rotate_validation(L):
    f = L.kvarn_rotate_query
    vp = ctypes.c_void_p
    assert f(96, 4, vp(FAKE), vp(FAKE), None) == 2
    assert f(128, -2, vp(FAKE), vp(FAKE), None) == 1
    assert f(128, 4, None, vp(FAKE), None) == 1
    assert f(128, 4, vp(FAKE + 8), vp(FAKE), None) == 3
    assert f(128, 0, None, None, None) == 0


def _decode_args(**over):
    from quantized_attention_tok_amd.kvarn import DecodeArgs
    a = DecodeArgs()
    B = over.pop("batch", 1)
    nt = over.pop("n_tiles", [4] * B)
    nw = over.pop("n_win", [0] * B)
    rs = over.pop("rec_start", [0] * B)
    a.head_dim, a.batch, a.n_q_heads, a.n_kv_heads = 128, B, 4, 1
    a.softmax_scale = 0.1
    a.max_tiles, a.max_win = max(nt), max(nw)
    a.q = a.q_rot = a.out = a.records = a.k_win = a.v_win = FAKE
    a.n_record_rows = 4 * B
    a.win_tok_stride, a.win_head_stride, a.win_seq_stride = 128, 128, 128 * 128
    keep = [(ctypes.c_int32 * B)(*nt), (ctypes.c_int32 * B)(*nw), (ctypes.c_int64 * B)(*rs)]
    a.n_tiles, a.n_win, a.rec_start = keep
    for k, v in over.items():
        setattr(a, k, v)
    return a, keep


def test_decode_validation_and_workspace_query(L):
    a, keep = _decode_args()
    need = L.kvarn_decode_workspace_bytes(ctypes.byref(a))
    assert need > 0
    # too-small workspace is rejected before any launch
    assert L.kvarn_decode_attention(ctypes.byref(a), ctypes.c_void_p(FAKE), need - 16, None) == 4
    assert L.kvarn_decode_attention(ctypes.byref(a), None, need, None) == 4
    bad = [
        (dict(head_dim=100), 2), (dict(n_q_heads=6), 2), (dict(n_q_heads=48, n_kv_heads=3), 2),
        (dict(batch=65, n_tiles=[1] * 65, n_win=[0] * 65, rec_start=[0] * 65), 2),
        (dict(n_tiles=[0], n_win=[0]), 1),               # no visible key
        (dict(max_tiles=2), 1),                           # n_tiles > bound
        (dict(n_record_rows=3), 1),                       # tiles beyond the pool
        (dict(q=FAKE + 4), 3), (dict(win_tok_stride=130), 3),
        (dict(q_len=9), 1), (dict(q_len=-1), 1),          # verify width 0..8
        (dict(q_len=2, n_win=[1], max_win=1), 1),         # the drafts must be in the window
        (dict(q_len=2, head_dim=256, n_win=[4], max_win=4), 2),   # verify is head_dim 128
        (dict(head_dim=128 | 0x80000), 2),                # unknown format bit
        (dict(head_dim=128 | 0x10000, n_record_rows=3), 1),   # f16-scale records, same checks
        (dict(head_dim=128 | (6 << 20) | (5 << 24), q_rot=None), 1),   # vector path needs q_rot
        (dict(head_dim=128 | (6 << 20), q_len=2, n_win=[4], max_win=4), 2),   # verify is K4V2 only
        (dict(head_dim=128 | (9 << 20)), 2),             # key width above 8
        # the appended token: both rows, a single-query decode, a window that holds it
        (dict(k_new=FAKE, n_win=[4], max_win=4), 1),
        (dict(v_new=FAKE, n_win=[4], max_win=4), 1),
        (dict(k_new=FAKE, v_new=FAKE, n_win=[0]), 1),
        (dict(k_new=FAKE, v_new=FAKE, q_len=2, n_win=[4], max_win=4), 1),
        (dict(k_new=FAKE + 4, v_new=FAKE, n_win=[4], max_win=4), 3),
    ]
    for over, want in bad:
        b, k2 = _decode_args(**over)
        assert L.kvarn_decode_attention(ctypes.byref(b), ctypes.c_void_p(FAKE), 1 << 30, None) == want, over
        assert L.kvarn_decode_workspace_bytes(ctypes.byref(b)) == 0


def test_noalloc_decode_validation_before_any_device_call(L):
    """The no-allocation decode rejects what the workspace decode rejects, and
    a call whose partials exceed its scratch array, before it touches the
    device (this host has no GPU, so any device call would fail)."""
    from quantized_attention_tok_amd import kvarn
    m = re.search(r"#define\s+KVARN_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kvarn.NOALLOC_SCRATCH_BYTES
    for over, want in [(dict(head_dim=100), 2), (dict(n_tiles=[0], n_win=[0]), 1), (dict(q=FAKE + 4), 3),
                       (dict(max_tiles=2), 1), (dict(q_len=9), 1)]:
        b, k2 = _decode_args(**over)
        assert L.kvarn_decode_attention_noalloc(ctypes.byref(b), None) == want, over
    # 8 sequences of 4000 tiles at the 8B shape: far more partials than the array holds
    B = 8
    big, kb = _decode_args(head_dim=128, batch=B, n_q_heads=32, n_kv_heads=8, n_tiles=[4000] * B,
                           n_win=[0] * B, rec_start=[4000 * b for b in range(B)], max_tiles=4000,
                           n_record_rows=4000 * B)
    assert L.kvarn_decode_workspace_bytes(ctypes.byref(big)) > kvarn.NOALLOC_SCRATCH_BYTES
    assert L.kvarn_decode_attention_noalloc(ctypes.byref(big), None) == 4


def test_verify_workspace_grows_with_width(L):
    a1, k1 = _decode_args(n_win=[8], max_win=8)
    a4, k4 = _decode_args(n_win=[8], max_win=8, q_len=4)
    n1 = L.kvarn_decode_workspace_bytes(ctypes.byref(a1))
    n4 = L.kvarn_decode_workspace_bytes(ctypes.byref(a4))
    assert n1 > 0 and n4 > n1
    # the workgroups rotate the verify rows themselves when q_rot is absent
    a4r, k4r = _decode_args(n_win=[8], max_win=8, q_len=4, q_rot=None)
    assert L.kvarn_decode_workspace_bytes(ctypes.byref(a4r)) == n4


def test_prefill_validation(L):
    from quantized_attention_tok_amd.kvarn import PrefillArgs

    def args(**over):
        a = PrefillArgs()
        a.head_dim, a.n_q_heads, a.n_kv_heads, a.window = 128, 8, 2, 256
        a.pos0, a.chunk, a.softmax_scale = 512, 256, 0.1
        a.q = a.q_rot = a.out = a.records = a.k = a.v = FAKE
        a.n_record_rows = 4
        a.tok_stride, a.head_stride, a.raw_base = 256, 128, 256
        for k, v in over.items():
            setattr(a, k, v)
        return a
    a = args()
    # the matrix-core prefill at head_dim 128: 256 rows x 8 heads make 16
    # workgroups of 128 row-heads, so 4 splits (the most), each partial 128 + 4 floats
    need128 = L.kvarn_prefill_workspace_bytes(ctypes.byref(a))
    assert need128 == 256 * 8 * 4 * (128 + 4) * 4
    assert L.kvarn_prefill_attention(ctypes.byref(a), ctypes.c_void_p(FAKE), need128 - 16, None) == 4
    assert L.kvarn_prefill_attention(ctypes.byref(a), ctypes.c_void_p(FAKE + 8), need128, None) == 3
    # 2048 rows x 32 heads over 8 KV heads: 512 workgroups fill the CUs unsplit, no partials
    assert L.kvarn_prefill_workspace_bytes(ctypes.byref(args(chunk=2048, n_q_heads=32, n_kv_heads=8))) == 0
    # the K4V2 kernels rotate the rows themselves when no rotated query is given
    # (the splits are the same); the vector-unit paths of other code widths need
    # a workspace too
    assert L.kvarn_prefill_workspace_bytes(ctypes.byref(args(q_rot=None))) == need128
    assert L.kvarn_prefill_workspace_bytes(
        ctypes.byref(args(head_dim=256, q_rot=None, tok_stride=512, head_stride=256))) > 0
    assert L.kvarn_prefill_attention(
        ctypes.byref(args(head_dim=256 | (6 << 20) | (5 << 24), q_rot=None, tok_stride=512, head_stride=256)),
        ctypes.c_void_p(FAKE), 1 << 30, None) == 1
    # head_dim 256 over K4V2 records keeps the tile-split and window-part
    # partials in the workspace, (256 + 4) floats per row, head and split: here
    # 16 tile workgroups (8 row groups of 16 rows each) would need 16 splits to
    # fill the 256 CUs, capped at the 4 tiles the rows see (one tile each), and
    # 64 window workgroups take 4 parts (2 x 256 / 64 = 8, at most 4)
    a256 = args(head_dim=256, tok_stride=256 * 2, head_stride=256)
    need = L.kvarn_prefill_workspace_bytes(ctypes.byref(a256))
    assert need == 256 * 8 * (4 + 4) * (256 + 4) * 4
    # the last 512-row chunk of a 4096-token prompt at 16/4 heads: 64 tile
    # workgroups, so 4 splits of 8 of the 29 tiles, and 2 window parts
    a4k = args(head_dim=256, n_q_heads=16, n_kv_heads=4, pos0=3584, chunk=512, n_record_rows=30,
               raw_base=3328, tok_stride=1024, head_stride=256)
    assert L.kvarn_prefill_workspace_bytes(ctypes.byref(a4k)) == 512 * 16 * (4 + 2) * (256 + 4) * 4
    assert L.kvarn_prefill_attention(ctypes.byref(a256), ctypes.c_void_p(FAKE), need - 16, None) == 4
    assert L.kvarn_prefill_attention(ctypes.byref(a256), None, need, None) == 4
    # the f16-scale format does not change the workspace
    a256h = args(head_dim=256 | 0x10000, tok_stride=256 * 2, head_stride=256)
    assert L.kvarn_prefill_workspace_bytes(ctypes.byref(a256h)) == need
    # other code widths at head_dim 128 take the vector-unit path and its workspace
    aw = args(head_dim=128 | (6 << 20) | (5 << 24))
    assert L.kvarn_prefill_workspace_bytes(ctypes.byref(aw)) > 0
    assert L.kvarn_prefill_attention(ctypes.byref(aw), None, 1 << 30, None) == 4
    bad = [(dict(head_dim=384), 2), (dict(head_dim=128 | 0x20000), 2), (dict(chunk=0), 1),
           (dict(pos0=-1), 1),
           (dict(n_record_rows=3), 1), (dict(raw_base=384), 1), (dict(k=FAKE + 4), 3),
           (dict(tok_stride=258), 3), (dict(n_q_heads=6), 2)]
    for over, want in bad:
        b = args(**over)
        assert L.kvarn_prefill_attention(ctypes.byref(b), ctypes.c_void_p(FAKE), 1 << 30, None) == want, over
