"""KVarN KV-cache hot path for AMD Instinct MI355X (gfx950).

The computation lives in libkvarn.so (HIP kernels behind the C ABI of
include/kvarn.h); this package is its Python binding plus the host-side
window/promotion bookkeeping of one sequence.
"""
from .kvarn import (KVarNError, compress_tile, decode_attention, decode_workspace_bytes,
                    lib, prefill_attention, rotate_query, tile_bytes, visible_tiles)
from .cache import SequenceCache

__all__ = ["KVarNError", "SequenceCache", "compress_tile", "decode_attention",
           "decode_workspace_bytes", "lib", "prefill_attention", "rotate_query", "tile_bytes",
           "visible_tiles"]
