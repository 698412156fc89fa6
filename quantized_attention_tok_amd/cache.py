"""Host bookkeeping of one sequence's KVarN cache.

Raw K/V rows are appended to a device buffer; the newest tokens form the FP32
window and, whenever the window reaches W + 128 tokens, its oldest 128 are
compressed into the next tile record (SharpInference PR #434 commit list: the
FP32 window is the staging area, with whole-tile promotion).  Compression runs
in the HIP kernel; this class only tracks counts and buffer views.
"""
from __future__ import annotations

import torch

from . import kvarn

TILE = 128


class SequenceCache:
    def __init__(self, n_kv: int, head_dim: int, window: int, capacity: int,
                 device: str | torch.device = "cuda", f16_scales: bool = False,
                 kbits: int = 4, vbits: int = 2):
        self.n_kv, self.d, self.window = n_kv, head_dim, window
        self.f16_scales, self.kbits, self.vbits = f16_scales, kbits, vbits
        self.k = torch.empty(capacity, n_kv, head_dim, dtype=torch.float32, device=device)
        self.v = torch.empty_like(self.k)
        self.records = torch.empty(capacity // TILE + 1, n_kv, kvarn.tile_bytes(head_dim, f16_scales, kbits, vbits),
                                   dtype=torch.uint8, device=device)
        self.n_tokens = 0
        self.n_tiles = 0

    @property
    def n_win(self) -> int:
        return self.n_tokens - TILE * self.n_tiles

    def window_views(self):
        """Raw window rows [128*n_tiles, n_tokens) as [n_win][n_kv][d] views."""
        lo = TILE * self.n_tiles
        return self.k[lo:self.n_tokens], self.v[lo:self.n_tokens]

    def append(self, k_rows: torch.Tensor, v_rows: torch.Tensor, stream=None) -> int:
        """Append [n][n_kv][d] rows and promote every tile that becomes due.
        Returns the number of tiles compressed."""
        n = k_rows.shape[0]
        if self.n_tokens + n > self.k.shape[0]:
            raise ValueError("sequence cache capacity exceeded")
        self.k[self.n_tokens:self.n_tokens + n] = k_rows
        self.v[self.n_tokens:self.n_tokens + n] = v_rows
        self.n_tokens += n
        due = kvarn.visible_tiles(self.n_tokens - 1, self.window)
        new = due - self.n_tiles
        if new > 0:
            lo = TILE * self.n_tiles
            kvarn.compress_tile(self.k[lo:], self.v[lo:], self.records[self.n_tiles:], new,
                                stream=stream, f16_scales=self.f16_scales, kbits=self.kbits,
                                vbits=self.vbits)
            self.n_tiles = due
        return max(new, 0)
