"""Host-side views of the pool-cache layout.

The pooled keys [B, P_max, D] live in the library's tile-interleaved pool cache
(include/dsa.h, dsa_kpool_compress): pools grouped in tiles of 16, and within a
tile the 16-byte pieces of the 16 pools stored piece-major.  These helpers
convert between that layout and row-major keys for callers that bring their
own keys or inspect the cache.  They only move data (torch views and copies).
"""
from __future__ import annotations

import torch


def pool_cache_pools(P_max: int) -> int:
    """Pools per sequence held by the pool cache: P_max rounded up to whole tiles."""
    return 16 * ((P_max + 15) // 16)


def tile_pool_cache(x: torch.Tensor) -> torch.Tensor:
    """Row-major keys [B, P, D] -> pool cache [B, pool_cache_pools(P), D] (padding pools zero)."""
    B, P, D = x.shape
    E = 16 // x.element_size()
    Pt = (P + 15) // 16
    pad = torch.zeros((B, Pt * 16, D), dtype=x.dtype, device=x.device)
    pad[:, :P] = x
    return pad.view(B, Pt, 16, D // E, E).permute(0, 1, 3, 2, 4).contiguous().view(B, Pt * 16, D)


def untile_pool_cache(t: torch.Tensor, P: int) -> torch.Tensor:
    """Pool cache [B, 16*Pt, D] -> the first P pools as row-major keys [B, P, D]."""
    B, Pp, D = t.shape
    E = 16 // t.element_size()
    Pt = Pp // 16
    return t.reshape(B, Pt, D // E, 16, E).permute(0, 1, 3, 2, 4).reshape(B, Pt * 16, D)[:, :P]
