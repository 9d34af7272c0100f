"""Host-side view of the int8 latent cache's tiled byte order.

palu_latent_append_i8 writes, and palu_decode_attn_i8 reads, each (b, g)
slab of an int8 cache [B, G, L_cap, r] (L_cap a multiple of 32, r in
{64, 128, 256}) as a run of 32-token blocks whose bytes are ordered the way
the decode kernel's matrix-core operands are laid out; include/palu.h gives
the order. These helpers permute host arrays between that order and plain
row order ([t, k] = latent k of token t), e.g. to bring an existing cache in
or to inspect one; they move bytes only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["i8_cache_offsets", "pack_i8_cache", "unpack_i8_cache"]


def i8_cache_offsets(kind: str, max_ctx: int, rank: int) -> np.ndarray:
    """Byte offset [max_ctx, rank] of latent (t, k) inside one (b, g) slab.
    kind: "k" (key latents) or "v" (value latents)."""
    if max_ctx % 32 or rank not in (64, 128, 256):
        raise ValueError("the int8 cache needs max_ctx % 32 == 0 and rank in {64, 128, 256}")
    t = np.arange(max_ctx, dtype=np.int64)[:, None]
    k = np.arange(rank, dtype=np.int64)[None, :]
    block = (t // 32) * 32 * rank
    if kind == "k":
        return (block + ((t % 32) // 16) * 16 * rank + (k // 64) * 1024 + ((k % 32) // 8) * 256
                + (t % 16) * 16 + ((k // 32) % 2) * 8 + k % 8)
    if kind == "v":
        return (block + (k // 32) * 1024 + ((t % 16) // 4) * 256 + (k % 16) * 16
                + ((k // 16) % 2) * 8 + ((t % 32) // 16) * 4 + t % 4)
    raise ValueError('kind must be "k" or "v"')


def pack_i8_cache(codes: np.ndarray, kind: str) -> np.ndarray:
    """Row-order codes [..., L, r] -> the same bytes in the cache's order."""
    *lead, L, r = codes.shape
    off = i8_cache_offsets(kind, L, r).ravel()
    flat = np.asarray(codes).reshape(-1, L * r)
    out = np.empty_like(flat)
    out[:, off] = flat
    return out.reshape(codes.shape)


def unpack_i8_cache(tiled: np.ndarray, kind: str) -> np.ndarray:
    """The cache's order [..., L, r] -> row-order codes."""
    *lead, L, r = tiled.shape
    off = i8_cache_offsets(kind, L, r).ravel()
    return np.asarray(tiled).reshape(-1, L * r)[:, off].reshape(tiled.shape)
