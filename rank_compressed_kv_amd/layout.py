"""Host-side view of the quantised latent caches' tiled order.

palu_latent_append_i8 writes, and palu_decode_attn_i8 reads, each (b, g)
slab of an int8 cache [B, G, L_cap, r] (L_cap a multiple of 32, r in
{64, 128, 256}) as a run of 32-token blocks whose bytes are ordered the way
the decode kernel's matrix-core operands are laid out; the int4 cache
[B, G, L_cap, r/2] holds two biased codes (code + 8) a byte in the int4
calls' nibble order. include/palu.h gives both orders. These helpers permute
host arrays between that order and plain row order ([t, k] = latent k of
token t), e.g. to bring an existing cache in or to inspect one; they move
codes only.
"""
from __future__ import annotations

import numpy as np

__all__ = ["i8_cache_offsets", "pack_i8_cache", "unpack_i8_cache", "i4_cache_offsets",
           "pack_i4_cache", "unpack_i4_cache"]


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


def i4_cache_offsets(kind: str, max_ctx: int, rank: int):
    """(byte offset, nibble) [max_ctx, rank] of latent (t, k) inside one (b, g)
    slab of L_cap*r/2 bytes; nibble 1 is the byte's high half."""
    if max_ctx % 32 or rank not in (64, 128, 256):
        raise ValueError("the int4 cache needs max_ctx % 32 == 0 and rank in {64, 128, 256}")
    t = np.arange(max_ctx, dtype=np.int64)[:, None]
    k = np.arange(rank, dtype=np.int64)[None, :]
    if kind == "k":
        u = (rank // 32) * ((t % 32) // 16) + k // 32
        lane = 16 * ((k % 32) // 8) + t % 16
        e = (k % 8) // 4 + 2 * (k % 2)
        nib = (k // 2) % 2
    elif kind == "v":
        u = k // 16
        lane = 16 * ((t % 16) // 4) + k % 16
        e = (t % 32) // 16 + 2 * (t % 2)
        nib = (t % 4) // 2
    else:
        raise ValueError('kind must be "k" or "v"')
    off = 16 * rank * (t // 32) + 1024 * (u // 4) + 16 * lane + 4 * (u % 4) + e
    shape = (max_ctx, rank)
    return np.broadcast_to(off, shape).copy(), np.broadcast_to(nib, shape).copy()


def pack_i4_cache(codes: np.ndarray, kind: str) -> np.ndarray:
    """Row-order codes [..., L, r] in [-7, 7] -> uint8 [..., L, r/2] in the
    cache's order."""
    *lead, L, r = codes.shape
    c = np.asarray(codes).astype(np.int64)
    if c.min(initial=0) < -8 or c.max(initial=0) > 7:
        raise ValueError("int4 codes must lie in [-8, 7]")
    off, nib = i4_cache_offsets(kind, L, r)
    off, nib = off.ravel(), nib.ravel()
    flat = (c.reshape(-1, L * r) + 8).astype(np.uint8)
    out = np.zeros((flat.shape[0], L * r // 2), dtype=np.uint8)
    lo, hi = nib == 0, nib == 1
    out[:, off[lo]] |= flat[:, lo]
    out[:, off[hi]] |= flat[:, hi] << 4
    return out.reshape(*lead, L, r // 2)


def unpack_i4_cache(tiled: np.ndarray, kind: str) -> np.ndarray:
    """The cache's order uint8 [..., L, r/2] -> row-order int8 codes [..., L, r]."""
    *lead, L, rh = tiled.shape
    r = 2 * rh
    off, nib = i4_cache_offsets(kind, L, r)
    b = np.asarray(tiled).reshape(-1, L * rh)[:, off.ravel()]
    n = (b >> (4 * nib.ravel()).astype(np.uint8)) & 0xF
    return (n.astype(np.int16) - 8).astype(np.int8).reshape(*lead, L, r)
