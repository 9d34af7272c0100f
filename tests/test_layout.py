"""The quantised caches' tiled order (host helpers of the binding): a
permutation inside each 32-token block, and exactly the operand order the
decode kernel assumes (word i of lane l = bytes [1024 i + 16 l, +16) of a
block; lane l = 16 kb + ln; int4: 32-bit unit u of a lane at 4u in its
words, operand element 2m in nibble m and 2m+1 in nibble m+4)."""
import numpy as np
import pytest

from rank_compressed_kv_amd.layout import (i4_cache_offsets, i8_cache_offsets, pack_i4_cache,
                                           pack_i8_cache, unpack_i4_cache, unpack_i8_cache)


@pytest.mark.parametrize("r", [64, 128, 256])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_permutation_within_blocks(kind, r):
    off = i8_cache_offsets(kind, 96, r)
    assert sorted(off.ravel().tolist()) == list(range(96 * r))
    assert np.all(off // (32 * r) == np.arange(96)[:, None] // 32)
    c = np.random.default_rng(r).integers(-127, 128, size=(2, 3, 96, r)).astype(np.int8)
    assert np.array_equal(unpack_i8_cache(pack_i8_cache(c, kind), kind), c)


def _inverse(off):
    return {int(o): (t, k) for (t, k), o in np.ndenumerate(off)}


@pytest.mark.parametrize("r", [64, 128, 256])
def test_key_bytes_are_score_operands(r):
    """Half h, chunk c: lane (kb, ln) holds latents 32c + 8kb + j of token
    16h + ln in word h*r/64 + c/2, bytes 8*(c%2) + j."""
    inv = _inverse(i8_cache_offsets("k", 32, r))
    for h in range(2):
        for c in range(r // 32):
            for lane in range(64):
                ln, kb = lane % 16, lane // 16
                for j in range(8):
                    byte = 1024 * (h * (r // 64) + c // 2) + 16 * lane + 8 * (c % 2) + j
                    assert inv[byte] == (16 * h + ln, 32 * c + 8 * kb + j)


@pytest.mark.parametrize("r", [64, 128, 256])
def test_value_bytes_are_value_operands(r):
    """Row block rb: lane (kb, ln) holds latent 16rb + ln of tokens 4kb + j
    (j < 4) and 16 + 4kb + j - 4 in word rb/2, bytes 8*(rb%2) + j."""
    inv = _inverse(i8_cache_offsets("v", 32, r))
    for rb in range(r // 16):
        for lane in range(64):
            ln, kb = lane % 16, lane // 16
            for j in range(8):
                byte = 1024 * (rb // 2) + 16 * lane + 8 * (rb % 2) + j
                tok = 4 * kb + j if j < 4 else 16 + 4 * kb + j - 4
                assert inv[byte] == (tok, 16 * rb + ln)


def test_rejects_unsupported_shapes():
    with pytest.raises(ValueError):
        i8_cache_offsets("k", 100, 128)
    with pytest.raises(ValueError):
        i8_cache_offsets("v", 64, 96)
    with pytest.raises(ValueError):
        i8_cache_offsets("x", 64, 64)


# ------------------------------------------------------------------ int4 ---

def _unit_nibble(r, lane, u, e):
    """Nibble index (2 * byte + high) of operand element e of 32-bit unit u of
    lane l inside a block of 16 r bytes."""
    nib = e // 2 if e % 2 == 0 else 4 + e // 2
    byte = 1024 * (u // 4) + 16 * lane + 4 * (u % 4) + nib // 2
    return 2 * byte + nib % 2


def _inverse4(kind, r):
    off, nib = i4_cache_offsets(kind, 32, r)
    return {int(2 * o + n): (t, k) for ((t, k), o), n in zip(np.ndenumerate(off), nib.ravel())}


@pytest.mark.parametrize("r", [64, 128, 256])
@pytest.mark.parametrize("kind", ["k", "v"])
def test_int4_permutation_within_blocks(kind, r):
    off, nib = i4_cache_offsets(kind, 96, r)
    assert sorted((2 * off + nib).ravel().tolist()) == list(range(96 * r))
    assert np.all(off // (16 * r) == np.arange(96)[:, None] // 32)
    c = np.random.default_rng(r).integers(-7, 8, size=(2, 3, 96, r)).astype(np.int8)
    packed = pack_i4_cache(c, kind)
    assert packed.shape == (2, 3, 96, r // 2) and packed.dtype == np.uint8
    assert np.array_equal(unpack_i4_cache(packed, kind), c)


@pytest.mark.parametrize("r", [64, 128, 256])
def test_int4_key_nibbles_are_score_operands(r):
    """Half h, chunk c: lane (kb, ln) holds latents 32c + 8kb + e of token
    16h + ln as elements e of its unit h*r/32 + c."""
    inv = _inverse4("k", r)
    for h in range(2):
        for c in range(r // 32):
            for lane in range(64):
                ln, kb = lane % 16, lane // 16
                for e in range(8):
                    n = _unit_nibble(r, lane, h * (r // 32) + c, e)
                    assert inv[n] == (16 * h + ln, 32 * c + 8 * kb + e)


@pytest.mark.parametrize("r", [64, 128, 256])
def test_int4_value_nibbles_are_value_operands(r):
    """Row block rb: lane (kb, ln) holds latent 16rb + ln of tokens 4kb + e
    (e < 4) and 16 + 4kb + e - 4 as elements e of its unit rb."""
    inv = _inverse4("v", r)
    for rb in range(r // 16):
        for lane in range(64):
            ln, kb = lane % 16, lane // 16
            for e in range(8):
                tok = 4 * kb + e if e < 4 else 16 + 4 * kb + e - 4
                assert inv[_unit_nibble(r, lane, rb, e)] == (tok, 16 * rb + ln)


def test_int4_biased_nibbles_by_hand():
    """Codes are stored as code + 8: key latents 0 and 2 of token 0 share byte
    0 (low, high nibble), latents 1 and 3 byte 2; value tokens 0 and 2 share a
    byte."""
    c = np.zeros((32, 64), dtype=np.int8)
    c[0, 0], c[0, 1], c[0, 2], c[0, 3] = -7, 7, 1, -1
    k = pack_i4_cache(c, "k")
    flat = k.reshape(-1)
    assert flat[0] == (8 - 7) | ((8 + 1) << 4)
    assert flat[2] == (8 + 7) | ((8 - 1) << 4)
    off, nib = i4_cache_offsets("v", 32, 64)
    assert off[0, 5] == off[2, 5] and (nib[0, 5], nib[2, 5]) == (0, 1)
    with pytest.raises(ValueError):
        pack_i4_cache(np.full((32, 64), 9), "k")
