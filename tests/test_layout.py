"""The int8 cache's tiled byte order (host helpers of the binding): a
permutation inside each 32-token block, and exactly the operand order the
decode kernel assumes (word i of lane l = bytes [1024 i + 16 l, +16) of a
block; lane l = 16 kb + ln)."""
import numpy as np
import pytest

from rank_compressed_kv_amd.layout import i8_cache_offsets, pack_i8_cache, unpack_i8_cache


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
