"""The seeded generator: determinism, shapes, the bf16 rounding of draws and the
distributions the workloads state."""
import numpy as np
import pytest

import workloads as W


def test_bf16_rounding_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 3 * 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    bits = W.f32_to_bf16_bits(f)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xBF82, 0x3F81]
    back = W.bf16_bits_to_f32(bits)
    assert back.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -(1.0 + 2 ** -6), 1.0 + 2 ** -7]


def test_deterministic_and_independent_streams():
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=64)
    a = W.generate(cfg)
    b = W.generate(cfg)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    # drawing the append tensors does not change the decode tensors
    c = W.generate(cfg, parts=("decode", "append"))
    np.testing.assert_array_equal(a["h_k"], c["h_k"])
    assert not np.array_equal(a["h_k"], a["h_v"])


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_shapes_and_dtypes(idx):
    cfg = W.CONFIGS[idx]
    small = cfg.scaled(batch=min(cfg.batch, 2), max_ctx=96,
                       ragged=(1, 96) if cfg.ragged else None)
    t = W.generate(small, parts=("decode", "append"))
    B, Hq, d, G, r = small.batch, small.n_q_heads, small.head_dim, small.n_groups, small.rank
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    assert t["q"].shape == (B, Hq, d) and t["q"].dtype == st
    assert t["h_k"].shape == (B, G, 96, r) and t["h_v"].dtype == st
    assert t["b_k"].shape == (G, r, small.group_dim)
    assert t["x"].shape == (B, small.d_model) and t["a_k"].shape == (small.d_model, G * r)
    assert t["lens"].dtype == np.int32 and t["lens"].shape == (B,)
    assert t["pos"].min() >= 0 and t["pos"].max() < 96


def test_distributions():
    cfg = W.CONFIGS[3].scaled(batch=1, max_ctx=4096)
    t = W.generate(cfg)
    h = W.bf16_bits_to_f32(t["h_k"])
    assert abs(h.mean()) < 0.01 and abs(h.std() - 1) < 0.01
    bk = W.bf16_bits_to_f32(t["b_k"])
    assert abs(bk.var() * cfg.rank - 1) < 0.02


def test_outlier_channels_and_ragged_lengths():
    cfg = W.CONFIGS[4].scaled(max_ctx=2048)
    t = W.generate(cfg)
    h = W.bf16_bits_to_f32(t["h_k"])[0]                 # [G, L, r]
    col_std = h.std(axis=1).reshape(-1)
    big = np.sort(col_std)[::-1]
    assert np.sum(col_std > 5) == round(0.01 * cfg.n_groups * cfg.rank) == 3
    assert 15 < big[0] < 25
    c5 = W.CONFIGS[5].scaled(rank=8)       # small rank: only the lengths matter here
    lens = W.generate(c5)["lens"]
    assert lens.shape == (32,) and lens.min() >= 1024 and lens.max() <= 16384
    assert len(set(lens.tolist())) > 20


def test_poison_tail():
    h = np.zeros((2, 1, 5, 3), dtype=np.uint16)
    p = W.poison_tail(h, np.array([2, 5]))
    assert np.all(p[0, :, 2:] == 0x7FC0) and np.all(p[0, :, :2] == 0) and np.all(p[1] == 0)


def test_lens_validation():
    cfg = W.CONFIGS[1]
    with pytest.raises(ValueError):
        W.generate(cfg, lens=np.array([cfg.max_ctx + 1]))
