"""GPU parity of the int8 latent cache (per-token codes with one fp32 scale
per cached row) in absorbed mode: the HIP path through palu_decode_attn_i8
against the fp64 oracle on the dequantised cache (code * scale, exact), to
the bf16 bar (max |d| <= 2e-2, relative L2 <= 5e-3)."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from tests.parity_util import assert_close, dev

pytestmark = pytest.mark.gpu

SMALL = {
    2: W.CONFIGS[2].scaled(batch=2, max_ctx=1000),            # MHA, 4 q heads per group, r 256
    3: W.CONFIGS[3].scaled(batch=2, max_ctx=1500),            # GQA, 16 q heads per group, r 256
    4: W.CONFIGS[4].scaled(max_ctx=3000),                     # r 128
    64: W.CONFIGS[3].scaled(n_groups=4, rank=64, batch=2, max_ctx=700, seed=71),   # r 64
    48: W.CONFIGS[3].scaled(n_kv_heads=24, n_q_heads=48, n_groups=4, rank=128, batch=1,
                            max_ctx=900, seed=72),            # 12 q heads: a partial head slice
}


def _run(cfg, t, *, split_tokens=0, q=None, sk=None, sv=None, latent_out=False, lens=True):
    import torch
    import rank_compressed_kv_amd as P
    out = P.decode_attention_i8(
        dev(t["q"] if q is None else q), dev(t["k_i8"]), dev(t["v_i8"]),
        dev(t["sk"] if sk is None else sk), dev(t["sv"] if sv is None else sv),
        dev(t["b_k"]), None if latent_out else dev(t["b_v"]),
        dev(t["lens"]) if lens else None, n_kv_heads=cfg.n_kv_heads,
        split_tokens=split_tokens, latent_out=latent_out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _want(t, *, q=None, sk=None, sv=None):
    hk = O.dequantize_rows_i8(t["k_i8"], t["sk"] if sk is None else sk)
    hv = O.dequantize_rows_i8(t["v_i8"], t["sv"] if sv is None else sv)
    return O.decode_attention(t["q"] if q is None else q, hk, hv, t["b_k"], t["b_v"], t["lens"])


@pytest.mark.parametrize("idx", sorted(SMALL))
@pytest.mark.parametrize("split_tokens", [0, 64, 192])
def test_int8_decode_parity(idx, split_tokens):
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "i8"))
    print(f"[int8] cfg{idx} split={split_tokens} lens={t['lens'].tolist()}", flush=True)
    assert_close(_run(cfg, t, split_tokens=split_tokens), _want(t), what=f"int8 cfg{idx}")


def test_int8_length_edges_and_poisoned_scales():
    """Lengths 0, 1, around the split size and the capacity; the scales of rows
    past each length are NaN, so any read beyond the context shows up."""
    L = 640
    edge = [0, 1, 63, 64, 65, 129, 511, L]
    cfg = SMALL[3].scaled(batch=len(edge), max_ctx=L, ragged=None)
    t = W.generate(cfg, parts=("decode", "i8"), lens=np.array(edge))
    sk, sv = t["sk"].copy(), t["sv"].copy()
    for b, n in enumerate(edge):
        sk[b, :, n:] = np.nan
        sv[b, :, n:] = np.nan
    want = _want(t)
    for st in (64, 128, 0):
        print(f"[int8 edges] split={st}", flush=True)
        got = _run(cfg, t, split_tokens=st, sk=sk, sv=sv)
        assert np.all(got[0] == 0.0)
        assert_close(got, want, what=f"int8 edges split{st}")


def test_int8_operand_range():
    """Query entries far beyond fp16's range (q * 2^16) with key scales * 2^-16
    (same scores) and value scales * 2^-20: the kernel's fp16 operands stay in
    range. Compared after undoing the 2^-20 on both sides."""
    cfg = SMALL[3]
    t = W.generate(cfg, parts=("decode", "i8"))
    q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(t["q"]) * np.float32(2.0 ** 16))
    sk = (t["sk"] * np.float32(2.0 ** -16)).astype(np.float32)
    sv = (t["sv"] * np.float32(2.0 ** -20)).astype(np.float32)
    got = _run(cfg, t, q=q, sk=sk, sv=sv) * 2.0 ** 20
    want = _want(t, q=q, sk=sk, sv=sv) * 2.0 ** 20
    assert_close(got, want, what="int8 operand range")
    # the same scores as the unscaled cache: the output only carries the 2^-20
    assert_close(got, _want(t), what="int8 scaled vs unscaled")


def test_int8_zero_scale_rows():
    """Rows quantised from all-zero latents have scale 0 (and codes 0): they
    score 0 and add nothing to the value sum."""
    cfg = SMALL[64]
    t = W.generate(cfg, parts=("decode", "i8"))
    sk, sv = t["sk"].copy(), t["sv"].copy()
    sk[:, :, ::7] = 0.0
    sv[:, :, ::5] = 0.0
    sv[0, 0, :] = 0.0          # a whole (b, g) of zero values: output 0 for its heads
    got = _run(cfg, t, sk=sk, sv=sv, split_tokens=128)
    assert_close(got, _want(t, sk=sk, sv=sv), what="int8 zero scales")


def test_int8_latent_output():
    """latent_out with int8 latents: u* [B, Hq, r], B_v never read."""
    cfg = SMALL[3]
    t = W.generate(cfg, parts=("decode", "i8"))
    hk = O.dequantize_rows_i8(t["k_i8"], t["sk"])
    hv = O.dequantize_rows_i8(t["v_i8"], t["sv"])
    want = O.decode_value_latents(t["q"], hk, hv, t["b_k"], t["lens"], cfg.group_dim)
    for st in (0, 64):
        got = _run(cfg, t, split_tokens=st, latent_out=True)
        assert got.shape == (cfg.batch, cfg.n_q_heads, cfg.rank)
        assert_close(got, want, what=f"int8 u* split{st}")


def test_int8_matches_bf16_path_on_exact_cache():
    """Codes times power-of-two scales are exact in bf16: the bf16 decode on
    that cache and the int8 decode compute the same attention."""
    import rank_compressed_kv_amd as P
    cfg = SMALL[4]
    t = W.generate(cfg, parts=("decode", "i8"))
    sk = np.full_like(t["sk"], 2.0 ** -7)
    sv = np.full_like(t["sv"], 2.0 ** -6)
    hk = W.f32_to_bf16_bits((t["k_i8"].astype(np.float32) * sk[..., None]).astype(np.float32))
    hv = W.f32_to_bf16_bits((t["v_i8"].astype(np.float32) * sv[..., None]).astype(np.float32))
    a = _run(cfg, t, sk=sk, sv=sv)
    import torch
    b = P.decode_attention(dev(t["q"]), dev(hk), dev(hv), dev(t["b_k"]), dev(t["b_v"]),
                           dev(t["lens"]), n_kv_heads=cfg.n_kv_heads, mode="absorbed")
    torch.cuda.synchronize()
    assert_close(a, b.cpu().numpy().astype(np.float64), max_abs=2e-3, rel_l2=5e-4,
                 what="int8 vs bf16 path")
