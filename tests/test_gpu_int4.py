"""GPU parity of the int4 latent cache (per-token 4-bit codes in [-7, 7] with
one fp32 scale per cached row) in absorbed mode: the HIP path through
palu_decode_attn_i4 / palu_latent_append_i4 against the fp64 oracle on the
dequantised cache (code * scale, exact), to the bf16 bar (max |d| <= 2e-2,
relative L2 <= 5e-3). The seeded codes are in row order; the device cache
holds them two a byte in the library's tiled nibble order."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache, unpack_i4_cache
from tests.parity_util import assert_close, code_bounds, dev

pytestmark = pytest.mark.gpu

SMALL = {
    2: W.CONFIGS[2].scaled(batch=2, max_ctx=1024),            # MHA, 4 q heads per group, r 256
    3: W.CONFIGS[3].scaled(batch=2, max_ctx=1504),            # GQA, 16 q heads per group, r 256
    4: W.CONFIGS[4].scaled(max_ctx=3008),                     # r 128
    64: W.CONFIGS[3].scaled(n_groups=4, rank=64, batch=2, max_ctx=704, seed=71),   # r 64
    48: W.CONFIGS[3].scaled(n_kv_heads=24, n_q_heads=48, n_groups=4, rank=128, batch=1,
                            max_ctx=896, seed=72),            # 12 q heads: a partial head slice
    32: W.CONFIGS[3].scaled(n_groups=1, rank=256, batch=2, max_ctx=704, seed=73),   # 32 q heads a group
}

APPEND = {
    "r256_g2": W.CONFIGS[3].scaled(batch=4, max_ctx=64, ragged=None),       # a row is a block
    "r256_b9": W.CONFIGS[3].scaled(batch=9, max_ctx=32, ragged=None, seed=83),   # two rounds of rows
    "r128_b12": W.CONFIGS[4].scaled(batch=12, max_ctx=32, ragged=None, seed=84),
    "r256_g8": W.CONFIGS[2].scaled(batch=3, max_ctx=32, ragged=None),
    "r128": W.CONFIGS[4].scaled(max_ctx=64, ragged=None),
    "r64": W.CONFIGS[3].scaled(n_groups=4, rank=64, batch=2, max_ctx=32, seed=81),
    "r64_f32": W.CONFIGS[1].scaled(rank=64, batch=3, max_ctx=32, ragged=None),      # fp32 inputs
}


def _cache(t, kind):
    return dev(pack_i4_cache(t[f"{kind}_i4"], kind))


def _run(cfg, t, *, split_tokens=0, q=None, sk=None, sv=None, latent_out=False, lens=None,
         hadamard=False, caches=None):
    import torch
    import rank_compressed_kv_amd as P
    hk, hv = caches if caches is not None else (_cache(t, "k"), _cache(t, "v"))
    out = P.decode_attention_i4(
        dev(t["q"] if q is None else q), hk, hv,
        dev(t["sk_i4"] if sk is None else sk), dev(t["sv_i4"] if sv is None else sv),
        dev(t["b_k"]), None if latent_out else dev(t["b_v"]),
        dev(t["lens"] if lens is None else lens), n_kv_heads=cfg.n_kv_heads,
        split_tokens=split_tokens, latent_out=latent_out, hadamard=hadamard)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _rows(t, *, sk=None, sv=None, rot=False):
    deq = O.dequantize_rows_i8_hadamard if rot else O.dequantize_rows_i8
    return (deq(t["k_i4"], t["sk_i4"] if sk is None else sk),
            deq(t["v_i4"], t["sv_i4"] if sv is None else sv))


def _want(t, *, q=None, sk=None, sv=None, rot=False, lens=None):
    hk, hv = _rows(t, sk=sk, sv=sv, rot=rot)
    return O.decode_attention(t["q"] if q is None else q, hk, hv, t["b_k"], t["b_v"],
                              t["lens"] if lens is None else lens)


@pytest.mark.parametrize("idx", sorted(SMALL))
@pytest.mark.parametrize("split_tokens", [0, 64, 192])
def test_int4_decode_parity(idx, split_tokens):
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "i4"))
    print(f"[int4] cfg{idx} split={split_tokens} lens={t['lens'].tolist()}", flush=True)
    assert_close(_run(cfg, t, split_tokens=split_tokens), _want(t), what=f"int4 cfg{idx}")


def test_int4_length_edges_and_poisoned_scales():
    """Lengths 0, 1, around the split size and the capacity; the scales of rows
    past each length are NaN, so any read beyond the context shows up."""
    L = 640
    edge = [0, 1, 63, 64, 65, 129, 511, L]
    cfg = SMALL[3].scaled(batch=len(edge), max_ctx=L, ragged=None)
    t = W.generate(cfg, parts=("decode", "i4"), lens=np.array(edge))
    sk, sv = t["sk_i4"].copy(), t["sv_i4"].copy()
    for b, n in enumerate(edge):
        sk[b, :, n:] = np.nan
        sv[b, :, n:] = np.nan
    want = _want(t)
    for st in (64, 128, 0):
        print(f"[int4 edges] split={st}", flush=True)
        got = _run(cfg, t, split_tokens=st, sk=sk, sv=sv)
        assert np.all(got[0] == 0.0)
        assert_close(got, want, what=f"int4 edges split{st}")


def test_int4_operand_range():
    """Query entries far beyond fp16's range (q * 2^16) with key scales * 2^-16
    (same scores) and value scales * 2^-20: the kernel's fp16 operands stay in
    range. Compared after undoing the 2^-20 on both sides."""
    cfg = SMALL[64]
    t = W.generate(cfg, parts=("decode", "i4"))
    q = W.f32_to_bf16_bits(W.bf16_bits_to_f32(t["q"]) * np.float32(2.0 ** 16))
    sk = (t["sk_i4"] * np.float32(2.0 ** -16)).astype(np.float32)
    sv = (t["sv_i4"] * np.float32(2.0 ** -20)).astype(np.float32)
    got = _run(cfg, t, q=q, sk=sk, sv=sv) * 2.0 ** 20
    assert_close(got, _want(t, q=q, sk=sk, sv=sv) * 2.0 ** 20, what="int4 operand range")
    assert_close(got, _want(t), what="int4 scaled vs unscaled")


def test_int4_zero_scale_rows():
    """Rows quantised from all-zero latents (scale 0): they score 0 and add
    nothing to the value sum."""
    cfg = SMALL[64]
    t = W.generate(cfg, parts=("decode", "i4"))
    sk, sv = t["sk_i4"].copy(), t["sv_i4"].copy()
    sk[:, :, ::7] = 0.0
    sv[:, :, ::5] = 0.0
    sv[0, 0, :] = 0.0
    got = _run(cfg, t, sk=sk, sv=sv, split_tokens=128)
    assert_close(got, _want(t, sk=sk, sv=sv), what="int4 zero scales")


def test_int4_latent_output():
    """latent_out with int4 latents: u* [B, Hq, r], B_v never read."""
    cfg = SMALL[4]
    t = W.generate(cfg, parts=("decode", "i4"))
    hk, hv = _rows(t)
    want = O.decode_value_latents(t["q"], hk, hv, t["b_k"], t["lens"], cfg.group_dim)
    for st in (0, 64):
        got = _run(cfg, t, split_tokens=st, latent_out=True)
        assert got.shape == (cfg.batch, cfg.n_q_heads, cfg.rank)
        assert_close(got, want, what=f"int4 u* split{st}")


@pytest.mark.parametrize("idx", [3, 64])
def test_int4_matches_int8_on_the_same_codes(idx):
    """Codes in [-7, 7] are also int8 codes: the int8 decode on them (same
    scales, the same fp16 q~ and weights) computes the same attention; the two
    differ only in the rounding of the fp32 score accumulators, which sum r
    products q~_k (code_k + bias) with bias 128 or 8, the bias term being taken
    back in fp32: with r = 256 and |code| <= 7 the int8 sums run about 20
    times larger than the scores, so each score carries a relative rounding
    error of order 20 * sqrt(r) * 2^-24 ~ 2e-5, and the outputs a few 1e-5."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "i4"))
    a = _run(cfg, t, split_tokens=64)
    b = P.decode_attention_i8(dev(t["q"]), dev(pack_i8_cache(t["k_i4"], "k")),
                              dev(pack_i8_cache(t["v_i4"], "v")), dev(t["sk_i4"]),
                              dev(t["sv_i4"]), dev(t["b_k"]), dev(t["b_v"]), dev(t["lens"]),
                              n_kv_heads=cfg.n_kv_heads, split_tokens=64)
    torch.cuda.synchronize()
    b = b.cpu().numpy().astype(np.float64)
    print(f"[int4 vs int8] cfg{idx} max|d|={np.max(np.abs(a - b)):.3e}", flush=True)
    assert_close(a, b, max_abs=2e-4, rel_l2=1e-4, what="int4 vs int8")


@pytest.mark.parametrize("idx", [3, 4, 64])
def test_int4_hadamard_decode_parity(idx):
    """A rotated int4 cache: compared with the oracle on (code*scale) H_r / r."""
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "i4"))
    print(f"[int4 hadamard] cfg{idx}", flush=True)
    assert_close(_run(cfg, t, hadamard=True), _want(t, rot=True), what=f"int4 rot cfg{idx}")


# ------------------------------------------------------ quantised cache write ---

def _check_rows(cfg, t, x, hk, hv, sk, sv, before, *, rot=False, zero_row=False):
    """Codes and scales at pos[b] equal the oracle's except within the fp32
    error bound of a decision boundary (and then by one step at most); every
    other code and scale is unchanged."""
    G, r, dm = cfg.n_groups, cfg.rank, cfg.d_model
    H = O.hadamard(r)
    mism = tot = 0
    for kind, codes_d, scales_d, a in (("k", hk, sk, t["a_k"]), ("v", hv, sv, t["a_v"])):
        codes, scales = unpack_i4_cache(codes_d.cpu().numpy(), kind), scales_d.cpu().numpy()
        h64 = O.latent_project(x, a).reshape(cfg.batch, G, r)
        E = (np.abs(O.to_f64(x))[:, :, None] * np.abs(O.to_f64(a))[None]).sum(1)
        E = E.reshape(cfg.batch, G, r) * dm * 2.0 ** -24
        for b, pos in enumerate(t["pos"]):
            wc, ws = (O.append_rows_i4_hadamard if rot else O.append_rows_i4)(h64[b])
            gc, gs = codes[b, :, pos, :].astype(np.int64), scales[b, :, pos]
            if zero_row and b == 0:
                assert np.all(gc == 0) and np.all(gs == 0.0)
                continue
            mism += int(np.sum(gc != wc))
            tot += gc.size
            for g in range(G):
                if rot:
                    e = h64[b, g] @ H
                    eb = 1.5 * (E[b, g].sum() + np.log2(r) * 2.0 ** -24 *
                                np.sum(np.abs(h64[b, g]) + E[b, g]))
                    amax_lo = max(float(np.max(np.abs(e)) - eb), 0.0)
                    amax_hi = float(np.max(np.abs(e)) + eb)
                else:
                    e, eb = h64[b, g], E[b, g]
                    amax_lo = max(float(np.max(np.abs(e) - eb)), 0.0)
                    amax_hi = float(np.max(np.abs(e) + eb))
                assert amax_lo / 7 * (1 - 2.0 ** -23) <= gs[g] <= amax_hi / 7 * (1 + 2.0 ** -23)
                if np.all(gc[g] == wc[g]):
                    continue
                lo, hi = code_bounds(e, eb, amax_lo, amax_hi, 7)
                assert np.all((gc[g] >= lo) & (gc[g] <= hi)), (b, g)
                assert np.max(np.abs(gc[g] - wc[g])) <= 1
    assert mism <= 0.01 * tot
    for i, (got, old) in enumerate(zip((hk, hv, sk, sv), before)):
        g, o = got.cpu().numpy(), old.cpu().numpy()
        if i < 2:
            g, o = unpack_i4_cache(g, "kv"[i]), unpack_i4_cache(o, "kv"[i])
        g, o = g.copy(), o.copy()
        for b, pos in enumerate(t["pos"]):
            g[b, :, int(pos)] = 0
            o[b, :, int(pos)] = 0
        assert np.array_equal(g, o)


@pytest.mark.parametrize("name", sorted(APPEND))
def test_int4_append(name):
    """h = x A quantised per row to 4 bits; a zero x row stores scale 0 and
    codes 0; the other token sharing each value byte keeps its code."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = APPEND[name]
    t = W.generate(cfg, parts=("decode", "append", "i4"))
    x = t["x"].copy()
    x[0] = 0
    hk, hv = _cache(t, "k"), _cache(t, "v")
    sk, sv = dev(t["sk_i4"]), dev(t["sv_i4"])
    before = [c.clone() for c in (hk, hv, sk, sv)]
    print(f"[int4 append] {name} pos={t['pos'].tolist()}", flush=True)
    P.latent_append_i4(dev(x), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv, dev(t["pos"]))
    torch.cuda.synchronize()
    _check_rows(cfg, t, x, hk, hv, sk, sv, before, zero_row=True)


@pytest.mark.parametrize("name", ["r256_g2", "r128", "r64_f32"])
def test_int4_hadamard_append(name):
    import torch
    import rank_compressed_kv_amd as P
    cfg = APPEND[name]
    t = W.generate(cfg, parts=("decode", "append", "i4"))
    hk, hv = _cache(t, "k"), _cache(t, "v")
    sk, sv = dev(t["sk_i4"]), dev(t["sv_i4"])
    before = [c.clone() for c in (hk, hv, sk, sv)]
    print(f"[int4 hadamard append] {name}", flush=True)
    P.latent_append_i4(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv,
                       dev(t["pos"]), hadamard=True)
    torch.cuda.synchronize()
    _check_rows(cfg, t, t["x"], hk, hv, sk, sv, before, rot=True)


def test_int4_append_neighbour_tokens_share_bytes():
    """Tokens t and t xor 2 share every value byte: appending both, one call
    after the other, leaves both rows as written (each call keeps the other
    nibble)."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=32, ragged=None, seed=120)
    t = W.generate(cfg, parts=("decode", "append", "i4"))
    hk, hv = _cache(t, "k"), _cache(t, "v")
    sk, sv = dev(t["sk_i4"]), dev(t["sv_i4"])
    first = np.array([5, 16], dtype=np.int32)
    second = first ^ 2
    x2 = t["x"][::-1].copy()
    P.latent_append_i4(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv, dev(first))
    P.latent_append_i4(dev(x2), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv, dev(second))
    torch.cuda.synchronize()
    G, r = cfg.n_groups, cfg.rank
    for kind, cd, sd, a in (("k", hk, sk, t["a_k"]), ("v", hv, sv, t["a_v"])):
        codes, scales = unpack_i4_cache(cd.cpu().numpy(), kind), sd.cpu().numpy()
        for xx, pos in ((t["x"], first), (x2, second)):
            h64 = O.latent_project(xx, a).reshape(cfg.batch, G, r)
            for b, p_ in enumerate(pos):
                wc, ws = O.append_rows_i4(h64[b])
                assert np.sum(codes[b, :, p_] != wc) <= 0.01 * wc.size
                assert np.max(np.abs(codes[b, :, p_].astype(np.int64) - wc)) <= 1
                assert np.allclose(scales[b, :, p_], ws, rtol=2e-3)


def test_int4_append_workspace_reuse_and_skipped_rows():
    """The counter area returns to zero after every call; positions outside
    [0, L) are skipped."""
    import torch
    import rank_compressed_kv_amd as P
    ws = None
    for i, batch in enumerate((4, 2, 4)):
        cfg = W.CONFIGS[3].scaled(batch=batch, max_ctx=32, seed=130 + i)
        t = W.generate(cfg, parts=("decode", "append", "i4"))
        pos = t["pos"].copy()
        pos[-1] = [-1, 32, 5][i]
        x, ak, av, dpos = dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), dev(pos)
        bufs = [_cache(t, "k"), _cache(t, "v"), dev(t["sk_i4"]), dev(t["sv_i4"])]
        fresh = [b.clone() for b in bufs]
        orig = [b.clone() for b in bufs]
        desc = P.append_desc(batch=batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                             rank=cfg.rank, max_ctx=32, dtype=P.PALU_BF16)
        if ws is None:
            ws = torch.zeros(P.palu_latent_append_i4_workspace(desc), dtype=torch.uint8,
                             device="cuda")
        P.palu_latent_append_i4(desc, x, ak, av, *bufs, dpos, ws)
        P.latent_append_i4(x, ak, av, *fresh, dpos)
        torch.cuda.synchronize()
        for a, b in zip(bufs, fresh):
            assert torch.equal(a, b)
        assert int(ws[:256].count_nonzero()) == 0
        if not 0 <= pos[-1] < 32:
            for a, o in zip(bufs, orig):
                assert torch.equal(a[-1], o[-1])


@pytest.mark.parametrize("rot", [False, True])
def test_int4_append_then_decode(rot):
    """A token written by the int4 append is read back by the int4 decode: the
    result matches the oracle on the cache holding the oracle's own quantised
    rows at pos."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=320, ragged=None, seed=90)
    t = W.generate(cfg, parts=("decode", "append", "i4"))
    pos = np.array([299, 150], dtype=np.int32)
    lens = pos + 1
    bufs = [_cache(t, "k"), _cache(t, "v"), dev(t["sk_i4"]), dev(t["sv_i4"])]
    P.latent_append_i4(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), *bufs, dev(pos),
                       hadamard=rot)
    out = P.decode_attention_i4(dev(t["q"]), *bufs, dev(t["b_k"]), dev(t["b_v"]), dev(lens),
                                n_kv_heads=cfg.n_kv_heads, hadamard=rot)
    torch.cuda.synchronize()
    G, r = cfg.n_groups, cfg.rank
    app = O.append_rows_i4_hadamard if rot else O.append_rows_i4
    deq = O.dequantize_rows_i8_hadamard if rot else O.dequantize_rows_i8
    caches = {}
    for key, codes, scales, a in (("k", "k_i4", "sk_i4", "a_k"), ("v", "v_i4", "sv_i4", "a_v")):
        c, sc = t[codes].copy(), t[scales].copy()
        h64 = O.latent_project(t["x"], t[a]).reshape(cfg.batch, G, r)
        for b, p_ in enumerate(pos):
            c[b, :, p_], sc[b, :, p_] = app(h64[b])
        caches[key] = deq(c, sc)
    want = O.decode_attention(t["q"], caches["k"], caches["v"], t["b_k"], t["b_v"], lens)
    assert_close(out.cpu().numpy().astype(np.float64), want, what=f"int4 append+decode rot={rot}")
