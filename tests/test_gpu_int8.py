"""GPU parity of the int8 latent cache (per-token codes with one fp32 scale
per cached row) in absorbed mode: the HIP path through palu_decode_attn_i8
against the fp64 oracle on the dequantised cache (code * scale, exact), to
the bf16 bar (max |d| <= 2e-2, relative L2 <= 5e-3). The seeded codes are in
row order; the device cache holds them in the library's tiled order."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from rank_compressed_kv_amd.layout import pack_i8_cache, unpack_i8_cache
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


def _cache(t, kind):
    return dev(pack_i8_cache(t[f"{kind}_i8"], kind))


def _run(cfg, t, *, split_tokens=0, q=None, sk=None, sv=None, latent_out=False, lens=True):
    import torch
    import rank_compressed_kv_amd as P
    out = P.decode_attention_i8(
        dev(t["q"] if q is None else q), _cache(t, "k"), _cache(t, "v"),
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


# ------------------------------------------------------ quantised cache write ---

APPEND = {
    "r256_g2": W.CONFIGS[3].scaled(batch=4, max_ctx=64, ragged=None),       # a row is a block
    "r256_b9": W.CONFIGS[3].scaled(batch=9, max_ctx=32, ragged=None, seed=83),   # two rounds of rows
    "r128_b12": W.CONFIGS[4].scaled(batch=12, max_ctx=32, ragged=None, seed=84),
    "r256_g8": W.CONFIGS[2].scaled(batch=3, max_ctx=32, ragged=None),
    "r128": W.CONFIGS[4].scaled(max_ctx=64, ragged=None),                   # one block per row
    "r64": W.CONFIGS[3].scaled(n_groups=4, rank=64, batch=2, max_ctx=32, seed=81),  # 2 per block
    "r64_f32": W.CONFIGS[1].scaled(rank=64, batch=3, max_ctx=32, ragged=None),      # fp32 inputs
}


def _code_bounds(e, E, amax_lo, amax_hi):
    return code_bounds(e, E, amax_lo, amax_hi, 127)


@pytest.mark.parametrize("name", sorted(APPEND))
def test_int8_append(name):
    """h = x A quantised per row: the codes and scales equal the oracle's
    (quantisation of the exact row rounded to fp32) except where the exact
    value sits within the fp32 summation error of a decision boundary, and
    there they lie between the decisions at exact -/+ that error; rows other
    than pos[b] are untouched; a zero x row stores scale 0 and codes 0."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = APPEND[name]
    t = W.generate(cfg, parts=("decode", "append", "i8"))
    x = t["x"].copy()
    x[0] = 0                                         # all-zero latent row for b = 0
    hk, hv = _cache(t, "k"), _cache(t, "v")
    sk, sv = dev(t["sk"]), dev(t["sv"])
    before = [c.clone() for c in (hk, hv, sk, sv)]
    print(f"[int8 append] {name} pos={t['pos'].tolist()}", flush=True)
    P.latent_append_i8(dev(x), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv, dev(t["pos"]))
    torch.cuda.synchronize()
    G, r, dm = cfg.n_groups, cfg.rank, cfg.d_model
    mism = tot = 0
    for kind, codes_d, scales_d, a in (("k", hk, sk, t["a_k"]), ("v", hv, sv, t["a_v"])):
        codes, scales = unpack_i8_cache(codes_d.cpu().numpy(), kind), scales_d.cpu().numpy()
        h64 = O.latent_project(x, a).reshape(cfg.batch, G, r)
        # bound on |fp32 sum - exact| for any summation order
        E = (np.abs(O.to_f64(x))[:, :, None] * np.abs(O.to_f64(a))[None]).sum(1)
        E = E.reshape(cfg.batch, G, r) * dm * 2.0 ** -24
        for b, pos in enumerate(t["pos"]):
            wc, ws = O.append_rows_i8(h64[b])            # [G, r], [G]
            gc, gs = codes[b, :, pos, :].astype(np.int64), scales[b, :, pos]
            if b == 0:
                assert np.all(gc == 0) and np.all(gs == 0.0)
                continue
            mism += int(np.sum(gc != wc))
            tot += gc.size
            for g in range(G):
                e, eb = h64[b, g], E[b, g]
                amax_lo = max(float(np.max(np.abs(e) - eb)), 0.0)
                amax_hi = float(np.max(np.abs(e) + eb))
                assert amax_lo / 127 * (1 - 2.0 ** -23) <= gs[g] <= amax_hi / 127 * (1 + 2.0 ** -23)
                if np.all(gc[g] == wc[g]) and gs[g] == ws[g]:
                    continue
                lo, hi = _code_bounds(e, eb, amax_lo, amax_hi)
                assert np.all((gc[g] >= lo) & (gc[g] <= hi)), (b, g)
                assert np.max(np.abs(gc[g] - wc[g])) <= 1
    assert mism <= 0.01 * tot
    # every other row is untouched
    for i, (got, old) in enumerate(zip((hk, hv, sk, sv), before)):
        g, o = got.cpu().numpy(), old.cpu().numpy()
        if i < 2:
            g, o = unpack_i8_cache(g, "kv"[i]), unpack_i8_cache(o, "kv"[i])
        g, o = g.copy(), o.copy()
        for b, pos in enumerate(t["pos"]):
            g[b, :, int(pos)] = 0
            o[b, :, int(pos)] = 0
        assert np.array_equal(g, o)


def test_int8_append_workspace_reuse_and_skipped_rows():
    """The counter area returns to zero after every call, so one workspace
    serves call after call with results identical to a fresh one; positions
    outside [0, L) are skipped."""
    import torch
    import rank_compressed_kv_amd as P
    ws = None
    for i, batch in enumerate((4, 2, 4)):
        cfg = W.CONFIGS[3].scaled(batch=batch, max_ctx=32, seed=110 + i)
        t = W.generate(cfg, parts=("decode", "append", "i8"))
        pos = t["pos"].copy()
        pos[-1] = [-1, 32, 5][i]
        x, ak, av, dpos = dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), dev(pos)
        bufs = [_cache(t, "k"), _cache(t, "v"), dev(t["sk"]), dev(t["sv"])]
        fresh = [b.clone() for b in bufs]
        orig = [b.clone() for b in bufs]
        desc = P.append_desc(batch=batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                             rank=cfg.rank, max_ctx=32, dtype=P.PALU_BF16)
        if ws is None:
            ws = torch.zeros(P.palu_latent_append_i8_workspace(desc), dtype=torch.uint8,
                             device="cuda")
        P.palu_latent_append_i8(desc, x, ak, av, *bufs, dpos, ws)
        P.latent_append_i8(x, ak, av, *fresh, dpos)
        torch.cuda.synchronize()
        for a, b in zip(bufs, fresh):
            assert torch.equal(a, b)
        assert int(ws[:256].count_nonzero()) == 0
        if not 0 <= pos[-1] < 32:
            for a, o in zip(bufs, orig):
                assert torch.equal(a[-1], o[-1])


def test_int8_append_then_decode():
    """A token written by the quantised append is read back by the int8 decode
    like any other row: attention over the updated cache matches the oracle on
    the cache with the oracle's own quantised rows at pos (a code one step off
    near a rounding boundary moves the output far less than the tolerance)."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3].scaled(batch=2, max_ctx=320, ragged=None, seed=90)
    t = W.generate(cfg, parts=("decode", "append", "i8"))
    pos = np.array([299, 150], dtype=np.int32)
    lens = pos + 1
    bufs = [_cache(t, "k"), _cache(t, "v"), dev(t["sk"]), dev(t["sv"])]
    P.latent_append_i8(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), *bufs, dev(pos))
    out = P.decode_attention_i8(dev(t["q"]), *bufs, dev(t["b_k"]), dev(t["b_v"]), dev(lens),
                                n_kv_heads=cfg.n_kv_heads)
    torch.cuda.synchronize()
    G, r = cfg.n_groups, cfg.rank
    caches = {}
    for key, codes, scales, a in (("k", "k_i8", "sk", "a_k"), ("v", "v_i8", "sv", "a_v")):
        c, sc = t[codes].copy(), t[scales].copy()
        h64 = O.latent_project(t["x"], t[a]).reshape(cfg.batch, G, r)
        for b, p_ in enumerate(pos):
            c[b, :, p_], sc[b, :, p_] = O.append_rows_i8(h64[b])
        caches[key] = O.dequantize_rows_i8(c, sc)
    want = O.decode_attention(t["q"], caches["k"], caches["v"], t["b_k"], t["b_v"], lens)
    assert_close(out.cpu().numpy().astype(np.float64), want, what="append then decode")


# --------------------------------------------------- Hadamard-rotated rows ---

def _want_rot(t, **kw):
    hk = O.dequantize_rows_i8_hadamard(t["k_i8"], t["sk"])
    hv = O.dequantize_rows_i8_hadamard(t["v_i8"], t["sv"])
    return O.decode_attention(t["q"], hk, hv, t["b_k"], t["b_v"], t["lens"], **kw)


@pytest.mark.parametrize("idx", [3, 4, 64])
@pytest.mark.parametrize("split_tokens", [0, 64])
def test_int8_hadamard_decode_parity(idx, split_tokens):
    """A rotated cache (rows h'' = h H_r): the kernel rotates q~ and the value
    sums back; compared with the oracle on the rows (codes*scale) H_r / r."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = SMALL[idx]
    t = W.generate(cfg, parts=("decode", "i8"))
    print(f"[int8 hadamard] cfg{idx} split={split_tokens}", flush=True)
    got = P.decode_attention_i8(dev(t["q"]), _cache(t, "k"), _cache(t, "v"), dev(t["sk"]),
                                dev(t["sv"]), dev(t["b_k"]), dev(t["b_v"]), dev(t["lens"]),
                                n_kv_heads=cfg.n_kv_heads, split_tokens=split_tokens,
                                hadamard=True)
    torch.cuda.synchronize()
    assert_close(got.cpu().numpy().astype(np.float64), _want_rot(t), what=f"rot cfg{idx}")


def test_int8_hadamard_latent_output():
    """latent_out on a rotated cache returns u* in the unrotated latent space."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = SMALL[4]
    t = W.generate(cfg, parts=("decode", "i8"))
    hk = O.dequantize_rows_i8_hadamard(t["k_i8"], t["sk"])
    hv = O.dequantize_rows_i8_hadamard(t["v_i8"], t["sv"])
    want = O.decode_value_latents(t["q"], hk, hv, t["b_k"], t["lens"], cfg.group_dim)
    got = P.decode_attention_i8(dev(t["q"]), _cache(t, "k"), _cache(t, "v"), dev(t["sk"]),
                                dev(t["sv"]), dev(t["b_k"]), None, dev(t["lens"]),
                                n_kv_heads=cfg.n_kv_heads, latent_out=True, hadamard=True)
    torch.cuda.synchronize()
    assert_close(got.cpu().numpy().astype(np.float64), want, what="rot u*")


@pytest.mark.parametrize("name", ["r256_g2", "r128", "r64", "r64_f32"])
def test_int8_hadamard_append(name):
    """Rotated quantised cache write: codes and scales of h H_r agree with the
    oracle's except within the fp32 error bound of a decision boundary (the
    sum's bound carried through the rotation, plus the rotation's own
    rounding), and never by more than one step."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = APPEND[name]
    t = W.generate(cfg, parts=("decode", "append", "i8"))
    hk, hv = _cache(t, "k"), _cache(t, "v")
    sk, sv = dev(t["sk"]), dev(t["sv"])
    print(f"[int8 hadamard append] {name}", flush=True)
    P.latent_append_i8(dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), hk, hv, sk, sv, dev(t["pos"]),
                       hadamard=True)
    torch.cuda.synchronize()
    G, r, dm = cfg.n_groups, cfg.rank, cfg.d_model
    H = O.hadamard(r)
    mism = tot = 0
    for kind, codes_d, scales_d, a in (("k", hk, sk, t["a_k"]), ("v", hv, sv, t["a_v"])):
        codes, scales = unpack_i8_cache(codes_d.cpu().numpy(), kind), scales_d.cpu().numpy()
        h64 = O.latent_project(t["x"], a).reshape(cfg.batch, G, r)
        E = (np.abs(O.to_f64(t["x"]))[:, :, None] * np.abs(O.to_f64(a))[None]).sum(1)
        E = E.reshape(cfg.batch, G, r) * dm * 2.0 ** -24
        for b, pos in enumerate(t["pos"]):
            wc, ws = O.append_rows_i8_hadamard(h64[b])
            gc, gs = codes[b, :, pos, :].astype(np.int64), scales[b, :, pos]
            mism += int(np.sum(gc != wc))
            tot += gc.size
            for g in range(G):
                e = h64[b, g] @ H
                eb = 1.5 * (E[b, g].sum() + np.log2(r) * 2.0 ** -24 *
                            np.sum(np.abs(h64[b, g]) + E[b, g]))
                amax_lo = max(float(np.max(np.abs(e)) - eb), 0.0)
                amax_hi = float(np.max(np.abs(e)) + eb)
                assert amax_lo / 127 * (1 - 2.0 ** -23) <= gs[g] <= amax_hi / 127 * (1 + 2.0 ** -23)
                if np.all(gc[g] == wc[g]):
                    continue
                lo, hi = _code_bounds(e, eb, amax_lo, amax_hi)
                assert np.all((gc[g] >= lo) & (gc[g] <= hi)), (b, g)
                assert np.max(np.abs(gc[g] - wc[g])) <= 1
    assert mism <= 0.01 * tot


def test_int8_hadamard_helps_on_outlier_channels():
    """Latents with outlier channels (20x on 1% of the channels, as in the
    131K workload), quantised per token with and without the rotation: the
    int8 decode on the rotated cache lands closer to attention over the
    unquantised latents."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[4].scaled(batch=2, max_ctx=1024, ragged=None, seed=91)
    t = W.generate(cfg)
    h = {kind: O.to_f64(t[f"h_{kind}"]) for kind in "kv"}
    exact = O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"])
    errs = {}
    for rot in (False, True):
        cache, scales = {}, {}
        for kind in "kv":
            c, s = (O.append_rows_i8_hadamard if rot else O.append_rows_i8)(h[kind])
            cache[kind] = dev(pack_i8_cache(c, kind))
            scales[kind] = dev(s)
        got = P.decode_attention_i8(dev(t["q"]), cache["k"], cache["v"], scales["k"],
                                    scales["v"], dev(t["b_k"]), dev(t["b_v"]), dev(t["lens"]),
                                    n_kv_heads=cfg.n_kv_heads, hadamard=rot)
        torch.cuda.synchronize()
        d = got.cpu().numpy().astype(np.float64) - exact
        errs[rot] = np.linalg.norm(d) / np.linalg.norm(exact)
    print(f"[int8 outliers] rel L2 error plain {errs[False]:.3e} rotated {errs[True]:.3e}",
          flush=True)
    assert errs[True] < 0.7 * errs[False]
