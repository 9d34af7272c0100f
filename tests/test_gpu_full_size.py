"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the library's own plan), on sampled outputs: the oracle
computes a few (sequence, query head) rows one by one (the first and the last,
a head of the longest sequence, and seeded picks) and those rows are held to
the same bar as the reduced-size tests (max |d| <= 2e-2, relative L2 <= 5e-3;
fp32: 1e-4 / 1e-5). The quantised caches are checked the same way at the
Llama-3-8B shape, against the oracle on the dequantised rows of the sampled
sequences."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache
from tests.parity_util import assert_close, dev, run_decode

pytestmark = pytest.mark.gpu

CASES = [(i, m) for i in sorted(W.CONFIGS) for m in W.CONFIGS[i].modes]


def _pairs(cfg, lens, k=6):
    rng = np.random.default_rng(7000 + cfg.seed)
    B, Hq = cfg.batch, cfg.n_q_heads
    pairs = {(0, 0), (B - 1, Hq - 1), (int(np.argmax(lens)), Hq // 2)}
    while len(pairs) < min(k, B * Hq):
        pairs.add((int(rng.integers(B)), int(rng.integers(Hq))))
    return sorted(pairs)


def _tol(cfg):
    return dict(max_abs=1e-4, rel_l2=1e-5) if cfg.dtype == "f32" else {}


@pytest.mark.parametrize("idx,mode", CASES)
def test_full_size_sampled(idx, mode):
    cfg = W.CONFIGS[idx]
    t = W.generate(cfg)
    pairs = _pairs(cfg, t["lens"])
    print(f"[full] cfg{idx} {cfg.name} {mode} pairs={pairs}", flush=True)
    got, theta = run_decode(cfg, t, mode)
    want = O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                              rope_theta=theta, select=pairs)
    sel = tuple(np.array(pairs).T)
    assert_close(got[sel], want[sel], what=f"full cfg{idx}/{mode}", **_tol(cfg))


@pytest.mark.parametrize("mode", ["reconstruct", "absorbed"])
@pytest.mark.parametrize("s,r", [(1, 32), (2, 64), (4, 128), (8, 256)])
def test_full_size_head_groupings_sampled(s, r, mode):
    """The head-grouping sweep the benchmark times (the Llama-3-8B shape at
    75% key compression, 32K context; rebuilt and rotated keys, or absorbed
    keys: 32 query heads a group at s = 8), one KV head a group (M-LRD) to
    all eight (J-LRD), in the library's own plan."""
    cfg = W.CONFIGS[3].scaled(n_groups=8 // s, rank=r)
    t = W.generate(cfg)
    pairs = _pairs(cfg, t["lens"])
    print(f"[full] grouping s={s} r={r} {mode} pairs={pairs}", flush=True)
    got, theta = run_decode(cfg, t, mode)
    assert (theta > 0) == (mode == "reconstruct")
    want = O.decode_attention(t["q"], t["h_k"], t["h_v"], t["b_k"], t["b_v"], t["lens"],
                              rope_theta=theta, select=pairs)
    sel = tuple(np.array(pairs).T)
    assert_close(got[sel], want[sel], what=f"full grouping s={s} r={r} {mode}")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("rot", [False, True])
def test_full_size_quantised_sampled(bits, rot):
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3]
    t = W.generate(cfg, parts=("decode", f"i{bits}"))
    sfx = "" if bits == 8 else "_i4"
    codes_k, codes_v = t[f"k_i{bits}"], t[f"v_i{bits}"]
    sk, sv = t["sk" + sfx], t["sv" + sfx]
    pack = pack_i8_cache if bits == 8 else pack_i4_cache
    fn = P.decode_attention_i8 if bits == 8 else P.decode_attention_i4
    pairs = _pairs(cfg, t["lens"])
    print(f"[full] int{bits} rot={rot} pairs={pairs}", flush=True)
    out = fn(dev(t["q"]), dev(pack(codes_k, "k")), dev(pack(codes_v, "v")), dev(sk), dev(sv),
             dev(t["b_k"]), dev(t["b_v"]), dev(t["lens"]), n_kv_heads=cfg.n_kv_heads,
             hadamard=rot)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    deq = O.dequantize_rows_i8_hadamard if rot else O.dequantize_rows_i8
    g_s, w_s = [], []
    for b, h in pairs:
        sl = slice(b, b + 1)
        w = O.decode_attention(t["q"][sl], deq(codes_k[sl], sk[sl]), deq(codes_v[sl], sv[sl]),
                               t["b_k"], t["b_v"], t["lens"][sl], select=[(0, h)])[0, h]
        g_s.append(got[b, h])
        w_s.append(w)
    assert_close(np.array(g_s), np.array(w_s), what=f"full int{bits} rot={rot}")


def test_full_size_step_sampled():
    """The step the benchmark times, at config 3's full size: one
    palu_latent_append_prepare call (the token's latents into row len-1 of
    both caches, the query absorption in the same launch), then the decode
    call with prepared = 1, in the library's own plan; sampled outputs
    against the oracle on the cache after its own append of that token."""
    import torch
    import rank_compressed_kv_amd as P
    cfg = W.CONFIGS[3]
    t = W.generate(cfg, parts=("decode", "append"))
    pairs = _pairs(cfg, t["lens"])
    print(f"[full] step cfg3 pairs={pairs}", flush=True)
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=P.PALU_BF16, mode="absorbed")
    adesc = P.append_desc(batch=cfg.batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                          rank=cfg.rank, max_ctx=cfg.max_ctx, dtype=P.PALU_BF16)
    pdesc = P.AttnDesc.from_buffer_copy(desc)
    pdesc.prepared = 1
    pos = (t["lens"] - 1).astype(np.int32)
    hk, hv = dev(t["h_k"]), dev(t["h_v"])
    ws = torch.empty(P.palu_decode_attn_workspace(desc), dtype=torch.uint8, device="cuda")
    aws = torch.zeros(P.palu_latent_append_workspace(adesc), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    q, bk, bv, lens = dev(t["q"]), dev(t["b_k"]), dev(t["b_v"]), dev(t["lens"])
    P.palu_latent_append_prepare(adesc, 0, dev(t["x"]), dev(t["a_k"]), dev(t["a_v"]), hk, hv,
                                 None, None, dev(pos), aws, desc, q, bk, ws)
    P.palu_decode_attn(pdesc, q, hk, hv, bk, bv, lens, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    # the oracle's own append of the token, then decode attention
    caches = []
    for cache, a in ((t["h_k"], t["a_k"]), (t["h_v"], t["a_v"])):
        h64 = O.latent_project(t["x"], a).reshape(cfg.batch, cfg.n_groups, cfg.rank)
        c = cache.copy()
        for b, p in enumerate(pos):
            c[b, :, int(p)] = O.append_rows_bf16(h64[b])
        caches.append(c)
    want = O.decode_attention(t["q"], caches[0], caches[1], t["b_k"], t["b_v"], t["lens"],
                              rope_theta=0.0, select=pairs)
    sel = tuple(np.array(pairs).T)
    assert_close(got[sel], want[sel], what="full cfg3 step")
