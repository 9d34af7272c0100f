"""palu_latent_append_prepare: the cache write and the decode call's query-side
operands in one call. Against the two calls made apart (palu_latent_append,
_i8 or _i4, then a decode call that forms its own operands) the caches and the
decode output are bit-identical, whether the absorption rides in the append's
launch (absorbed keys, dtype cache or int8 / int4 codes, bf16 or fp32) or the
call falls back to two launches (rebuilt keys, the uncompressed baseline); one
case is also held to the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import palu_oracle as O
from rank_compressed_kv_amd.layout import pack_i4_cache, pack_i8_cache
from tests.parity_util import assert_close, dev

pytestmark = pytest.mark.gpu

# one group of eight KV heads at rank 32, a short cache: many small sequences
CARRY = W.CONFIGS[3].scaled(n_q_heads=8, n_kv_heads=8, n_groups=1, rank=32, max_ctx=64,
                            ragged=None)

CASES = {
    # the absorption carried by the append's launch
    "bf16_absorbed": (W.CONFIGS[3].scaled(batch=3, max_ctx=512, ragged=None, seed=90), 0,
                      "absorbed"),
    "bf16_absorbed_b9": (W.CONFIGS[3].scaled(batch=9, max_ctx=256, ragged=None, seed=91), 0,
                         "absorbed"),
    "bf16_absorbed_mha": (W.CONFIGS[2].scaled(batch=2, max_ctx=256, ragged=None, seed=92), 0,
                          "absorbed"),
    "f32_absorbed": (W.CONFIGS[1].scaled(batch=2, max_ctx=256, ragged=None, seed=93), 0,
                     "absorbed"),
    "int8_absorbed": (W.CONFIGS[3].scaled(batch=3, max_ctx=512, ragged=None, seed=94), 8,
                      "absorbed"),
    "int4_absorbed": (W.CONFIGS[3].scaled(batch=5, max_ctx=512, ragged=None, seed=95), 4,
                      "absorbed"),
    "int4_absorbed_r128": (W.CONFIGS[4].scaled(batch=2, max_ctx=512, ragged=None, seed=96), 4,
                           "absorbed"),
    # two launches: B_k transposed for the rebuilt keys, scaled q for the baseline
    "bf16_reconstruct": (W.CONFIGS[3].scaled(batch=3, max_ctx=512, ragged=None, seed=97), 0,
                         "reconstruct"),
    "bf16_full_rank": (W.CONFIGS[3].scaled(batch=2, max_ctx=256, ragged=None, seed=98,
                                           n_groups=8, rank=128), 0, "full_rank"),
    # the projection stored transposed [G*r, d_model]: the one-pass cache
    # write, carrying the absorption or followed by the prepare launch
    "bf16_absorbed_cols": (W.CONFIGS[3].scaled(batch=9, max_ctx=256, ragged=None, seed=99), 0,
                           "absorbed", 1),
    "f32_absorbed_cols": (W.CONFIGS[1].scaled(batch=2, max_ctx=256, ragged=None, seed=100), 0,
                          "absorbed", 1),
    "bf16_reconstruct_cols": (W.CONFIGS[3].scaled(batch=3, max_ctx=512, ragged=None, seed=101),
                              0, "reconstruct", 1),
    # the carried absorption's launch bound: with a_k, a_v [d_model, G*r] the
    # absorb workgroups are further grid rows (d_model / 128 + Hkv * B rows at
    # r = 32); 4096 sequences stay within the 65535 rows of a launch, 8192
    # cross it and make two launches; the transposed form's one-dimensional
    # grid carries both
    "carry_bound_below": (CARRY.scaled(batch=4096, seed=102), 0, "absorbed"),
    "carry_bound_above": (CARRY.scaled(batch=8192, seed=103), 0, "absorbed"),
    "carry_bound_above_cols": (CARRY.scaled(batch=8192, seed=104), 0, "absorbed", 1),
}


def _setup(cfg, qbits, mode, a_layout=0):
    import torch
    import rank_compressed_kv_amd as P
    parts = ("decode", "append") + (("i8",) if qbits == 8 else ("i4",) if qbits == 4 else ())
    t = W.generate(cfg, parts=parts)
    dt = P.PALU_BF16 if cfg.dtype == "bf16" else P.PALU_F32
    theta = cfg.rope_theta if mode == "reconstruct" else 0.0
    desc = P.attn_desc(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_groups=cfg.n_groups, rank=cfg.rank,
                       max_ctx=cfg.max_ctx, dtype=dt, mode=mode, rope_theta=theta)
    adesc = P.append_desc(batch=cfg.batch, d_model=cfg.d_model, n_groups=cfg.n_groups,
                          rank=cfg.rank, max_ctx=cfg.max_ctx, dtype=dt, a_layout=a_layout)
    # the appended token is the last of each sequence's context
    pos = np.minimum(t["pos"], cfg.max_ctx - 1).astype(np.int32)
    lens = (pos + 1).astype(np.int32)
    if qbits == 8:
        cache = [dev(pack_i8_cache(t["k_i8"], "k")), dev(pack_i8_cache(t["v_i8"], "v")),
                 dev(t["sk"]), dev(t["sv"])]
    elif qbits == 4:
        cache = [dev(pack_i4_cache(t["k_i4"], "k")), dev(pack_i4_cache(t["v_i4"], "v")),
                 dev(t["sk_i4"]), dev(t["sv_i4"])]
    else:
        cache = [dev(t["h_k"]), dev(t["h_v"]), None, None]
    ak, av = t["a_k"], t["a_v"]
    if a_layout:
        ak, av = np.ascontiguousarray(ak.T), np.ascontiguousarray(av.T)
    ops = dict(x=dev(t["x"]), a_k=dev(ak), a_v=dev(av), pos=dev(pos),
               q=dev(t["q"]), b_k=dev(t["b_k"]), b_v=dev(t["b_v"]), lens=dev(lens))
    wsz = P.palu_decode_attn_workspace(desc)
    asz = P.palu_latent_append_workspace(adesc)
    fresh = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")
    return t, desc, adesc, cache, ops, wsz, asz, fresh, pos, lens, theta


def _decode(P, qbits, desc, ops, cache, out, ws):
    hk, hv, sk, sv = cache
    if qbits == 0:
        P.palu_decode_attn(desc, ops["q"], hk, hv, ops["b_k"], ops["b_v"], ops["lens"], out, ws)
    else:
        fn = P.palu_decode_attn_i8 if qbits == 8 else P.palu_decode_attn_i4
        fn(desc, ops["q"], hk, hv, sk, sv, ops["b_k"], ops["b_v"], ops["lens"], out, ws)


@pytest.mark.parametrize("name", sorted(CASES))
def test_step_matches_separate_calls(name):
    import torch
    import rank_compressed_kv_amd as P
    cfg, qbits, mode = CASES[name][:3]
    a_layout = CASES[name][3] if len(CASES[name]) > 3 else 0
    t, desc, adesc, cache0, ops, wsz, asz, fresh, pos, lens, theta = _setup(cfg, qbits, mode,
                                                                             a_layout)
    print(f"[step] {name} qbits={qbits} mode={mode} a_layout={a_layout} B={cfg.batch} "
          f"pos={pos.tolist()}", flush=True)
    bk = None if mode == "full_rank" else ops["b_k"]
    shape = (cfg.batch, cfg.n_q_heads, cfg.head_dim)

    # apart: the append call, then a decode call forming its own operands
    ca = [None if c is None else c.clone() for c in cache0]
    out_a = torch.empty(shape, dtype=torch.float32, device="cuda")
    if qbits == 0:
        P.palu_latent_append(adesc, ops["x"], ops["a_k"], ops["a_v"], ca[0], ca[1], ops["pos"],
                             fresh(asz))
    else:
        fn = P.palu_latent_append_i8 if qbits == 8 else P.palu_latent_append_i4
        fn(adesc, ops["x"], ops["a_k"], ops["a_v"], *ca, ops["pos"], fresh(asz))
    _decode(P, qbits, desc, ops, ca, out_a, fresh(wsz))

    # together, twice on the same workspaces (the append's counters return to
    # zero; the second step rewrites the same rows)
    cb = [None if c is None else c.clone() for c in cache0]
    pdesc = P.AttnDesc.from_buffer_copy(desc)
    pdesc.prepared = 1
    aws, ws = fresh(asz), fresh(wsz)
    for rep in range(2):
        out_b = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        P.palu_latent_append_prepare(adesc, qbits, ops["x"], ops["a_k"], ops["a_v"], cb[0], cb[1],
                                     cb[2], cb[3], ops["pos"], aws, desc, ops["q"], bk, ws)
        _decode(P, qbits, pdesc, ops, cb, out_b, ws)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(ca, cb)):
            if x is not None:
                assert torch.equal(x, y), f"{name}: cache tensor {i} differs (step {rep})"
        assert torch.equal(out_a, out_b), f"{name}: output differs (step {rep})"


def test_step_against_oracle():
    """The bf16 absorbed step (one launch before the decode call) against the
    oracle on inputs the oracle forms itself: its own cache write of the
    token (x A, rounded to fp32 then to bf16) into row pos[b] of the seeded
    caches, then decode attention over those caches. The GPU-written rows are
    also held to the oracle's within bf16 rounding of the fp32 sum."""
    import torch
    import rank_compressed_kv_amd as P
    cfg, qbits, mode = CASES["bf16_absorbed"]
    t, desc, adesc, cache, ops, wsz, asz, fresh, pos, lens, theta = _setup(cfg, qbits, mode)
    pdesc = P.AttnDesc.from_buffer_copy(desc)
    pdesc.prepared = 1
    ws = fresh(wsz)
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device="cuda")
    P.palu_latent_append_prepare(adesc, 0, ops["x"], ops["a_k"], ops["a_v"], cache[0], cache[1],
                                 None, None, ops["pos"], fresh(asz), desc, ops["q"], ops["b_k"],
                                 ws)
    _decode(P, 0, pdesc, ops, cache, out, ws)
    torch.cuda.synchronize()
    bits = lambda c: c.cpu().view(torch.int16).numpy().view(np.uint16)
    as_f = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    oracle_caches = []
    for h, seeded, a in ((bits(cache[0]), t["h_k"], t["a_k"]), (bits(cache[1]), t["h_v"], t["a_v"])):
        h64 = O.latent_project(t["x"], a).reshape(cfg.batch, cfg.n_groups, cfg.rank)
        got = np.stack([as_f(h[b, :, int(p)]) for b, p in enumerate(pos)])
        np.testing.assert_allclose(got, h64, rtol=2.0 ** -7, atol=1e-6)
        c = seeded.copy()
        for b, p in enumerate(pos):
            c[b, :, int(p)] = O.append_rows_bf16(h64[b])
        oracle_caches.append(c)
    want = O.decode_attention(t["q"], oracle_caches[0], oracle_caches[1], t["b_k"], t["b_v"],
                              lens, rope_theta=0.0)
    assert_close(out.cpu().numpy().astype(np.float64), want, what="step vs oracle")
